"""Seeded synthetic inputs for dense-array reduction.

This module only draws and lays out input arrays.  It holds none of the
reduction arithmetic, imports neither the oracle nor the HIP library, and is
the one piece of code both sides use: the tests hand the same arrays to the
oracle and to the GPU.

Every array comes from numpy's ``default_rng(seed)`` (PCG64).  Draws are
float64 and rounded to float32; 16-bit tiles are then rounded from float32
to binary16 (numpy) or bfloat16 (round to nearest even on the bit pattern).
Large arrays are drawn in fixed-size chunks from one generator, which yields
the same values as one monolithic draw (checked in tests/test_workloads.py)
while bounding host memory.

The five workloads (sizes, distributions, seeds):

1. ``rows32``: 4096 rows x 32 fp32, uniform[-1, 1), seed 0; then, from the
   same generator, one 16 x 16 fp32 tile, uniform[0.5, 1.5).
2. ``vec16m``: one fp32 vector of 2^24 elements, uniform[-1, 1), seed 1;
   accum runs preset the destination to 3.25.
3. ``colprod4k``: 4096 x 16384 fp32 tile, uniform[0.999, 1.001), seed 2; then
   an int32 tile of the same shape with values drawn uniformly from
   {-3, -2, -1, 1, 2, 3}.
4. ``vec1g``: one fp32 vector of 2^30 + 7 elements, standard normal, seed 3;
   then an independent Bernoulli(0.01) mask from the same generator whose
   entries are multiplied by 1e6 (in float32).
5. ``rows1000``: 65536 rows x 1000 fp32, uniform[-1, 1), seed 4; then a
   2048 x 32768 bfloat16 tile and a 2048 x 32768 binary16 tile, both
   uniform[0.99, 1.01), drawn in that order from the same generator.
"""
from __future__ import annotations

import numpy as np

CHUNK = 1 << 24  # elements per draw for large arrays

N_VEC16M = 1 << 24
N_VEC1G = (1 << 30) + 7
ACCUM_PRESET = 3.25


def _uniform_f32(rng, lo, hi, n, out=None):
    """n float32 values rounded from float64 uniform[lo, hi) draws."""
    if out is None:
        out = np.empty(n, np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = rng.uniform(lo, hi, e - s)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Used only to quantise synthetic inputs (no NaN occurs in them)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_u.size, CHUNK):
        e = min(flat_u.size, s + CHUNK)
        v = flat_u[s:e].astype(np.uint64)
        flat_o[s:e] = ((v + 0x7FFF + ((v >> 16) & 1)) >> 16).astype(np.uint16)
    return out


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round to nearest even."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def rows32():
    """(A[4096, 32] f32, T[16, 16] f32)."""
    rng = np.random.default_rng(0)
    a = _uniform_f32(rng, -1.0, 1.0, 4096 * 32).reshape(4096, 32)
    t = _uniform_f32(rng, 0.5, 1.5, 16 * 16).reshape(16, 16)
    return a, t


def vec16m():
    """x[2^24] f32."""
    rng = np.random.default_rng(1)
    return _uniform_f32(rng, -1.0, 1.0, N_VEC16M)


def colprod4k_f32_i32():
    """(F[4096, 16384] f32, I[4096, 16384] i32)."""
    rng = np.random.default_rng(2)
    R, C = 4096, 16384
    f = _uniform_f32(rng, 0.999, 1.001, R * C).reshape(R, C)
    choices = np.array([-3, -2, -1, 1, 2, 3], np.int32)
    i = np.empty(R * C, np.int32)
    for s in range(0, R * C, CHUNK):
        e = min(R * C, s + CHUNK)
        i[s:e] = choices[rng.integers(0, 6, e - s)]
    return f, i.reshape(R, C)


def vec1g(n: int = N_VEC1G):
    """x[n] f32: standard normal, 1 % of entries (i.i.d.) scaled by 1e6.
    ``n`` defaults to 2^30 + 7; smaller n gives a prefix-consistent recipe
    for tests of the generator itself."""
    rng = np.random.default_rng(3)
    x = np.empty(n, np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        x[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    big = np.float32(1e6)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        m = rng.random(e - s) < 0.01
        seg = x[s:e]
        seg[m] *= big
    return x


def rows1000_x():
    """X[65536, 1000] f32 alone (the first draw of rows1000's generator)."""
    rng = np.random.default_rng(4)
    return _uniform_f32(rng, -1.0, 1.0, 65536 * 1000).reshape(65536, 1000)


def rows1000():
    """(X[65536, 1000] f32, B[2048, 32768] bf16 bits, H[2048, 32768] f16 bits)."""
    rng = np.random.default_rng(4)
    x = _uniform_f32(rng, -1.0, 1.0, 65536 * 1000).reshape(65536, 1000)
    R, C = 2048, 32768
    b = to_bf16_bits(_uniform_f32(rng, 0.99, 1.01, R * C)).reshape(R, C)
    h = to_f16_bits(_uniform_f32(rng, 0.99, 1.01, R * C)).reshape(R, C)
    return x, b, h


def odd_i32_tile(R: int = 4096, C: int = 16384, seed: int = 102):
    """Supplementary int32 tile with odd values {-3, -1, 1, 3}: unlike the
    {-3..3} tile its column products are almost never 0 mod 2^32."""
    rng = np.random.default_rng(seed)
    choices = np.array([-3, -1, 1, 3], np.int32)
    return choices[rng.integers(0, 4, R * C)].reshape(R, C)


# ---------------------------------------------------------------------------
# generic seeded helpers for edge-case tests
# ---------------------------------------------------------------------------

def uniform_f32(seed: int, shape, lo: float = -1.0, hi: float = 1.0):
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape)) if np.ndim(shape) else int(shape)
    return _uniform_f32(rng, lo, hi, n).reshape(shape)


def integers_i32(seed: int, shape, lo: int, hi: int):
    """int32 values uniform in [lo, hi)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, shape, dtype=np.int64).astype(np.int32)
