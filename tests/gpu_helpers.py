"""Helpers shared by the GPU parity tests: device upload, tolerance checks,
and flushed progress lines naming each case before it runs on the GPU."""
from __future__ import annotations

import math
import sys

import numpy as np

# Tolerances (fixed by the stated contract of each operation):
SUM_TOL = 1e-6          # |gpu - S| <= SUM_TOL * A, A = sum of |terms|
COLPROD_F32_TOL = 4e-4  # relative, R <= 4096 (any order is within (R-1)*2^-24)
COLPROD_16_TOL = 2e-2   # relative, f16 / bf16 with one final rounding


def say(msg: str) -> None:
    """Print and flush a line naming the case about to run on the GPU."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f32bits(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


def zero_sum_sign_ok(got, s) -> np.ndarray:
    """IEEE-754 addition (round to nearest) gives -0 only for two negative
    zeros, so a sum that comes out exactly zero is -0 when every term is -0
    and +0 otherwise, whatever the order.  The oracle's sum S follows the
    same rule (it is -0 exactly when every term is -0).  True where `got`
    is not zero or carries that sign."""
    g = np.asarray(got, np.float64)
    w = np.asarray(s, np.float64)
    want_neg = (w == 0) & np.signbit(w)
    return (g != 0) | np.isnan(g) | (np.signbit(g) == want_neg)


def check_sum(got: float, s: float, a: float, what: str, tol: float = SUM_TOL):
    if math.isnan(s) or math.isinf(s):
        if math.isnan(s):
            assert math.isnan(got), (what, got, s)
        else:
            assert got == s, (what, got, s)
        return
    err = abs(float(got) - s)
    assert err <= tol * a, "%s: |%r - %r| = %g > %g * %g" % (what, float(got), s, err, tol, a)
    assert zero_sum_sign_ok(got, s), "%s: zero sum %r, oracle %r" % (what, float(got), s)


def check_sums(got, s, a, what: str, tol: float = SUM_TOL):
    """check_sum over arrays of per-row / per-column results (non-finite
    oracle sums compare by class: NaN to NaN, inf to the same inf)."""
    got = np.asarray(got)
    g = got.astype(np.float64)
    finite = np.isfinite(s)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - s)
    bad = finite & ~(err <= tol * a)
    assert not bad.any(), "%s: index %d got %r want %r (A %r)" % (
        what, int(np.nonzero(bad)[0][0]), g[bad][0], s[bad][0], a[bad][0])
    nan = np.isnan(s)
    assert np.isnan(g[nan]).all(), what
    inf = np.isinf(s)
    assert (g[inf] == s[inf]).all(), what
    sign = zero_sum_sign_ok(g, s)
    assert sign.all(), "%s: index %d: zero sum with the wrong sign (got %r, oracle %r)" % (
        what, int(np.nonzero(~sign)[0][0]), g[~sign][0], s[~sign][0])


def has_both_zeros(values, old=None, accum=False, axis=None) -> np.ndarray:
    """True where the reduced values (plus the old destination under accum)
    hold a +0 and a -0: there either zero is a correct max / min.  `axis`
    is the axis reduced (None: the whole array)."""
    v = np.asarray(values, np.float32)
    bits = v.view(np.uint32)
    pos = (bits == 0x00000000).any(axis=axis)
    neg = (bits == 0x80000000).any(axis=axis)
    if accum and old is not None:
        ob = np.asarray(old, np.float32).view(np.uint32)
        pos = pos | (ob == 0x00000000)
        neg = neg | (ob == 0x80000000)
    return np.asarray(pos & neg)


def valid_region(a, rows, cols, ld) -> np.ndarray:
    """The rows x cols valid region of a row-major buffer of row stride ld
    (given flat or 2-D)."""
    flat = np.asarray(a).reshape(-1)
    if rows == 0 or cols == 0:
        return flat[:0].reshape(rows, cols)
    need = rows * ld
    if flat.size < need:
        flat = np.concatenate([flat, np.zeros(need - flat.size, flat.dtype)])
    return flat[:need].reshape(rows, ld)[:, :cols]


def extremes_match(got, want, both_zeros) -> np.ndarray:
    """Element-wise max / min parity: the same bits, or NaN for NaN, or any
    zero for a zero where `both_zeros` (see has_both_zeros)."""
    g = np.asarray(got, np.float32)
    w = np.asarray(want, np.float32)
    same = g.view(np.uint32) == w.view(np.uint32)
    nan = np.isnan(g) & np.isnan(w)
    either = np.asarray(both_zeros) & (g == 0) & (w == 0)
    return same | nan | either


def check_exact(got, want, what: str, both_zeros: bool = False):
    """Bit-exact float equality (max / min).  A zero of the other sign is
    accepted only when `both_zeros`: the reduced values hold zeros of both
    signs, so either zero is a correct extreme."""
    g, w = np.float32(got), np.float32(want)
    if math.isnan(w):
        assert math.isnan(g), (what, g, w)
        return
    if both_zeros and w == 0 and g == 0:
        return
    assert f32bits(g) == f32bits(w), (what, float(g), float(w))


def check_extremes(got, want, both_zeros, what: str):
    eq = extremes_match(got, want, both_zeros)
    assert eq.all(), "%s: index %d got %r want %r" % (
        what, int(np.nonzero(~eq)[0][0]), np.asarray(got)[~eq][0], np.asarray(want)[~eq][0])


def check_rel(got: np.ndarray, want: np.ndarray, tol: float, what: str):
    """Relative error of products.  A zero product must be a zero of the
    oracle's sign: the sign of an exactly zero product is the XOR of the
    factors' signs, whatever the order (PTO ISA TCOLPROD, Math
    Interpretation: the product over the column)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    zero = want == 0
    assert (got[zero] == 0).all(), "%s: nonzero result for a zero product" % what
    sign = np.signbit(got[zero]) == np.signbit(want[zero])
    assert sign.all(), "%s: zero product %d with the wrong sign" % (
        what, int(np.nonzero(zero)[0][np.nonzero(~sign)[0][0]]))
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, "%s: max relative error %g > %g" % (what, worst, tol)
    return worst


def signed_zero_patterns(rows, n, seed):
    """A (rows, n) fp32 array whose rows cycle through six patterns: all -0; all +0; zeros of random
    signs; -0 with one +0; negative numbers with one -0 (max is -0); positive
    numbers with one +0 (min is +0)."""
    rng = np.random.default_rng(seed)
    x = np.empty((rows, n), np.float32)
    for r in range(rows):
        k = r % 6
        if k == 0:
            x[r] = -0.0
        elif k == 1:
            x[r] = 0.0
        elif k == 2:
            x[r] = np.where(rng.random(n) < 0.5, 0.0, -0.0)
        elif k == 3:
            x[r] = -0.0
            x[r, rng.integers(0, n)] = 0.0
        elif k == 4:
            x[r] = -rng.uniform(0.5, 2.0, n)
            x[r, rng.integers(0, n)] = -0.0
        else:
            x[r] = rng.uniform(0.5, 2.0, n)
            x[r, rng.integers(0, n)] = 0.0
    return x
