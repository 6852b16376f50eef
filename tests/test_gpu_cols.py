"""GPU parity of the column sum / max / min (the reduction taken along the
rows of a 2-D fp32 tile) against the CPU oracle: a 4096 x 16384 tile,
padded, misaligned and ragged shapes, special values, empty tiles and
run-to-run determinism.  max / min bit-exact; sum within 1e-6 * A per
column."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (check_extremes, check_sums, dev, has_both_zeros, host, say,
                         signed_zero_patterns, valid_region)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run_cols(red, op, sd, C, accum=False, old=None):
    out = (torch.zeros(max(C, 1), dtype=torch.float32, device="cuda") if old is None
           else dev(np.asarray(old, np.float32)))
    getattr(red, op + "_cols_f32")(sd, out, C=C, accum=accum)
    return host(out)[:C]


def check_cols(orc, op, src, R, C, ld, got, accum=False, old=None, what=""):
    if op == "sum":
        s, a = orc.cols_sum_f32(src, R, C, ld, accum, old)
        check_sums(got, s, a, what)
        with np.errstate(invalid="ignore"):  # inf - inf in non-finite columns
            err = np.abs(got.astype(np.float64) - s)
        finite = np.isfinite(s)
        return float(np.max(err[finite] / np.maximum(a[finite], 1e-300), initial=0.0))
    else:
        fn = orc.cols_max_f32 if op == "max" else orc.cols_min_f32
        want = fn(src, R, C, ld, accum, old)
        both = has_both_zeros(valid_region(src, R, C, ld), old, accum, axis=0)
        check_extremes(got, want, both, what)


@pytest.fixture(scope="module")
def tile4k():
    say("generate 4096 x 16384 uniform[-1,1) tile (seed 60)")
    t = workloads.uniform_f32(60, (4096, 16384))
    return t, dev(t)


@pytest.mark.parametrize("accum", [False, True])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_cols_4k(red, orc, tile4k, op, accum):
    t, td = tile4k
    say("cols 4096x16384 %s accum=%s" % (op, accum))
    old = workloads.uniform_f32(61, 16384, -3.0, 3.0) if accum else None
    got = run_cols(red, op, td, 16384, accum, old)
    worst = check_cols(orc, op, t, 4096, 16384, 16384, got, accum, old, "cols4k %s" % op)
    if op == "sum":
        say("cols 4096x16384 sum: worst |gpu - exact| / sum|x| = %.3g (tolerance 1e-6)" % worst)


SHAPES = [  # (R, C, ld, element offset of the base pointer)
    (1, 1, 1, 0), (1, 37, 37, 0), (16, 16, 16, 0), (37, 1, 1, 0), (5, 3, 4, 1),
    (100, 259, 260, 0), (257, 515, 515, 0), (33, 1024, 1024, 3),
    (1000, 130, 136, 2), (8191, 72, 72, 0), (3000, 2049, 2049, 1),
]


@pytest.mark.parametrize("R,C,ld,off", SHAPES)
def test_cols_shapes(red, orc, R, C, ld, off):
    say("cols shape R=%d C=%d ld=%d off=%d" % (R, C, ld, off))
    flat = workloads.uniform_f32(62, R * ld + off + 8, -4.0, 4.0)
    flat[off:off + R * ld].reshape(R, ld)[:, C:] = np.nan  # padding, never read
    fd = dev(flat)
    src = flat[off:off + R * ld].reshape(R, ld)
    sd = fd[off:off + R * ld].view(R, ld)
    old = workloads.uniform_f32(63, C, -2.0, 2.0)
    for op in ("sum", "max", "min"):
        for accum in (False, True):
            got = run_cols(red, op, sd, C, accum, old if accum else None)
            check_cols(orc, op, src, R, C, ld, got, accum, old if accum else None,
                       "R=%d C=%d ld=%d off=%d %s accum=%s" % (R, C, ld, off, op, accum))


def test_cols_special_values(red, orc):
    say("cols special values")
    nan, inf = float("nan"), float("inf")
    R, C = 300, 8
    t = workloads.uniform_f32(64, (R, C))
    t[:, 0] = nan                      # all NaN -> NaN
    t[::2, 1] = nan                    # some NaN -> ignored by max / min
    t[7, 2] = inf
    t[9, 3] = -inf
    t[:, 4] = 2.0 ** -149              # subnormals kept
    t[:, 5] = -0.0
    td = dev(t)
    for op in ("sum", "max", "min"):
        got = run_cols(red, op, td, C)
        check_cols(orc, op, t, R, C, C, got, what="special %s" % op)
    got = run_cols(red, "sum", td, C)
    assert got[4] == np.float32(R * 2.0 ** -149)
    assert got[2] == inf and got[3] == -inf and math.isnan(got[0])


@pytest.mark.parametrize("R,C", [(3000, 12), (1000, 130), (200000, 16), (300, 4099),
                                 (4096, 2048), (16, 262144)])
def test_cols_signed_zeros(red, orc, R, C):
    """Columns cycling through all -0, all +0, zeros of random signs, -0
    with one +0, negatives with one -0 and positives with one +0: a zero
    max / min carries the only sign of zero its column holds, and a zero
    sum is -0 exactly when every term is -0 (old -0 in even columns, +0 in
    odd ones under accum)."""
    say("cols signed zeros R=%d C=%d" % (R, C))
    t = np.ascontiguousarray(signed_zero_patterns(C, R, 70 + C).T)
    td = dev(t)
    old = np.where(np.arange(C) % 2 == 0, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    for op in ("sum", "max", "min"):
        for accum in (False, True):
            got = run_cols(red, op, td, C, accum, old if accum else None)
            check_cols(orc, op, t, R, C, C, got, accum, old if accum else None,
                       "signed zeros R=%d C=%d %s accum=%s" % (R, C, op, accum))


def test_cols_empty_untouched(red):
    say("cols empty")
    for op in ("sum", "max", "min"):
        out = torch.full((8,), 7.0, dtype=torch.float32, device="cuda")
        getattr(red, op + "_cols_f32")(torch.ones((0, 8), device="cuda"), out, accum=True)
        getattr(red, op + "_cols_f32")(torch.ones((4, 8), device="cuda"), out, C=0)
        assert (host(out) == 7.0).all()


def test_cols_deterministic(red, tile4k):
    say("cols determinism")
    _, td = tile4k
    ref = run_cols(red, "sum", td, 16384)
    for _ in range(2):
        assert run_cols(red, "sum", td, 16384).tobytes() == ref.tobytes()
