"""GPU parity of the segmented row reductions against the CPU oracle.

Rows of at most 64 elements run the TVM page's thread-scope order and must
match the oracle's replay of that order bit for bit; longer rows are held
to the sum tolerance; max / min are bit-exact everywhere."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (check_exact, check_extremes, check_sum, check_sums, dev,
                         has_both_zeros, host, say, signed_zero_patterns,
                         valid_region)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run_rows(red, op, xd, n, old=None, accum=False):
    rows = xd.shape[0]
    out = (torch.zeros(rows, dtype=torch.float32, device="cuda") if old is None
           else dev(np.asarray(old, np.float32)))
    getattr(red, "%s_rows_f32" % op)(xd, out, n=n, accum=accum)
    return host(out)


def check_rows(orc, op, x, n, got, accum=False, old=None, what=""):
    rows, ld = x.shape
    if op == "sum":
        if n <= 64:  # the page's own order, bit for bit
            want = orc.rows_page_sum_f32(x, rows, n, ld, accum, old)
            bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
            assert bad.size == 0, "%s: row %d got %r want %r" % (
                what, bad[0], got[bad[0]], want[bad[0]])
        s, a = orc.rows_sum_f32(x, rows, n, ld, accum, old)
        check_sums(got, s, a, what)
        with np.errstate(invalid="ignore"):
            err = np.abs(got.astype(np.float64) - s)
        return float(np.nanmax(err / np.maximum(a, 1e-300), initial=0.0))
    else:
        fn = orc.rows_max_f32 if op == "max" else orc.rows_min_f32
        want = fn(x, rows, n, ld, accum, old)
        both = has_both_zeros(valid_region(x, x.shape[0], n, x.shape[1]), old, accum, axis=1)
        check_extremes(got, want, both, what)


@pytest.fixture(scope="module")
def rows32():
    say("generate 4096 x 32 rows (seed 0)")
    a, _ = workloads.rows32()
    return a, dev(a)


@pytest.mark.parametrize("accum", [False, True])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_rows32(red, orc, rows32, op, accum):
    x, xd = rows32
    say("rows32 op=%s accum=%s" % (op, accum))
    old = workloads.uniform_f32(30, 4096, -3.0, 3.0) if accum else None
    got = run_rows(red, op, xd, 32, old, accum)
    check_rows(orc, op, x, 32, got, accum, old, "rows32 %s" % op)


def test_rows32_demo_sum_is_exact_for_integers(red):
    """The page's demonstration length (32 elements, one thread): with
    integer values the result equals the exact sum."""
    say("rows32 integer demo")
    x = workloads.integers_i32(31, (4096, 32), -100, 101).astype(np.float32)
    got = run_rows(red, "sum", dev(x), 32)
    assert (got == x.astype(np.int64).sum(axis=1)).all()


@pytest.fixture(scope="module")
def rows1000():
    say("generate 65536 x 1000 rows (seed 4)")
    x = workloads.rows1000_x()
    return x, dev(x)


@pytest.mark.parametrize("op", ["sum", "max"])
def test_rows1000(red, orc, rows1000, op):
    x, xd = rows1000
    say("rows1000 op=%s" % op)
    got = run_rows(red, op, xd, 1000)
    worst = check_rows(orc, op, x, 1000, got, what="rows1000 %s" % op)
    if op == "sum":
        say("rows1000 sum: worst |gpu - exact| / sum|x| = %.3g (tolerance 1e-6)" % worst)


SHAPES = [  # (rows, n, ld, element offset of the base pointer)
    (1, 1, 1, 0), (5, 7, 7, 0), (9, 8, 8, 0), (9, 9, 9, 1), (33, 17, 19, 2),
    (300, 64, 64, 0), (300, 64, 67, 3), (257, 65, 65, 0), (100, 100, 103, 1),
    (70, 1000, 1000, 2), (3, 4097, 4100, 0), (1, 16385, 16385, 0),
    (2, 100003, 100010, 1), (4096, 31, 32, 0), (2049, 250, 256, 0),
    # every lanes-per-row / rows-per-wave choice of the 64 < n <= 1024 kernel,
    # at its boundaries, with row counts that leave ragged workgroup steps
    (1, 65, 65, 0), (17, 127, 127, 1), (33, 128, 128, 0), (63, 129, 131, 3),
    (100, 200, 200, 2), (65, 255, 255, 1), (129, 256, 256, 0), (7, 257, 260, 0),
    (1000, 300, 300, 3), (31, 511, 511, 2), (4099, 512, 512, 0), (9, 513, 515, 1),
    (70, 700, 701, 0), (5, 1023, 1023, 3), (300, 1024, 1024, 0),
    (300000, 100, 100, 0), (70001, 384, 384, 1),
    # 17 to 64 elements staged as one span (stride <= 64, or <= 128 with
    # padding of at most an eighth of the row): unaligned starts, padding,
    # and the last tile cut short; then strides just past that rule, read
    # element by element
    (5000, 40, 40, 1), (777, 64, 64, 3), (3000, 17, 18, 1), (2049, 33, 36, 0),
    (129, 50, 64, 2), (100_001, 24, 28, 0),
    (3000, 64, 65, 0), (777, 64, 72, 1), (2049, 60, 67, 3), (5000, 40, 45, 2),
    (100_001, 33, 37, 0), (300, 64, 73, 0), (1000, 48, 60, 1), (2000, 17, 33, 1),
    (999, 20, 24, 3), (7001, 30, 30, 2), (2049, 62, 62, 0), (1000, 26, 30, 1),
    # long rows: split into chunks per row (with and without a second pass)
    (5, 300000, 300001, 1), (600, 20000, 20000, 0), (100, 5000, 5003, 2),
    (3000, 2000, 2000, 0), (1, (1 << 22) + 3, (1 << 22) + 3, 0), (37, 65536, 65540, 3),
]


@pytest.mark.parametrize("rows,n,ld,off", SHAPES)
def test_rows_shapes(red, orc, rows, n, ld, off):
    say("rows shape rows=%d n=%d ld=%d off=%d" % (rows, n, ld, off))
    flat = workloads.uniform_f32(32, rows * ld + off + 4, -4.0, 4.0)
    flat[off:off + rows * ld].reshape(rows, ld)[:, n:] = np.nan  # padding
    fd = dev(flat)
    x = flat[off:off + rows * ld].reshape(rows, ld)
    xd = fd[off:off + rows * ld].view(rows, ld)
    old = workloads.uniform_f32(33, rows, -2.0, 2.0)
    for op in ("sum", "max", "min"):
        for accum in (False, True):
            got = run_rows(red, op, xd, n, old if accum else None, accum)
            check_rows(orc, op, x, n, got, accum, old if accum else None,
                       "rows=%d n=%d ld=%d off=%d %s accum=%s" % (rows, n, ld, off, op, accum))


# Rows of 1 to 7 elements.  Up to 4 elements: 8 rows per thread and step,
# a grid of a few workgroups per CU walking 2048-row steps; row counts end
# inside a step and inside a thread's 8 rows, and the largest need several
# grid passes.  5 to 7 elements: one row per thread.
SHORT = [  # (rows, n, ld, element offset of the base pointer)
    (1, 1, 1, 0), (255, 1, 1, 0), (2049, 1, 1, 1), (3_000_001, 1, 1, 0), (100_000, 1, 4, 2),
    (257, 2, 2, 0), (1_100_000, 2, 2, 0), (70_001, 2, 3, 1), (4097, 3, 3, 0),
    (2_500_003, 3, 3, 0), (33_333, 3, 4, 3), (2047, 4, 4, 0), (600_001, 4, 4, 0),
    (10_000, 4, 5, 1), (9999, 5, 5, 0), (700_007, 5, 8, 0), (6143, 6, 6, 2),
    (800_000, 6, 6, 0), (2049, 7, 7, 3), (900_001, 7, 7, 0), (12_345, 7, 16, 0),
]


@pytest.mark.parametrize("rows,n,ld,off", SHORT)
def test_rows_short(red, orc, rows, n, ld, off):
    say("rows short rows=%d n=%d ld=%d off=%d" % (rows, n, ld, off))
    flat = workloads.uniform_f32(34, rows * ld + off + 4, -4.0, 4.0)
    flat[off:off + rows * ld].reshape(rows, ld)[:, n:] = np.nan  # padding
    fd = dev(flat)
    x = flat[off:off + rows * ld].reshape(rows, ld)
    xd = fd[off:off + rows * ld].view(rows, ld)
    old = workloads.uniform_f32(35, rows, -2.0, 2.0)
    for op in ("sum", "max", "min"):
        for accum in (False, True):
            got = run_rows(red, op, xd, n, old if accum else None, accum)
            check_rows(orc, op, x, n, got, accum, old if accum else None,
                       "rows=%d n=%d ld=%d off=%d %s accum=%s" % (rows, n, ld, off, op, accum))


@pytest.mark.parametrize("rows,n", [(3000, 1), (3000, 3), (3000, 7), (3000, 32), (3000, 40),
                                    (3000, 100), (300, 1000), (300, 2000), (5, 70000)])
def test_rows_signed_zeros(red, orc, rows, n):
    """A zero result carries the only sign of zero the row holds (max /
    min), and a zero sum is -0 exactly when every term is -0; under accum
    the old value (-0 in even rows, +0 in odd ones) takes part."""
    say("rows signed zeros rows=%d n=%d" % (rows, n))
    x = signed_zero_patterns(rows, n, 40 + n)
    xd = dev(x)
    old = np.where(np.arange(rows) % 2 == 0, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    for op in ("sum", "max", "min"):
        for accum in (False, True):
            got = run_rows(red, op, xd, n, old if accum else None, accum)
            check_rows(orc, op, x, n, got, accum, old if accum else None,
                       "signed zeros rows=%d n=%d %s accum=%s" % (rows, n, op, accum))


def test_rows_empty_untouched(red):
    say("rows empty")
    x = torch.ones((4, 8), dtype=torch.float32, device="cuda")
    for op in ("sum", "max", "min"):
        out = torch.full((4,), 9.5, dtype=torch.float32, device="cuda")
        getattr(red, op + "_rows_f32")(x, out, n=0, accum=True)
        assert (host(out) == 9.5).all()
        e = torch.ones((0, 8), dtype=torch.float32, device="cuda")
        getattr(red, op + "_rows_f32")(e, out, n=8)
        assert (host(out) == 9.5).all()
