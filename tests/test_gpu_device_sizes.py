"""GPU parity under the launch plans of other device sizes.

Every launch plan starts from the device's compute-unit count: the 1-D
grids (and whether a long vector is streamed region by region, which needs
a count divisible by the 8 XCDs), the row kernels' workgroup caps and row
splits, and the column kernels' choice of layout, row shares and second
pass.  The library's test hook RED_TEST_CUS replaces that count, so these
cases run the plans of a 1-CU device, an odd count that no XCD split
divides, one 32-CU partition of an MI355X, a 304-CU part and a 2048-CU
part on this GPU, and check every entry point against the oracle as the
other parity tests do.  (A 2048-CU plan streams a 256 MiB vector on 2048
workgroups, whose 24 KiB of partials exceed the allocation-free call's
16 KiB buffer: that call must refuse it and enqueue nothing.)"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (COLPROD_16_TOL, COLPROD_F32_TOL, check_exact, check_extremes,
                         check_rel, check_sum, check_sums, dev, has_both_zeros, host, say,
                         valid_region)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CUS = [1, 7, 32, 304, 2048]


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(params=CUS, ids=lambda c: "cus%d" % c)
def cus(request, monkeypatch):
    monkeypatch.setenv("RED_TEST_CUS", str(request.param))
    return request.param


def vector(seed, n, off):
    """n values uniform in [-1, 1) with a few scaled by 1e6, starting `off`
    elements into a device buffer."""
    x = workloads.uniform_f32(seed, n)
    x[:: 9973] *= np.float32(1e6)
    flat = np.zeros(n + off, np.float32)
    flat[off:] = x
    return x, dev(flat)[off:]


def stream_grid(n, off, cus):
    """Workgroups of the 1-D first pass for n elements starting `off`
    elements past a 16-byte boundary: one per 32 KiB sweep of whole 16-byte
    vectors, at most one per CU; from 256 MiB, on a CU count divisible by 8
    (and at least one sweep per CU), exactly one per CU."""
    head = min((4 - off % 4) % 4, n)
    sweeps = -(-((n - head) // 4) // 8192)
    if 4 * n >= (256 << 20) and cus % 8 == 0 and sweeps >= cus:
        return cus
    return max(1, min(sweeps, cus))


@pytest.mark.parametrize("n,off", [(100, 0), (9000, 1), ((1 << 22) + 5, 3), ((1 << 26) + 7, 0)])
def test_vector(red, orc, cus, n, off):
    what = "1-D n=%d off=%d cus=%d" % (n, off, cus)
    say(what)
    x, xd = vector(40 + off, n, off)
    s, a = orc.sum_f32(x)
    mx, mn = orc.max_f32(x), orc.min_f32(x)
    outs = {}
    for op in ("sum", "max", "min"):
        out = torch.zeros(1, device="cuda")
        getattr(red, op + "_f32")(xd, out)
        outs[op] = host(out)[0]
    check_sum(outs["sum"], s, a, what)
    check_exact(outs["max"], mx, what + " max")
    check_exact(outs["min"], mn, what + " min")
    fused = torch.zeros(3, device="cuda")
    red.sum_max_min_f32(xd, fused)
    f = host(fused)
    want = np.array([outs["sum"], outs["max"], outs["min"]], np.float32)
    assert (f.view(np.uint32) == want.view(np.uint32)).all(), (what, f, want)
    # the allocation-free call: the same results, or a refusal when the
    # plan's partials exceed its static buffer
    noalloc = torch.full((3,), 7.0, device="cuda")
    if stream_grid(n, off, cus) * 12 > 16384:
        with pytest.raises(red.ReduceError) as e:
            red.sum_max_min_f32_noalloc(xd, noalloc)
        assert e.value.status == red.RED_ERR_SCRATCH
        assert (host(noalloc) == 7.0).all(), what
    else:
        red.sum_max_min_f32_noalloc(xd, noalloc)
        assert (host(noalloc).view(np.uint32) == f.view(np.uint32)).all(), what
    # the single-pass variants, with accum into a preset value
    for op in ("sum", "max", "min"):
        out = dev(np.array([0.25], np.float32))
        getattr(red, op + "_f32_atomic")(xd, out, accum=True)
        got = host(out)[0]
        if op == "sum":
            s2, a2 = orc.sum_f32(x, accum=True, old=0.25)
            check_sum(got, s2, a2, what + " atomic sum")
        else:
            want1 = getattr(orc, op + "_f32")(x, accum=True, old=0.25)
            check_exact(got, want1, what + " atomic " + op)


# (rows, n, ld): one shape for each row kernel (short, one thread per row,
# LDS tile, segment, one wave per row, split rows with a second pass).
ROWS = [(5000, 3, 3), (3000, 12, 13), (4000, 40, 41), (5000, 300, 300),
        (3000, 2000, 2000), (64, 3000, 3000), (3, 70_000, 70_001)]


@pytest.mark.parametrize("rows,n,ld", ROWS)
def test_rows(red, orc, cus, rows, n, ld):
    what = "rows %d x %d ld %d cus=%d" % (rows, n, ld, cus)
    say(what)
    x = workloads.uniform_f32(50 + n, rows * ld).reshape(rows, ld)
    old = workloads.uniform_f32(51 + n, rows, -3.0, 3.0)
    xd = dev(x)
    out = dev(old.copy())
    red.sum_rows_f32(xd, out, n=n, accum=True)
    s, a = orc.rows_sum_f32(x, rows, n, ld, True, old)
    check_sums(host(out), s, a, what)
    for op in ("max", "min"):
        out = torch.zeros(rows, dtype=torch.float32, device="cuda")
        getattr(red, op + "_rows_f32")(xd, out, n=n)
        want = getattr(orc, "rows_%s_f32" % op)(x, rows, n, ld)
        both = has_both_zeros(valid_region(x, rows, n, ld), axis=1)
        check_extremes(host(out), want, both, what + " " + op)


def factors(seed, shape):
    """+-1 with rare +-2 and +-0.5: exact products whatever the order."""
    rng = np.random.default_rng(seed)
    u = rng.random(shape)
    v = np.where(u < 3e-4, 2.0, np.where(u < 6e-4, 0.5, 1.0))
    return (v * np.where(rng.random(shape) < 0.5, -1.0, 1.0)).astype(np.float32)


# (kind, R, C, ld): one block per workgroup (rows shared or not), several
# blocks per workgroup, wide strips, unaligned rows, narrow rows.
COLS = [("f32", 4096, 4096, 4096), ("f32", 64, 65536, 65536), ("f32", 1500, 1000, 1003),
        ("f32", 20_000, 12, 12), ("bf16", 2048, 2048, 2048), ("f16", 777, 3000, 3000),
        ("i32", 1000, 1000, 1003), ("i32", 3000, 8192, 8192),
        ("f16", 10, 1_187_589, 1_187_592), ("bf16", 3, 300_100, 300_104)]


@pytest.mark.parametrize("kind,R,C,ld", COLS)
def test_colprod(red, orc, cus, kind, R, C, ld):
    what = "colprod %s %d x %d ld %d cus=%d" % (kind, R, C, ld, cus)
    say(what)
    if kind == "i32":
        src = workloads.integers_i32(60 + C, R * ld, -(2 ** 31), 2 ** 31).reshape(R, ld) | 1
        out = torch.zeros(C, dtype=torch.int32, device="cuda")
        red.colprod_i32(dev(src), out, C=C)
        got, want = host(out), orc.colprod_i32(src, R, C, ld)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "%s: column %d" % (what, bad[0])
        return
    x = factors(60 + C, (R, ld))
    if kind == "f32":
        out = torch.zeros(C, dtype=torch.float32, device="cuda")
        red.colprod_f32(dev(x), out, C=C)
        check_rel(host(out), orc.colprod_f32(x, R, C, ld), COLPROD_F32_TOL, what)
        return
    bits = (workloads.to_f16_bits if kind == "f16" else workloads.to_bf16_bits)(x.reshape(-1))
    bits = bits.reshape(R, ld)
    tdt = torch.float16 if kind == "f16" else torch.bfloat16
    out = torch.zeros(C, dtype=tdt, device="cuda")
    getattr(red, "colprod_" + kind)(dev(bits.view(np.int16)).view(tdt), out, C=C)
    want = (orc.colprod_f16 if kind == "f16" else orc.colprod_bf16)(bits, R, C, ld)
    check_rel(host(out.float()), want, COLPROD_16_TOL, what)


@pytest.mark.parametrize("R,C,ld", [(3000, 700, 700), (200, 5000, 5001), (50_000, 8, 8)])
def test_cols(red, orc, cus, R, C, ld):
    what = "cols %d x %d ld %d cus=%d" % (R, C, ld, cus)
    say(what)
    x = workloads.uniform_f32(70 + C, R * ld).reshape(R, ld)
    old = workloads.uniform_f32(71 + C, C, -3.0, 3.0)
    xd = dev(x)
    out = dev(old.copy())
    red.sum_cols_f32(xd, out, C=C, accum=True)
    s, a = orc.cols_sum_f32(x, R, C, ld, True, old)
    check_sums(host(out), s, a, what)
    for op in ("max", "min"):
        out = dev(old.copy())
        getattr(red, op + "_cols_f32")(xd, out, C=C, accum=True)
        want = getattr(orc, "cols_%s_f32" % op)(x, R, C, ld, True, old)
        both = has_both_zeros(valid_region(x, R, C, ld), old, True, axis=0)
        check_extremes(host(out), want, both, what + " " + op)
