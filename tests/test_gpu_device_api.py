"""GPU parity of the device-side header include/reduce_device.hpp.

Test kernels in tests/device_api/ call each function of the header from
inside a kernel.  Thread-scope sums must reproduce the TVM page's eight-slot
order bit for bit (the oracle replays that order in C); max / min are
bit-exact everywhere; wave and workgroup sums, whose order is a fixed tree,
are held to the rounding bound of that tree."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from gpu_helpers import dev, extremes_match, has_both_zeros, host, say, zero_sum_sign_ok

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "device_api", "libdevapitest.so")
THREAD_SIZES = (1, 3, 5, 8, 9, 16, 17, 32, 33, 64)
OPS = {"sum": 0, "max": 1, "min": 2}
U = 2.0 ** -24  # unit roundoff of fp32


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBRARY):
        pytest.fail("tests/device_api/libdevapitest.so is not built "
                    "(python tests/device_api/build.py)")
    lib = ctypes.CDLL(LIBRARY)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.devtest_thread.argtypes = [P, I, I, P, I, I, P]
    lib.devtest_wave.argtypes = [P, I, P, I]
    lib.devtest_block.argtypes = [P, I, I, P, I]
    for f in (lib.devtest_thread, lib.devtest_wave, lib.devtest_block):
        f.restype = I
    return lib


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def specials(rows, n, rng):
    """Random rows with a few special rows planted: NaN, infinities, zeros of
    both signs, subnormals and values that cancel."""
    x = rng.uniform(-1.0, 1.0, (rows, n)).astype(np.float32)
    x[0] = -0.0
    x[1] = 0.0
    x[2, 0] = np.nan
    x[3] = np.nan
    x[4, -1] = np.inf
    x[5, 0] = -np.inf
    x[6] = np.float32(1e-42)  # subnormal
    x[7, :] = np.float32(3.0)
    x[7, ::2] = np.float32(-3.0)
    x[8] = rng.uniform(-1e30, 1e30, n).astype(np.float32)
    return x


def same_bits(got, want):
    """Element-wise bit equality, with any NaN matching any NaN."""
    return (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))


def run_thread(lib, x, op, accum=False, old=None):
    rows, n = x.shape
    xd = dev(x)
    out = torch.full((rows,), 7.0, dtype=torch.float32, device="cuda")
    oldd = dev(np.zeros(rows, np.float32) if old is None else old)
    rc = lib.devtest_thread(xd.data_ptr(), n, rows, out.data_ptr(), OPS[op],
                            int(accum), oldd.data_ptr())
    assert rc == 0, "launch failed: %d" % rc
    return host(out)


@pytest.mark.parametrize("n", THREAD_SIZES)
@pytest.mark.parametrize("accum", [False, True])
def test_thread_sum_page_order(lib, orc, n, accum):
    say("device header thread_sum N=%d accum=%d" % (n, accum))
    rng = np.random.default_rng(1000 + n)
    rows = 3000
    x = specials(rows, n, rng)
    old = rng.uniform(-4, 4, rows).astype(np.float32)
    old[10] = -0.0
    got = run_thread(lib, x, "sum", accum, old)
    want = orc.rows_page_sum_f32(x, rows, n, n, accum, old if accum else None)
    bad = np.nonzero(~same_bits(got, want))[0]
    assert bad.size == 0, "row %d: got %r want %r" % (bad[0], got[bad[0]], want[bad[0]])


@pytest.mark.parametrize("n", THREAD_SIZES)
@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("accum", [False, True])
def test_thread_extreme(lib, orc, n, op, accum):
    say("device header thread_%s N=%d accum=%d" % (op, n, accum))
    rng = np.random.default_rng(2000 + n)
    rows = 3000
    x = specials(rows, n, rng)
    old = rng.uniform(-2, 2, rows).astype(np.float32)
    old[11] = np.nan
    got = run_thread(lib, x, op, accum, old)
    fn = orc.rows_max_f32 if op == "max" else orc.rows_min_f32
    want = fn(x, rows, n, n, accum, old if accum else None)
    eq = extremes_match(got, want, has_both_zeros(x, old, accum, axis=1))
    bad = np.nonzero(~eq)[0]
    assert bad.size == 0, "row %d: got %r want %r" % (bad[0], got[bad[0]], want[bad[0]])


def test_thread_rejects_unknown_size(lib):
    say("device header thread size 7 is rejected by the launcher")
    rc = lib.devtest_thread(None, 7, 0, None, 0, 0, None)
    assert rc != 0


def check_groups(orc, x, got, op, depth, what):
    """x: (groups, m) inputs; got: (groups, m) outputs, every thread holding
    its group's result.  A sum over a tree of the given depth has error at
    most depth * u * sum|x| (first order)."""
    groups, m = x.shape
    assert (same_bits(got, got[:, :1].repeat(m, axis=1))).all(), \
        "%s: threads of one group disagree" % what
    res = got[:, 0].copy()
    if op == "sum":
        s, a = orc.rows_sum_f32(x, groups, m, m)
        finite = np.isfinite(s)
        tol = (depth + 1) * U
        err = np.abs(res[finite].astype(np.float64) - s[finite])
        assert (err <= tol * a[finite]).all(), "%s: worst %g" % (
            what, float((err / np.maximum(a[finite], 1e-300)).max()))
        nan = np.isnan(s)
        assert np.isnan(res[nan]).all(), what
        inf = np.isinf(s)
        assert (res[inf] == s[inf]).all(), what
        assert zero_sum_sign_ok(res, s).all(), "%s: zero sum with the wrong sign" % what
    else:
        fn = orc.rows_max_f32 if op == "max" else orc.rows_min_f32
        want = fn(x, groups, m, m)
        eq = extremes_match(res, want, has_both_zeros(x, axis=1))
        assert eq.all(), "%s: group %d" % (what, int(np.nonzero(~eq)[0][0]))


@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_wave(lib, orc, op):
    say("device header wave_%s over 2048 waves" % op)
    rng = np.random.default_rng(3000 + OPS[op])
    waves = 2048
    x = specials(waves, 64, rng)
    x[20, 5] = np.nan            # one NaN lane among finite values
    x[21, :63] = np.nan          # a single finite lane
    x[21, 63] = 2.5
    xd = dev(x)
    out = torch.empty(waves * 64, dtype=torch.float32, device="cuda")
    assert lib.devtest_wave(xd.data_ptr(), waves, out.data_ptr(), OPS[op]) == 0
    got = host(out).reshape(waves, 64)
    check_groups(orc, x, got, op, 6, "wave_%s" % op)
    # the result depends only on the inputs
    out2 = torch.empty_like(out)
    assert lib.devtest_wave(xd.data_ptr(), waves, out2.data_ptr(), OPS[op]) == 0
    assert (host(out2).view(np.uint32) == host(out).view(np.uint32)).all()


@pytest.mark.parametrize("waves", [1, 4, 16])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_block(lib, orc, waves, op):
    say("device header block_%s with %d waves" % (op, waves))
    rng = np.random.default_rng(4000 + 16 * OPS[op] + waves)
    blocks = 600
    m = 64 * waves
    x = specials(blocks, m, rng)
    x[30, m - 1] = np.nan        # NaN in the last wave only
    x[31, :] = np.nan
    x[31, m // 2] = -1.5         # a single finite value mid-block
    xd = dev(x)
    out = torch.empty(blocks * m, dtype=torch.float32, device="cuda")
    assert lib.devtest_block(xd.data_ptr(), blocks, waves, out.data_ptr(), OPS[op]) == 0
    got = host(out).reshape(blocks, m)
    check_groups(orc, x, got, op, 6 + waves - 1, "block_%s<%d>" % (op, waves))


def test_block_rejects_unknown_width(lib):
    say("device header block width 3 is rejected by the launcher")
    assert lib.devtest_block(None, 0, 3, None, 0) != 0
