"""GPU parity of the 1-D fp32 reductions (sum / max / min, accum, atomic
variant) against the CPU oracle: the full-size 2^24 and 2^30 + 7 vectors,
every small length with every 16-byte misalignment, special values,
extreme positions, exact integer sums and run-to-run determinism."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check_exact, check_sum, dev, has_both_zeros, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


OPS = ("sum", "max", "min")


def run(red, op, x_dev, accum=False, old=0.0, atomic=False):
    out = torch.full((1,), old, dtype=torch.float32, device="cuda")
    fn = getattr(red, "%s_f32%s" % (op, "_atomic" if atomic else ""))
    fn(x_dev, out, accum=accum)
    return host(out)[0]


def check(orc, op, x, got, accum=False, old=0.0, what=""):
    if op == "sum":
        s, a = orc.sum_f32(x, accum, old)
        check_sum(got, s, a, what)
        if a > 0 and x.size >= (1 << 20):
            say("%s: |gpu - exact| / sum|x| = %.3g (tolerance 1e-6)"
                % (what, abs(float(got) - s) / a))
    else:
        both = bool(has_both_zeros(x, np.float32(old), accum))
        want = orc.max_f32(x, accum, old) if op == "max" else orc.min_f32(x, accum, old)
        check_exact(got, want, what, both)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def vec16m():
    say("generate 2^24 uniform[-1,1) vector (seed 1)")
    x = workloads.vec16m()
    return x, dev(x)


@pytest.mark.parametrize("atomic", [False, True], ids=["twopass", "atomic"])
@pytest.mark.parametrize("accum", [False, True], ids=["noaccum", "accum3.25"])
@pytest.mark.parametrize("op", OPS)
def test_vec16m(red, orc, vec16m, op, accum, atomic):
    x, xd = vec16m
    old = workloads.ACCUM_PRESET if accum else 0.0
    say("vec16m op=%s accum=%s atomic=%s" % (op, accum, atomic))
    got = run(red, op, xd, accum, old, atomic)
    check(orc, op, x, got, accum, old, "vec16m %s" % op)
    if op == "max" and accum:
        assert got == np.float32(3.25)  # closed form: 3.25 exceeds every x


@pytest.fixture(scope="module")
def vec1g():
    say("generate 2^30+7 normal vector, 1% scaled by 1e6 (seed 3)")
    x = workloads.vec1g()
    return x, dev(x)


@pytest.mark.parametrize("op", OPS)
def test_vec1g(red, orc, vec1g, op):
    x, xd = vec1g
    say("vec1g n=2^30+7 op=%s" % op)
    got = run(red, op, xd)
    check(orc, op, x, got, what="vec1g %s" % op)


@pytest.mark.parametrize("op", OPS)
def test_vec1g_atomic(red, orc, vec1g, op):
    x, xd = vec1g
    say("vec1g atomic op=%s" % op)
    got = run(red, op, xd, atomic=True)
    check(orc, op, x, got, what="vec1g atomic %s" % op)


# ---------------------------------------------------------------------------
# small and ragged lengths, every misalignment
# ---------------------------------------------------------------------------

# (up to 4 x 8192 + 3 elements, the whole vector is one workgroup's loads in
# flight at once; the cases straddle that bound at every offset)
SIZES = (list(range(1, 18)) + [31, 32, 33, 63, 64, 65, 255, 256, 257, 1000,
                               4095, 4096, 4097, 8195, 8196, 32767, 32768, 32771,
                               32772, 32775, 65537]
         + [(1 << 20) + k for k in range(8)])


@pytest.fixture(scope="module")
def base():
    x = workloads.uniform_f32(21, (1 << 20) + 16, -10.0, 10.0)
    return x, dev(x)


@pytest.mark.parametrize("atomic", [False, True], ids=["twopass", "atomic"])
@pytest.mark.parametrize("n", SIZES)
def test_lengths_and_offsets(red, orc, base, n, atomic):
    x, xd = base
    say("lengths n=%d atomic=%s" % (n, atomic))
    for off in range(4):
        xs, xds = x[off:off + n], xd[off:off + n]
        for op in OPS:
            for accum, old in ((False, 0.0), (True, -2.5)):
                got = run(red, op, xds, accum, old, atomic)
                check(orc, op, xs, got, accum, old,
                      "n=%d off=%d %s accum=%s" % (n, off, op, accum))


@pytest.mark.parametrize("n", [7, 1000, (1 << 20) + 5])
def test_extreme_positions(red, orc, n):
    say("extreme positions n=%d" % n)
    rng = np.random.default_rng(22)
    for where in sorted({0, 1, n // 2, n - 4, n - 2, n - 1} & set(range(n))):
        x = rng.uniform(-1, 1, n).astype(np.float32)
        x[where] = 5.0
        assert run(red, "max", dev(x)) == np.float32(5.0), where
        x[where] = -5.0
        assert run(red, "min", dev(x)) == np.float32(-5.0), where


# Vectors of 128 MiB and more are streamed region by region (one contiguous
# eighth of the sweeps per XCD): lengths that leave a partial last sweep in
# the last region, odd element counts and misaligned starts.
REGIONAL = [((1 << 25), 0), ((1 << 25) + 7, 1), ((1 << 25) + 3 * 8192 + 5, 3),
            ((1 << 25) + 12345678, 2), ((1 << 26) - 1, 1)]


@pytest.fixture(scope="module")
def regional_base():
    say("generate the base vector of the regional cases")
    x = workloads.uniform_f32(41, (1 << 26) + 16, -3.0, 3.0)
    return x, dev(x)


@pytest.mark.parametrize("n,off", REGIONAL)
def test_regional_lengths(red, orc, regional_base, n, off):
    base, bd = regional_base
    x, xd = base[off:off + n], bd[off:off + n]
    say("regional n=%d off=%d" % (n, off))
    for op in OPS:
        for atomic in (False, True):
            for accum, old in ((False, 0.0), (True, -1.5)):
                got = run(red, op, xd, accum, old, atomic)
                check(orc, op, x, got, accum, old,
                      "regional n=%d off=%d %s atomic=%s accum=%s" % (n, off, op, atomic, accum))
    check_fused(red, orc, x, xd, True, (2.0, -7.0, 7.0), "regional n=%d off=%d" % (n, off))


def test_integer_sums_are_exact(red):
    """Integers in [-8, 8]: every partial sum is an integer below 2^24, so
    every order is exact and the fp32 result equals the exact sum."""
    say("integer sums")
    for n, seed in (((1 << 20) + 3, 23), (12345, 24), (2, 25)):
        x = workloads.integers_i32(seed, n, -8, 9).astype(np.float32)
        want = float(np.sum(x.astype(np.int64)))
        assert run(red, "sum", dev(x)) == want
        assert run(red, "sum", dev(x), True, 7.0) == want + 7.0


SPECIAL_CASES = [
    [float("nan"), 1.0, float("nan"), -3.0],
    [float("nan")] * 9,
    [float("nan")] * 3000 + [2.0] + [float("nan")] * 3000,
    [float("inf"), 1.0, -2.0],
    [-float("inf"), 1.0, 5.0] * 100,
    [float("inf"), -float("inf"), 1.0],
    [2.0 ** -149, -(2.0 ** -149), 0.0, 2.0 ** -140] * 50,
    [-(2.0 ** -149), -(2.0 ** -126) + 2.0 ** -149] * 3,
    [0.0, -0.0] * 1000,
    [-0.0] * 17,
    [-0.0] * 20000,
    [0.0] * 17,
    [0.0] * 20000,
    [-0.0] * 9000 + [0.0] + [-0.0] * 9000,
    [-1.0, -0.0, -2.0] * 7,
    [1.0, -0.0, 2.0] * 7,
    [1.0, -1.0] * 5000,
]


@pytest.mark.parametrize("atomic", [False, True])
def test_special_values(red, orc, atomic):
    """NaN, infinities, subnormals and signed zeros through the
    deterministic and the single-pass atomic entry points, with and
    without accum (old -0.0, +0.0 and 1.5)."""
    say("special values atomic=%s" % atomic)
    for vals in SPECIAL_CASES:
        x = np.array(vals, np.float32)
        xd = dev(x)
        for op in OPS:
            for accum, old in ((False, 0.0), (True, -0.0), (True, 0.0), (True, 1.5)):
                got = run(red, op, xd, accum, old, atomic)
                what = "special %s atomic=%s accum=%s old=%r n=%d %s" % (
                    op, atomic, accum, old, len(vals), vals[:4])
                check(orc, op, x, got, accum, old, what)
    # subnormals are summed, not flushed: exact small integer multiples
    for n in (1000, 100000):
        x = np.full(n, 2.0 ** -149, np.float32)
        assert run(red, "sum", dev(x), atomic=atomic) == np.float32(n * 2.0 ** -149), n
        assert run(red, "sum", dev(-x), atomic=atomic) == np.float32(-n * 2.0 ** -149), n
    # accum under NaN policy
    x = dev(np.array([float("nan"), float("nan")], np.float32))
    assert run(red, "max", x, True, 1.5, atomic) == np.float32(1.5)
    assert math.isnan(run(red, "min", x, atomic=atomic))


def test_special_values_fused(red, orc):
    """The same special values through the fused sum / max / min call:
    each result bit-identical to the single call's and checked against the
    oracle."""
    say("special values fused")
    for vals in SPECIAL_CASES:
        x = np.array(vals, np.float32)
        xd = dev(x)
        for accum, old in ((False, 0.0), (True, -0.0), (True, 0.0), (True, 1.5)):
            check_fused(red, orc, x, xd, accum, (old, old, old),
                        "special n=%d %s accum=%s old=%r" % (len(vals), vals[:4], accum, old))


def test_empty_leaves_out_untouched(red):
    say("empty input")
    x = torch.empty(0, dtype=torch.float32, device="cuda")
    for op in OPS:
        for atomic in (False, True):
            for accum in (False, True):
                assert run(red, op, x, accum, 42.0, atomic) == np.float32(42.0)


def test_deterministic(red, vec16m):
    """The default path gives the same bits every time and on any stream."""
    say("determinism")
    _, xd = vec16m
    for op in OPS:
        ref = run(red, op, xd)
        for _ in range(3):
            assert np.float32(run(red, op, xd)).tobytes() == np.float32(ref).tobytes()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            out = torch.zeros(1, dtype=torch.float32, device="cuda")
            getattr(red, op + "_f32")(xd, out)
        s.synchronize()
        assert host(out)[0].tobytes() == np.float32(ref).tobytes()


def test_plan_matches_call(red, vec16m):
    """A pre-marshalled plan enqueues the same call: same bits."""
    say("plan vs call")
    _, xd = vec16m
    for op in OPS:
        ref = run(red, op, xd, True, 1.25)
        out = torch.full((1,), 1.25, dtype=torch.float32, device="cuda")
        p = red.plan(op + "_f32", xd, out, accum=True)
        p()
        assert host(out)[0].tobytes() == np.float32(ref).tobytes()
    with pytest.raises(red.ReduceError):
        bad = red.plan("sum_f32", xd, torch.zeros(1, device="cuda"))
        bad.args = (0,) + bad.args[1:]  # a null input pointer is rejected
        bad()


# ---------------------------------------------------------------------------
# fused sum + max + min (one read)
# ---------------------------------------------------------------------------

def run_fused(red, x_dev, accum=False, old=(0.0, 0.0, 0.0)):
    out = torch.tensor(list(old), dtype=torch.float32, device="cuda")
    red.sum_max_min_f32(x_dev, out, accum=accum)
    return host(out)


def check_fused(red, orc, x, xd, accum, old, what):
    got = run_fused(red, xd, accum, old)
    for j, op in enumerate(OPS):
        sep = run(red, op, xd, accum, old[j])
        assert got[j].tobytes() == np.float32(sep).tobytes(), (what, op, got[j], sep)
        check(orc, op, x, got[j], accum, old[j], "%s fused %s" % (what, op))


@pytest.mark.parametrize("accum", [False, True], ids=["noaccum", "accum"])
def test_fused_vec16m(red, orc, vec16m, accum):
    """One read gives the same three results, bit for bit, as three calls."""
    x, xd = vec16m
    say("fused vec16m accum=%s" % accum)
    old = (3.25, 3.25, 3.25) if accum else (0.0, 0.0, 0.0)
    check_fused(red, orc, x, xd, accum, old, "vec16m")


def test_fused_vec1g(red, orc, vec1g):
    x, xd = vec1g
    say("fused vec1g")
    check_fused(red, orc, x, xd, False, (0.0, 0.0, 0.0), "vec1g")


@pytest.mark.parametrize("n", [1, 3, 7, 8, 9, 33, 257, 4097, 32771, 32772, (1 << 20) + 5])
def test_fused_lengths(red, orc, base, n):
    x, xd = base
    say("fused lengths n=%d" % n)
    for off in range(4):
        for accum, old in ((False, (0.0, 0.0, 0.0)), (True, (-2.5, 100.0, -100.0))):
            check_fused(red, orc, x[off:off + n], xd[off:off + n], accum, old,
                        "n=%d off=%d" % (n, off))


def test_workspace_allocation_failure(red, vec16m):
    """A failed workspace allocation is reported as RED_ERR_NOMEM, nothing
    is enqueued, and the next call on that stream allocates normally.  The
    failure is forced from the host (RED_TEST_FAIL_ALLOC=1 makes the library
    skip hipMalloc for a new stream's workspace)."""
    import os
    say("workspace allocation failure on a new stream")
    _, xd = vec16m
    ref = run(red, "sum", xd)
    s = torch.cuda.Stream()
    out = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    os.environ["RED_TEST_FAIL_ALLOC"] = "1"
    try:
        with pytest.raises(red.ReduceError) as err:
            red.sum_f32(xd, out, stream=s)
        assert err.value.status == red.RED_ERR_NOMEM
        # The atomic variant needs no workspace and still runs.
        red.sum_f32_atomic(xd, out, stream=s)
        s.synchronize()
        check_sum(host(out)[0], *oracle.get().sum_f32(workloads.vec16m()), "atomic")
    finally:
        del os.environ["RED_TEST_FAIL_ALLOC"]
    out.fill_(7.0)
    torch.cuda.synchronize()
    red.sum_f32(xd, out, stream=s)
    s.synchronize()
    assert host(out)[0].tobytes() == np.float32(ref).tobytes()


def _f32_from_bits(u):
    return np.array([u], np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("op", ["max", "min"])
def test_atomic_extremes(red, orc, op):
    """The atomic max / min fold every workgroup's partial with one integer
    atomic on the fp32 bit pattern (signed for a non-negative partial,
    unsigned for a negative one).  Cover partials of both signs and of one
    sign only, NaN shares, signed zeros, and every kind of old value under
    accum: numbers, infinities, zeros, and NaNs of either sign and with
    payloads (the NaN that wins the integer comparison is swapped out by
    compare-and-swap first)."""
    say("atomic %s: signs, NaN, zeros, old values" % op)
    n = 1 << 20  # 128 workgroups
    rng = np.random.default_rng(77)
    base = rng.standard_normal(n).astype(np.float32)
    arrays = {
        "mixed": base,
        "all_negative": -np.abs(base) - np.float32(0.5),
        "all_positive": np.abs(base) + np.float32(0.5),
        "first_half_nan": np.where(np.arange(n) < n // 2, np.float32(np.nan), base),
        "all_nan": np.full(n, np.nan, np.float32),
        "zeros": np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)),
        "neg_zeros": np.full(n, -0.0, np.float32),
    }
    olds = [0.0, -0.0, 1.5, -1.5, 1e30, -1e30, float("inf"), float("-inf"),
            _f32_from_bits(0x7fc00000), _f32_from_bits(0xffc00000),
            _f32_from_bits(0x7f800001), _f32_from_bits(0xffffffff)]
    fn = getattr(red, op + "_f32_atomic")
    for name, x in arrays.items():
        xd = dev(x)
        got = run(red, op, xd, atomic=True)
        check(orc, op, x, got, what="atomic %s %s" % (op, name))
        for old in olds:
            old = np.float32(old)
            out = dev(np.array([old], np.float32))  # keeps the NaN's sign and payload
            fn(xd, out, accum=True)
            got = host(out)[0]
            check(orc, op, x, got, True, old, "atomic %s %s old=%08x" % (
                op, name, int(np.array([old]).view(np.uint32)[0])))
