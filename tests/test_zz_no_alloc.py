"""The allocation-free fused call red_sum_max_min_f32_noalloc, through the
C ABI: its results must equal red_sum_max_min_f32's bit for bit (same
kernels and grid, partials in the static scratch instead of a workspace)
and match the oracle, on two calls in a row, the second with a smaller
input, and with accum; a grid that would need more scratch than the
buffer holds is refused (forced from the host with the library's
RED_TEST_SCRATCH_LIMIT hook), with nothing enqueued; and calls captured
into a HIP graph on a stream without a workspace replay to the eager
results."""
import ctypes
import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check_exact, check_sum, dev, has_both_zeros, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LIBRARY = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "fp32_reductions_amd", "libreduce.so")
RED_OK, RED_ERR_SCRATCH = 0, 5


@pytest.fixture(scope="module")
def lib():
    import fp32_reductions_amd  # noqa: F401  (the library this process uses)
    lib = ctypes.CDLL(LIBRARY)
    for name in ("red_sum_max_min_f32", "red_sum_max_min_f32_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                       ctypes.c_void_p]
        fn.restype = ctypes.c_int
    return lib


def enqueue(lib, name, xd, old, accum):
    """Enqueue one call on torch's current stream; returns its out tensor."""
    out = dev(np.array(old, np.float32))
    stream = torch.cuda.current_stream().cuda_stream
    rc = getattr(lib, name)(xd.data_ptr(), xd.numel(), out.data_ptr(), int(accum), stream)
    assert rc == RED_OK, (name, rc)
    return out


def call(lib, name, xd, old, accum):
    return host(enqueue(lib, name, xd, old, accum))


def check_oracle(x, got, accum, old, what):
    orc = oracle.get()
    s, a = orc.sum_f32(x, accum, old[0])
    check_sum(got[0], s, a, what + " sum")
    for k, op in ((1, "max"), (2, "min")):
        want = getattr(orc, op + "_f32")(x, accum, old[k])
        check_exact(got[k], want, what + " " + op,
                    bool(has_both_zeros(x, np.float32(old[k]), accum)))


@pytest.mark.parametrize("accum", [False, True])
def test_noalloc_matches_fused_call(lib, accum):
    """Two calls in a row on the static scratch, enqueued back to back:
    2^24 + 3 elements (the full grid), then 100003 elements (a smaller grid,
    the first call's partials still in the buffer)."""
    old = (3.25, 3.25, 3.25) if accum else (0.0, 0.0, 0.0)
    cases = [((1 << 24) + 3, 600), (100003, 601)]
    xs = [workloads.uniform_f32(seed, n, -2.0, 2.0) for n, seed in cases]
    xds = [dev(x) for x in xs]
    torch.cuda.synchronize()
    say("noalloc two calls in a row, n=%s accum=%s" % ([n for n, _ in cases], accum))
    outs = [enqueue(lib, "red_sum_max_min_f32_noalloc", xd, old, accum) for xd in xds]
    got = [host(o) for o in outs]
    for x, xd, g in zip(xs, xds, got):
        want = call(lib, "red_sum_max_min_f32", xd, old, accum)
        assert g.tobytes() == want.tobytes(), (x.size, g, want)
        check_oracle(x, g, accum, old, "noalloc n=%d" % x.size)


def test_noalloc_short_and_misaligned(lib):
    """One-workgroup grids (the first kernel writes the result itself) and
    a start that is not 16-byte aligned."""
    base = workloads.uniform_f32(602, 70001)
    bd = dev(base)
    for off, n in ((0, 1), (1, 7), (3, 8195), (2, 70000 - 2)):
        say("noalloc short n=%d off=%d" % (n, off))
        x, xd = base[off:off + n], bd[off:off + n]
        got = call(lib, "red_sum_max_min_f32_noalloc", xd, (1.0, -5.0, 5.0), True)
        want = call(lib, "red_sum_max_min_f32", xd, (1.0, -5.0, 5.0), True)
        assert got.tobytes() == want.tobytes(), (n, off)
        check_oracle(x, got, True, (1.0, -5.0, 5.0), "noalloc short n=%d" % n)


def test_noalloc_rejects_a_grid_beyond_the_scratch(lib, monkeypatch):
    """With the scratch limit lowered from the host to 1 KiB (room for the
    partials of 85 workgroups), a full grid (one workgroup per CU) is
    refused and the destination is left untouched; an 8-workgroup grid
    still runs."""
    say("noalloc scratch limit")
    monkeypatch.setenv("RED_TEST_SCRATCH_LIMIT", "1024")
    x = workloads.uniform_f32(603, 1 << 24)
    xd = dev(x)
    out = dev(np.array([7.0, 7.0, 7.0], np.float32))
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.red_sum_max_min_f32_noalloc(xd.data_ptr(), xd.numel(), out.data_ptr(), 0, stream)
    assert rc == RED_ERR_SCRATCH
    assert (host(out) == 7.0).all()
    small = xd[: 8 * 2048 * 4]            # 8 sweeps of 32 KiB: 8 workgroups
    got = call(lib, "red_sum_max_min_f32_noalloc", small, (0.0, 0.0, 0.0), False)
    check_oracle(x[: 8 * 2048 * 4], got, False, (0.0, 0.0, 0.0), "noalloc under the limit")


def test_noalloc_graph_replay(lib):
    """The use the entry point exists for: two calls captured into a HIP
    graph on a stream that has never made a library call (they need no
    workspace), the second smaller and with accum, after one eager call on
    the device (which looks up the scratch address), then replayed four
    times with new inputs copied in between and an eager fused call on
    another stream in between; every replay equals the eager fused call
    bit for bit."""
    say("noalloc graph capture and 4 replays")
    n1, n2 = (1 << 22) + 5, 100003
    x1 = torch.empty(n1, dtype=torch.float32, device="cuda")
    x2 = torch.empty(n2, dtype=torch.float32, device="cuda")
    o1 = torch.zeros(3, dtype=torch.float32, device="cuda")
    o2 = torch.zeros(3, dtype=torch.float32, device="cuda")
    old2 = (1.0, -5.0, 5.0)
    call(lib, "red_sum_max_min_f32_noalloc", x2[:8], (0.0, 0.0, 0.0), False)  # set-up
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        h = torch.cuda.current_stream().cuda_stream
        rc1 = lib.red_sum_max_min_f32_noalloc(x1.data_ptr(), n1, o1.data_ptr(), 0, h)
        rc2 = lib.red_sum_max_min_f32_noalloc(x2.data_ptr(), n2, o2.data_ptr(), 1, h)
    assert rc1 == RED_OK and rc2 == RED_OK, (rc1, rc2)
    torch.cuda.synchronize()
    eager_stream = torch.cuda.Stream()
    for rep in range(4):
        a = workloads.uniform_f32(610 + rep, n1, -2.0, 2.0)
        b = workloads.uniform_f32(620 + rep, n2, -2.0, 2.0)
        x1.copy_(torch.from_numpy(a))
        x2.copy_(torch.from_numpy(b))
        o2.copy_(torch.tensor(old2, dtype=torch.float32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(eager_stream):
            w1 = call(lib, "red_sum_max_min_f32", x1, (0.0, 0.0, 0.0), False)
            w2 = call(lib, "red_sum_max_min_f32", x2, old2, True)
        g1, g2 = host(o1), host(o2)
        assert g1.tobytes() == w1.tobytes(), ("replay", rep, g1, w1)
        assert g2.tobytes() == w2.tobytes(), ("replay", rep, g2, w2)
        check_oracle(a, g1, False, (0.0, 0.0, 0.0), "noalloc graph replay %d" % rep)
        check_oracle(b, g2, True, old2, "noalloc graph replay %d accum" % rep)
