"""Calls from several host threads at once: each thread on
hipStreamPerThread (one handle, a different stream in every thread), and
several threads sharing one stream.  Every result must equal the same call
made alone on one stream (the default entry points are deterministic) and
match the oracle: max / min bit for bit, sum within 1e-6 * sum |x|."""
import ctypes
import threading

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check_exact, check_sum, dev, has_both_zeros, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PER_THREAD_STREAM = 2  # hipStreamPerThread
OPS = ("sum", "max", "min")
THREADS = 4
ROUNDS = 25


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(scope="module")
def hip():
    """The HIP runtime the process already uses (torch's and libreduce's)."""
    path = None
    with open("/proc/self/maps") as fh:
        for line in fh:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    lib = ctypes.CDLL(path or "libamdhip64.so")
    lib.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipStreamSynchronize.restype = ctypes.c_int
    return lib


def inputs():
    """One vector per thread, of different lengths (so different grids) and
    values."""
    xs = []
    for t in range(THREADS):
        n = (1 << 21) + 7919 * t + 3
        xs.append(workloads.uniform_f32(500 + t, n, -1.0 - t, 1.0 + 2 * t))
    return xs


def reference(red, xd):
    """Each call alone on torch's current stream."""
    out = torch.zeros(len(OPS), dtype=torch.float32, device="cuda")
    for j, op in enumerate(OPS):
        getattr(red, op + "_f32")(xd, out[j:j + 1])
    return host(out)


def check_against_oracle(orc, x, got, what):
    s, a = orc.sum_f32(x)
    check_sum(got[0], s, a, what + " sum")
    both = bool(has_both_zeros(x))
    check_exact(got[1], orc.max_f32(x), what + " max", both)
    check_exact(got[2], orc.min_f32(x), what + " min", both)


def run_threads(target):
    errors = []

    def wrap(t):
        try:
            target(t)
        except BaseException as e:  # reported on the main thread
            errors.append((t, e))

    threads = [threading.Thread(target=wrap, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors


def test_threads_on_per_thread_stream(red, orc, hip):
    say("%d host threads, hipStreamPerThread, %d rounds of sum/max/min" % (THREADS, ROUNDS))
    xs = inputs()
    xds = [dev(x) for x in xs]
    refs = [reference(red, xd) for xd in xds]
    outs = [torch.zeros((ROUNDS, len(OPS)), dtype=torch.float32, device="cuda")
            for _ in range(THREADS)]
    torch.cuda.synchronize()
    released = [None] * THREADS

    def work(t):
        for k in range(ROUNDS):
            for j, op in enumerate(OPS):
                getattr(red, op + "_f32")(xds[t], outs[t][k, j:j + 1], stream=PER_THREAD_STREAM)
        assert hip.hipStreamSynchronize(PER_THREAD_STREAM) == 0
        red.release_workspace(PER_THREAD_STREAM)
        released[t] = True

    run_threads(work)
    assert all(released)
    for t in range(THREADS):
        got = host(outs[t])
        assert (got.view(np.uint32) == refs[t].view(np.uint32)).all(), \
            "thread %d: a result differs from the same call made alone" % t
        check_against_oracle(orc, xs[t], got[0], "thread %d" % t)


def test_threads_sharing_one_stream(red, orc):
    """Calls of several threads on one stream are ordered by it: each call's
    two kernels stay together, whatever the interleaving of the threads."""
    say("%d host threads sharing one stream" % THREADS)
    xs = inputs()
    xds = [dev(x) for x in xs]
    refs = [reference(red, xd) for xd in xds]
    outs = [torch.zeros((ROUNDS, len(OPS)), dtype=torch.float32, device="cuda")
            for _ in range(THREADS)]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    handle = stream.cuda_stream

    def work(t):
        for k in range(ROUNDS):
            for j, op in enumerate(OPS):
                getattr(red, op + "_f32")(xds[t], outs[t][k, j:j + 1], stream=handle)

    run_threads(work)
    stream.synchronize()
    for t in range(THREADS):
        got = host(outs[t])
        assert (got.view(np.uint32) == refs[t].view(np.uint32)).all(), \
            "thread %d: a result differs from the same call made alone" % t
        check_against_oracle(orc, xs[t], got[0], "shared stream, thread %d" % t)
    red.release_workspace(stream)


def test_release_then_reuse(red, orc):
    """After its workspace is released a stream allocates a new one on its
    next call; releasing a stream without a workspace does nothing."""
    say("release workspace, then call again")
    x = workloads.uniform_f32(510, (1 << 20) + 1)
    xd = dev(x)
    stream = torch.cuda.Stream()
    red.release_workspace(stream)            # nothing to free yet
    out = torch.zeros(3, dtype=torch.float32, device="cuda")
    for _ in range(2):
        with torch.cuda.stream(stream):
            for j, op in enumerate(OPS):
                getattr(red, op + "_f32")(xd, out[j:j + 1], stream=stream)
        red.release_workspace(stream)        # waits for the calls first
        check_against_oracle(orc, x, host(out), "after release")
