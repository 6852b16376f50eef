"""Benchmark of libreduce on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant twopass|fused|atomic] [--cpu-seconds S]
                    [--no-configs]

Prints ONE JSON line on stdout.  A step is one pass of the workload's calls
over its input.  The default workload is ``vec1g``: one fp32 vector of
2^30 + 7 elements (normal(0,1), 1 % of the entries scaled by 1e6, seed 3)
reduced by sum, max and min.  ``value`` is whole-step effective bandwidth:
algorithmic bytes of all calls in a step divided by the wall time per step,
with every input already resident in HBM.

``per_config`` (default run only; --no-configs skips it) times the other
workloads in the same process, after the headline's timed region, with an
event pair around every call: the 4096 x 32 rows and 16 x 16 tile
(``rows32``, latency only), the 2^24 vector with and without accum
(``vec16m``), the 4096 x 16384 fp32 / int32 column products
(``colprod4k``), and the 65536 x 1000 row sum / max with the
2048 x 32768 bf16 / fp16 column products (``rows1000``).  Each call reports
microseconds per call, GB/s, the fraction of the 8 TB/s peak and, when a
counter summary for that call and source is committed, its HBM traffic.
``read_ceiling`` gives the same figures for a read-only streaming kernel
(the 1-D stream kernel with its reduction replaced by a trivial sink) over
the 2^30 + 7 and the 2^24 vectors, and over 128 MiB and 256 MiB, the byte
counts of the 16-bit and the fp32 tiles.  A call whose byte count is within
3 % of a ceiling's also reports its rate over that ceiling
(``of_read_ceiling``).

Cold cache: MI355X's 256 MB Infinity Cache would hold a 64 MiB vector
between calls, so a small input exists as several identical copies in HBM
and consecutive calls read different copies, which puts at least 1 GiB of
other traffic between two reads of the same copy.  No flush runs in the
timed region.

``roofline`` covers the dominant kernel: its algorithmic bytes per launch
over its mean launch duration, measured with HIP events recorded on the
launch stream around every launch inside the timed region.  ``traffic`` is
the HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE,
WRITE_SIZE, scaled against a plain copy kernel), read from the committed
counter summary under profiles/, or null when that summary was taken on a
different kernel or host-planning source.

``cpu_baseline`` times the CPU oracle on whole steps of the headline
workload: on T host threads (T = the CPU share of this process: its
affinity, capped by OMP_NUM_THREADS) with the oracle's threaded forms, and
single-threaded as written, about ``--cpu-seconds`` each, as a reference
point only.

Other workloads (--workload): vec16m, vec16m_fused (sum / max / min from
one read per call), vec16m_atomic (the vec16m step through the single-pass
atomic variant), vec1g_fused and vec1g_atomic (the same for the 2^30 + 7
vector), colprod4k, rows1000, rows32, colprod_int (int16 and uint32 column
products), cols4k (column sum / max / min of a 4096 x 16384 tile), copycal
(a plain device copy, for counter calibration).  --variant fused / atomic
selects the <workload>_fused / <workload>_atomic form of vec1g or vec16m.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "effective HBM GB/s (% of peak) for fp32 vector sum/max/min and colprod"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s
COLD_BYTES = 1 << 30   # other traffic between two reads of the same copy
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "fp32_reductions_amd", "csrc")
DEVICE_HEADERS = ["device.hpp", "../../include/reduce_device.hpp"]
# Host-side planning (grids, row splits, workgroups per CU): a change here
# changes what the kernels read, so it also invalidates counter summaries.
HOST_PLANNING = ["api.hip", "internal.hpp"]
SOURCES_1D = ["reduce1d.hip"] + DEVICE_HEADERS + HOST_PLANNING
SOURCES_ROWS = ["rows.hip"] + DEVICE_HEADERS + HOST_PLANNING
SOURCES_COLS = ["colprod.hip"] + DEVICE_HEADERS + HOST_PLANNING
SOURCES_ROWS_COLS = SOURCES_ROWS + ["colprod.hip"]  # row calls and column products


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


class HipEvents:
    """Timing-only HIP events recorded on the launch stream.

    Created with hipEventDisableSystemFence: recording such an event skips
    the system-scope cache writeback / invalidate a default event performs
    (on MI355X a default event pair added ~7 us to every 16 us launch).  The
    events come from the HIP runtime already loaded in the process (the one
    torch and libreduce share), and are read only after a device-wide
    synchronize."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        hip = ctypes.CDLL(path or "libamdhip64.so")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                            ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip = hip
        self.record_fn = hip.hipEventRecord

    def create(self) -> int:
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev: int) -> None:
        self.hip.hipEventDestroy(ev)


class Call:
    """One library call in a step: make(step_index) returns a pre-marshalled
    plan (fp32_reductions_amd.plan) that enqueues it when called."""

    def __init__(self, name, kernel, nbytes, make):
        self.name, self.kernel, self.nbytes, self.make = name, kernel, nbytes, make


class Workload:
    def __init__(self, name, desc, config, calls, dominant, sources, cpu,
                 device_inputs=()):
        self.name = name
        self.device_inputs = list(device_inputs)  # the workload's input tensors
        self.desc = desc
        self.config = config      # extra config keys
        self.calls = calls
        self.dominant = dominant  # call names timed for the roofline
        self.sources = sources    # csrc files that define the kernels and their grids
        # CPU oracle calls of one step: (bytes, single-threaded callable,
        # callable taking a thread count, or None when no threaded form exists)
        self.cpu = cpu


class Rotor:
    """Identical copies of one device tensor, handed out round-robin.

    With ``uses`` reads of the tensor per step and ``step_bytes`` read by the
    whole step, enough copies are made that at least COLD_BYTES of other
    reads separate two reads of the same copy.  A tensor of COLD_BYTES or
    more needs no copies."""

    def __init__(self, t, uses: int, step_bytes: int):
        nbytes = t.numel() * t.element_size()
        if nbytes >= COLD_BYTES:
            count = 1
        else:
            count = max(2, -(-uses * COLD_BYTES // step_bytes) + 1)
        self.copies = [t] + [t.clone() for _ in range(count - 1)]
        self.i = 0

    def next(self):
        t = self.copies[self.i]
        self.i = (self.i + 1) % len(self.copies)
        return t

    def __len__(self):
        return len(self.copies)


# The column kernel (one 256-byte column block per 512-thread workgroup at
# these shapes); a second kernel runs only when the plan splits the rows.
COLRED = "colred_kernel<{0}, true, 32, 512> (+ colred_finish_kernel<{0}> if rows are split)"


def up(torch, a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def vector_cpu(orc, x, accums):
    """Oracle calls of a 1-D step: sum, max, min for each accum setting
    (destination preset 3.25 under accum), single-threaded and threaded."""
    n = x.size
    cpu = []
    for accum in accums:
        nbytes = 4 * n + (8 if accum else 4)
        cpu += [(nbytes, lambda a=accum: orc.sum_f32(x, a, 3.25),
                 lambda t, a=accum: orc.sum_f32_mt(x, t, a, 3.25)),
                (nbytes, lambda a=accum: orc.max_f32(x, a, 3.25),
                 lambda t, a=accum: orc.max_f32_mt(x, t, a, 3.25)),
                (nbytes, lambda a=accum: orc.min_f32(x, a, 3.25),
                 lambda t, a=accum: orc.min_f32_mt(x, t, a, 3.25))]
    return cpu


def wl_vec16m(torch, red, orc, steps):
    x = workloads.vec16m()
    n = x.size
    xs = Rotor(up(torch, x), 6, 6 * 4 * n)
    outs = torch.zeros((steps, 3), dtype=torch.float32, device="cuda")
    accs = torch.full((steps, 3), workloads.ACCUM_PRESET, dtype=torch.float32,
                      device="cuda")
    calls = []
    for j, op in enumerate(("sum", "max", "min")):
        def plain(k, op=op, j=j):
            return red.plan(op + "_f32", xs.next(), outs[k, j:j + 1])

        def accum(k, op=op, j=j):
            return red.plan(op + "_f32", xs.next(), accs[k, j:j + 1], accum=True)

        kern = "reduce1d_stream_kernel<Op{0}, false> + reduce1d_finish_kernel<Op{0}>".format(
            op.capitalize())
        calls.append(Call(op, kern, 4 * n + 4, plain))
        calls.append(Call(op + "_accum", kern, 4 * n + 8, accum))
    calls = [calls[0], calls[2], calls[4], calls[1], calls[3], calls[5]]
    cpu = vector_cpu(orc, x, (False, True))
    return Workload(
        "vec16m",
        "one fp32 vector of 2^24 elements, uniform[-1,1), seed 1; sum, max, min, "
        "then sum, max, min with accum into a destination preset to 3.25",
        {"n": n, "calls_per_step": 6, "cold_copies": len(xs)},
        calls, ["sum"], SOURCES_1D, cpu)


def wl_vec16m_atomic(torch, red, orc, steps):
    """The vec16m step through the single-pass atomic variant."""
    x = workloads.vec16m()
    n = x.size
    xs = Rotor(up(torch, x), 6, 6 * 4 * n)
    outs = torch.zeros((steps, 3), dtype=torch.float32, device="cuda")
    accs = torch.full((steps, 3), workloads.ACCUM_PRESET, dtype=torch.float32,
                      device="cuda")
    calls = []
    for j, op in enumerate(("sum", "max", "min")):
        def plain(k, op=op, j=j):
            return red.plan(op + "_f32_atomic", xs.next(), outs[k, j:j + 1])

        def accum(k, op=op, j=j):
            return red.plan(op + "_f32_atomic", xs.next(), accs[k, j:j + 1], accum=True)

        kern = "reduce1d_atomic_kernel<Op{0}, false>".format(op.capitalize())
        calls.append(Call(op, "fill_u32_kernel + " + kern, 4 * n + 4, plain))
        calls.append(Call(op + "_accum", kern, 4 * n + 8, accum))
    calls = [calls[0], calls[2], calls[4], calls[1], calls[3], calls[5]]
    cpu = vector_cpu(orc, x, (False, True))
    return Workload(
        "vec16m_atomic",
        "one fp32 vector of 2^24 elements, uniform[-1,1), seed 1; sum, max, min, "
        "then with accum into a destination preset to 3.25, each as one pass "
        "with one device-scope atomic per workgroup",
        {"n": n, "calls_per_step": 6, "cold_copies": len(xs)},
        calls, ["sum_accum"], SOURCES_1D, cpu)


def wl_vec16m_fused(torch, red, orc, steps):
    x = workloads.vec16m()
    n = x.size
    xs = Rotor(up(torch, x), 2, 2 * 4 * n)
    outs = torch.zeros((steps, 3), dtype=torch.float32, device="cuda")
    accs = torch.full((steps, 3), workloads.ACCUM_PRESET, dtype=torch.float32,
                      device="cuda")
    kern = "reduce1d_summaxmin_stream_kernel<false> + reduce1d_summaxmin_finish_kernel"
    calls = [Call("sum_max_min", kern, 4 * n + 12,
                  lambda k: red.plan("sum_max_min_f32", xs.next(), outs[k])),
             Call("sum_max_min_accum", kern, 4 * n + 24,
                  lambda k: red.plan("sum_max_min_f32", xs.next(), accs[k], accum=True))]

    def oracle_all(accum, t=None):
        if t is None:
            return (orc.sum_f32(x, accum, 3.25), orc.max_f32(x, accum, 3.25),
                    orc.min_f32(x, accum, 3.25))
        return (orc.sum_f32_mt(x, t, accum, 3.25), orc.max_f32_mt(x, t, accum, 3.25),
                orc.min_f32_mt(x, t, accum, 3.25))
    cpu = [(4 * n + 12, lambda: oracle_all(False), lambda t: oracle_all(False, t)),
           (4 * n + 24, lambda: oracle_all(True), lambda t: oracle_all(True, t))]
    return Workload(
        "vec16m_fused",
        "one fp32 vector of 2^24 elements, uniform[-1,1), seed 1; sum, max and min "
        "from one read (fused call), then again with accum into destinations preset "
        "to 3.25",
        {"n": n, "calls_per_step": 2, "cold_copies": len(xs)},
        calls, ["sum_max_min"], SOURCES_1D, cpu)


def wl_vec1g(torch, red, orc, steps):
    log("generating 2^30+7 vector")
    x = workloads.vec1g()
    n = x.size
    xd = up(torch, x)
    outs = torch.zeros((steps, 3), dtype=torch.float32, device="cuda")
    calls = []
    for j, op in enumerate(("sum", "max", "min")):
        kern = ("reduce1d_stream_kernel<Op{0}, true> (+ reduce1d_finish_kernel<Op{0}>, one "
                "workgroup)".format(op.capitalize()))
        calls.append(Call(op, kern, 4 * n + 4,
                          lambda k, op=op, j=j: red.plan(op + "_f32", xd, outs[k, j:j + 1])))
    cpu = vector_cpu(orc, x, (False,))
    return Workload(
        "vec1g",
        "one fp32 vector of 2^30+7 elements, normal(0,1) with 1% of entries "
        "scaled by 1e6, seed 3; sum, max, min",
        {"n": n, "calls_per_step": 3, "cold_copies": 1},
        calls, ["sum"], SOURCES_1D, cpu, device_inputs=[xd])


def wl_vec1g_fused(torch, red, orc, steps):
    """The vec1g step as one fused call: sum, max and min from one read."""
    log("generating 2^30+7 vector")
    x = workloads.vec1g()
    n = x.size
    xd = up(torch, x)
    outs = torch.zeros((steps, 3), dtype=torch.float32, device="cuda")
    kern = "reduce1d_summaxmin_stream_kernel<true> + reduce1d_summaxmin_finish_kernel"
    calls = [Call("sum_max_min", kern, 4 * n + 12,
                  lambda k: red.plan("sum_max_min_f32", xd, outs[k]))]

    def oracle_all(t=None):
        if t is None:
            return orc.sum_f32(x), orc.max_f32(x), orc.min_f32(x)
        return orc.sum_f32_mt(x, t), orc.max_f32_mt(x, t), orc.min_f32_mt(x, t)
    cpu = [(4 * n + 12, lambda: oracle_all(), lambda t: oracle_all(t))]
    return Workload(
        "vec1g_fused",
        "one fp32 vector of 2^30+7 elements, normal(0,1) with 1% of entries "
        "scaled by 1e6, seed 3; sum, max and min from one read (fused call)",
        {"n": n, "calls_per_step": 1, "cold_copies": 1},
        calls, ["sum_max_min"], SOURCES_1D, cpu, device_inputs=[xd])


def wl_vec1g_atomic(torch, red, orc, steps):
    """The vec1g step through the single-pass atomic variant."""
    log("generating 2^30+7 vector")
    x = workloads.vec1g()
    n = x.size
    xd = up(torch, x)
    outs = torch.zeros((steps, 3), dtype=torch.float32, device="cuda")
    calls = []
    for j, op in enumerate(("sum", "max", "min")):
        kern = "fill_u32_kernel + reduce1d_atomic_kernel<Op{0}, true>".format(op.capitalize())
        calls.append(Call(op, kern, 4 * n + 4,
                          lambda k, op=op, j=j: red.plan(op + "_f32_atomic", xd,
                                                         outs[k, j:j + 1])))
    cpu = vector_cpu(orc, x, (False,))
    return Workload(
        "vec1g_atomic",
        "one fp32 vector of 2^30+7 elements, normal(0,1) with 1% of entries "
        "scaled by 1e6, seed 3; sum, max, min, each as one pass with one "
        "device-scope atomic per workgroup",
        {"n": n, "calls_per_step": 3, "cold_copies": 1},
        calls, ["sum"], SOURCES_1D, cpu, device_inputs=[xd])


def wl_colprod4k(torch, red, orc, steps):
    log("generating 4096 x 16384 f32 / i32 tiles")
    f, i = workloads.colprod4k_f32_i32()
    R, C = f.shape
    nbytes = 4 * R * C + 4 * C
    fs = Rotor(up(torch, f), 1, 2 * nbytes)
    is_ = Rotor(up(torch, i), 1, 2 * nbytes)
    of = torch.zeros(C, dtype=torch.float32, device="cuda")
    oi = torch.zeros(C, dtype=torch.int32, device="cuda")
    calls = [Call("colprod_f32", COLRED.format("TraitsF32, OpMul<float>"), nbytes,
                  lambda k: red.plan("colprod_f32", fs.next(), of)),
             Call("colprod_i32", COLRED.format("TraitsI32, OpMul<unsigned int>"), nbytes,
                  lambda k: red.plan("colprod_i32", is_.next(), oi))]
    cpu = [(nbytes, lambda: orc.colprod_f32(f, R, C, C),
            lambda t: orc.colprod_f32_mt(f, R, C, C, t)),
           (nbytes, lambda: orc.colprod_i32(i, R, C, C),
            lambda t: orc.colprod_i32_mt(i, R, C, C, t))]
    return Workload(
        "colprod4k",
        "column products of a 4096 x 16384 fp32 tile, uniform[0.999,1.001), and "
        "an int32 tile of the same shape, values in {-3..3}\\{0}, seed 2",
        {"R": R, "C": C, "calls_per_step": 2, "cold_copies": len(fs)},
        calls, ["colprod_f32"], SOURCES_COLS, cpu)


def wl_colprod_int(torch, red, orc, steps):
    """The other integer element types at the large tile shapes (odd values
    from {-3, -1, 1, 3}, whose products do not vanish)."""
    log("generating int16 2048 x 32768 and uint32 4096 x 16384 tiles")
    h = workloads.odd_i32_tile(2048, 32768, seed=51).astype(np.int16)
    u = workloads.odd_i32_tile(4096, 16384, seed=52)  # int32 bits of uint32 values
    hb = 2 * h.size + 2 * h.shape[1]
    ub = 4 * u.size + 4 * u.shape[1]
    hs = Rotor(up(torch, h), 1, hb + ub)
    us = Rotor(up(torch, u), 1, hb + ub)
    oh = torch.zeros(h.shape[1], dtype=torch.int16, device="cuda")
    ou = torch.zeros(u.shape[1], dtype=torch.int32, device="cuda")
    calls = [Call("colprod_i16", COLRED.format("TraitsU16, OpMul<unsigned int>"), hb,
                  lambda k: red.plan("colprod_i16", hs.next(), oh)),
             Call("colprod_u32", COLRED.format("TraitsI32, OpMul<unsigned int>"), ub,
                  lambda k: red.plan("colprod_u32", us.next(), ou))]
    cpu = [(hb, lambda: orc.colprod_u16(h.view(np.uint16), 2048, 32768, 32768), None),
           (ub, lambda: orc.colprod_u32(u.view(np.uint32), 4096, 16384, 16384), None)]
    return Workload(
        "colprod_int",
        "column products of a 2048 x 32768 int16 tile and a 4096 x 16384 uint32 tile, "
        "values uniform over {-3, -1, 1, 3} (seeds 51, 52)",
        {"calls_per_step": 2, "cold_copies": [len(hs), len(us)]},
        calls, ["colprod_i16"], SOURCES_COLS, cpu)


def wl_rows1000(torch, red, orc, steps):
    log("generating 65536 x 1000 rows and 2048 x 32768 bf16 / f16 tiles")
    x, b, h = workloads.rows1000()
    rows, n = x.shape
    R, C = b.shape
    rbytes = 4 * rows * n + 4 * rows
    tbytes = 2 * R * C + 2 * C
    step = 2 * rbytes + 2 * tbytes
    xs = Rotor(up(torch, x), 2, step)
    bs = Rotor(up(torch, b).view(torch.bfloat16), 1, step)
    hs = Rotor(up(torch, h).view(torch.float16), 1, step)
    o1 = torch.zeros(rows, dtype=torch.float32, device="cuda")
    o2 = torch.zeros(rows, dtype=torch.float32, device="cuda")
    ob = torch.zeros(C, dtype=torch.bfloat16, device="cuda")
    oh = torch.zeros(C, dtype=torch.float16, device="cuda")
    calls = [Call("rows_sum", "rows_seg_kernel<OpSum, 64, 4, 2>", rbytes,
                  lambda k: red.plan("sum_rows_f32", xs.next(), o1)),
             Call("rows_max", "rows_seg_kernel<OpMax, 64, 4, 2>", rbytes,
                  lambda k: red.plan("max_rows_f32", xs.next(), o2)),
             Call("colprod_bf16", COLRED.format("TraitsBF16, OpMul<float>"), tbytes,
                  lambda k: red.plan("colprod_bf16", bs.next(), ob)),
             Call("colprod_f16", COLRED.format("TraitsF16, OpMul<float>"), tbytes,
                  lambda k: red.plan("colprod_f16", hs.next(), oh))]
    cpu = [(rbytes, lambda: orc.rows_sum_f32(x, rows, n, n),
            lambda t: orc.rows_sum_f32_mt(x, rows, n, n, t)),
           (rbytes, lambda: orc.rows_max_f32(x, rows, n, n),
            lambda t: orc.rows_max_f32_mt(x, rows, n, n, t)),
           (tbytes, lambda: orc.colprod_bf16(b, R, C, C),
            lambda t: orc.colprod_bf16_mt(b, R, C, C, t)),
           (tbytes, lambda: orc.colprod_f16(h, R, C, C),
            lambda t: orc.colprod_f16_mt(h, R, C, C, t))]
    return Workload(
        "rows1000",
        "65536 rows x 1000 fp32, uniform[-1,1), row sum and row max; then column "
        "products of 2048 x 32768 bf16 and f16 tiles, uniform[0.99,1.01), seed 4",
        {"rows": rows, "n": n, "R": R, "C": C, "calls_per_step": 4,
         "cold_copies": [len(xs), len(bs), len(hs)]},
        calls, ["rows_sum"], SOURCES_ROWS_COLS, cpu)


def wl_cols4k(torch, red, orc, steps):
    log("generating a 4096 x 16384 fp32 tile")
    t = workloads.uniform_f32(60, (4096, 16384))
    R, C = t.shape
    nbytes = 4 * R * C + 4 * C
    ts = Rotor(up(torch, t), 3, 3 * nbytes)
    outs = [torch.zeros(C, dtype=torch.float32, device="cuda") for _ in range(3)]
    calls = [Call(op + "_cols", COLRED.format("TraitsF32, Op%s" % op.capitalize()),
                  nbytes, lambda k, op=op, j=j: red.plan(op + "_cols_f32", ts.next(), outs[j]))
             for j, op in enumerate(("sum", "max", "min"))]
    cpu = [(nbytes, lambda: orc.cols_sum_f32(t, R, C, C), None),
           (nbytes, lambda: orc.cols_max_f32(t, R, C, C), None),
           (nbytes, lambda: orc.cols_min_f32(t, R, C, C), None)]
    return Workload(
        "cols4k",
        "column sum, max and min of a 4096 x 16384 fp32 tile, uniform[-1,1), seed 60",
        {"R": R, "C": C, "calls_per_step": 3, "cold_copies": len(ts)},
        calls, ["sum_cols"], SOURCES_COLS, cpu)


def wl_rows32(torch, red, orc, steps):
    a, t = workloads.rows32()
    rows, n = a.shape
    ad, td = up(torch, a), up(torch, t)
    o = [torch.zeros(rows, dtype=torch.float32, device="cuda") for _ in range(3)]
    ot = torch.zeros(16, dtype=torch.float32, device="cuda")
    rbytes = 4 * rows * n + 4 * rows
    calls = [Call("rows_sum", "rows_tile_kernel<OpSum>", rbytes,
                  lambda k: red.plan("sum_rows_f32", ad, o[0])),
             Call("rows_max", "rows_tile_kernel<OpMax>", rbytes,
                  lambda k: red.plan("max_rows_f32", ad, o[1])),
             Call("rows_min", "rows_tile_kernel<OpMin>", rbytes,
                  lambda k: red.plan("min_rows_f32", ad, o[2])),
             Call("colprod_tile16", "colred_narrow_kernel<TraitsF32, OpMul<float>>", 16 * 16 * 4 + 64,
                  lambda k: red.plan("colprod_f32", td, ot))]
    cpu = [(rbytes, lambda: orc.rows_page_sum_f32(a, rows, n, n), None),
           (rbytes, lambda: orc.rows_max_f32(a, rows, n, n), None),
           (rbytes, lambda: orc.rows_min_f32(a, rows, n, n), None),
           (16 * 16 * 4 + 64, lambda: orc.colprod_f32(t, 16, 16, 16), None)]
    return Workload(
        "rows32",
        "4096 rows x 32 fp32, uniform[-1,1), seed 0: row sum, max, min (one "
        "thread per row, rows staged in LDS); one 16 x 16 fp32 tile column product",
        {"rows": rows, "n": n, "calls_per_step": 4, "cold_copies": 1},
        calls, ["rows_sum"], SOURCES_ROWS_COLS, cpu)


def wl_copycal(torch, red, orc, steps):
    """A plain elementwise copy of known size (256 MiB read, 256 MiB
    written) for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 26
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    calls = [Call("copy", "elementwise copy", 8 * n,
                  lambda k: (lambda: torch.neg(src, out=dst)))]
    return Workload("copycal", "plain device copy of 2^26 fp32 (256 MiB in, 256 MiB out)",
                    {"n": n, "calls_per_step": 1, "cold_copies": 1},
                    calls, ["copy"], [], [])


WORKLOADS = {"vec16m": wl_vec16m, "vec16m_fused": wl_vec16m_fused, "vec16m_atomic": wl_vec16m_atomic, "vec1g": wl_vec1g,
             "vec1g_fused": wl_vec1g_fused, "vec1g_atomic": wl_vec1g_atomic, "colprod4k": wl_colprod4k,
             "rows1000": wl_rows1000, "colprod_int": wl_colprod_int, "cols4k": wl_cols4k, "rows32": wl_rows32, "copycal": wl_copycal}


# ---------------------------------------------------------------------------
# counters committed under profiles/
# ---------------------------------------------------------------------------

def _code_only(text: str) -> str:
    """The source without comments and blank space, so that a change to a
    comment alone does not mark the counters as taken on other code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(files, csrc: str = CSRC) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(wl: Workload, call: str, profiles: str = PROFILES,
                      csrc: str = CSRC):
    """HBM bytes per launch of `call` from the committed counter summary
    profiles/<call>_<workload>_counters.txt, or None if it is absent or was
    taken on different kernel or planning source."""
    path = os.path.join(profiles, "%s_%s_counters.txt" % (call, wl.name))
    if not wl.sources or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_hash(wl.sources, csrc):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def time_calls(hev, stream_handle, plans, calls, first, count):
    """An event pair around every call of steps first .. first + count - 1;
    returns {call name: [durations in ms]}."""
    import torch
    record = hev.record_fn
    evs = [[(hev.create(), hev.create()) for _ in calls] for _ in range(count)]
    torch.cuda.synchronize()
    for k in range(count):
        for j, p in enumerate(plans[first + k]):
            record(evs[k][j][0], stream_handle)
            p()
            record(evs[k][j][1], stream_handle)
    torch.cuda.synchronize()
    durs = {c.name: [hev.elapsed_ms(*evs[k][j]) for k in range(count)]
            for j, c in enumerate(calls)}
    for row in evs:
        for a, b in row:
            hev.destroy(a)
            hev.destroy(b)
    return durs


def call_entry(call, durs, traffic=None):
    mean_ms = float(np.mean(durs))
    gbs = call.nbytes / (mean_ms * 1e-3) / 1e9
    entry = {"kernel": call.kernel, "bytes": call.nbytes,
             "mean_us": round(1e3 * mean_ms, 3),
             "median_us": round(1e3 * float(np.median(durs)), 3),
             "gbs_mean": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if traffic is not None:
        entry["traffic"] = traffic
        entry["traffic_over_algorithmic"] = round(traffic / call.nbytes, 4)
    return entry


def against_ceiling(entry, ceiling, within=0.03):
    """Add to a per-call entry its rate over the read-only ceiling measured
    on the same byte count (to within `within`), when there is one: how
    close the call comes to a plain read of its bytes with the same launch
    style."""
    best = None
    for label, c in ceiling.items():
        rel = abs(c["bytes"] - entry["bytes"]) / entry["bytes"]
        if rel <= within and (best is None or rel < best[0]):
            best = (rel, label, c)
    if best is not None:
        entry["read_ceiling"] = best[1]
        entry["of_read_ceiling"] = round(entry["gbs_mean"] / best[2]["gbs_mean"], 4)
    return entry


def measure_workload(torch, red, orc, name, steps, warmup, hev, stream_handle):
    """Per-call event timings of one workload (for per_config)."""
    wl = WORKLOADS[name](torch, red, orc, steps + warmup)
    plans = [[c.make(k) for c in wl.calls] for k in range(steps + warmup)]
    for k in range(warmup):
        for p in plans[k]:
            p()
    torch.cuda.synchronize()
    durs = time_calls(hev, stream_handle, plans, wl.calls, warmup, steps)
    out = {"workload": "%s: %s" % (wl.name, wl.desc),
           "calls": {c.name: call_entry(c, durs[c.name], committed_traffic(wl, c.name))
                     for c in wl.calls}}
    del plans, wl
    return out


def read_ceiling(torch, hev, stream_handle, x_dev, copies, steps, warmup, cus):
    """Event-timed read-only streaming kernel (libreduce_calib.so) over the
    device vector x_dev (and its extra cold copies)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "fp32_reductions_amd", "libreduce_calib.so"))
    lib.calib_read_grid.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    lib.calib_read_grid.restype = ctypes.c_int
    lib.calib_read_f32.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_uint, ctypes.c_int, ctypes.c_void_p]
    lib.calib_read_f32.restype = ctypes.c_int
    vecs = [x_dev] + list(copies)
    n = x_dev.numel()
    grid = max(lib.calib_read_grid(v.data_ptr(), n, cus) for v in vecs)
    sink = torch.zeros(grid * 512, dtype=torch.int32, device="cuda")
    match = 0x5EED1E55  # a thread stores its XOR only if it equals this

    def launch(k):
        v = vecs[k % len(vecs)]
        rc = lib.calib_read_f32(v.data_ptr(), n, sink.data_ptr(), match, cus, stream_handle)
        if rc != 0:
            raise RuntimeError("calib_read_f32: hipError %d" % rc)

    for k in range(warmup):
        launch(k)
    torch.cuda.synchronize()
    record = hev.record_fn
    evs = [(hev.create(), hev.create()) for _ in range(steps)]
    for k in range(steps):
        record(evs[k][0], stream_handle)
        launch(warmup + k)
        record(evs[k][1], stream_handle)
    torch.cuda.synchronize()
    durs = [hev.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hev.destroy(a)
        hev.destroy(b)
    mean_ms = float(np.mean(durs))
    gbs = 4 * n / (mean_ms * 1e-3) / 1e9
    return {"kernel": "read_sink_kernel (1-D stream kernel, XOR sink)", "bytes": 4 * n,
            "mean_us": round(1e3 * mean_ms, 3), "gbs_mean": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "cold_copies": len(vecs)}


# ---------------------------------------------------------------------------
# CPU baseline
# ---------------------------------------------------------------------------

def cpu_threads() -> int:
    """Host threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set (the per-job CPU share on a shared
    host)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _time_cpu(calls, budget_s):
    total_bytes, steps, t0 = 0, 0, time.perf_counter()
    while True:
        for nbytes, fn in calls:
            fn()
            total_bytes += nbytes
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return total_bytes / dt / 1e9, steps, dt


def cpu_baseline(wl: Workload, budget_s: float = 10.0):
    """The oracle on whole steps of the workload, threaded on cpu_threads()
    cores (reported as the baseline) and single-threaded (single_core)."""
    if not wl.cpu:
        return None
    v1, s1, d1 = _time_cpu([(b, f1) for b, f1, _ in wl.cpu], budget_s)
    single = {"value": round(v1, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "sample": "%d whole step(s) of the workload (all %d calls, same host "
                        "arrays), single-threaded C oracle, %.1f s" % (s1, len(wl.cpu), d1)}
    threads = cpu_threads()
    if threads == 1 or any(ft is None for _, _, ft in wl.cpu):
        return dict(single, single_core=None)
    vt, st, dt = _time_cpu([(b, (lambda f=ft: f(threads))) for b, _, ft in wl.cpu], budget_s)
    return {"value": round(vt, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole step(s) of the workload (all %d calls, same host arrays), "
                      "the C oracle's threaded form: %d contiguous pieces on %d threads, "
                      "combined in order, %.1f s" % (st, len(wl.cpu), threads, threads, dt),
            "single_core": single}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

# The other workloads timed after the headline (one per remaining input
# configuration, the smallest first).
PER_CONFIG = ["rows32", "vec16m", "colprod4k", "rows1000"]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="vec1g", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of each CPU-oracle baseline (0: skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per_config and read_ceiling blocks")
    ap.add_argument("--variant", default="twopass", choices=["twopass", "fused", "atomic"],
                    help="the 1-D calls of the workload: the deterministic two-kernel "
                         "calls (default), the fused sum+max+min call, or the single-pass "
                         "atomic variant")
    args = ap.parse_args(argv)
    name = args.workload
    if args.variant != "twopass":
        name = "%s_%s" % (args.workload, args.variant)
        if name not in WORKLOADS:
            print("workload %s has no %s variant (variants exist for: %s)" % (
                args.workload, args.variant,
                ", ".join(sorted(w.rsplit("_", 1)[0] for w in WORKLOADS
                                 if w.endswith("_" + args.variant)))), file=sys.stderr)
            return 2

    if args.gpus != 1:
        print("bench.py measures one GPU only: multi-GPU runs are not part of "
              "this library (got --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import torch

    import fp32_reductions_amd as red
    import oracle

    orc = oracle.get()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    K, W = args.steps, args.warmup
    wl = WORKLOADS[name](torch, red, orc, K + W)
    stream = torch.cuda.current_stream()

    log("workload %s: %d calls/step, warmup %d, steps %d" % (wl.name, len(wl.calls), W, K))
    plans = [[call.make(k) for call in wl.calls] for k in range(W + K)]
    for k in range(W):
        for p in plans[k]:
            p()
    torch.cuda.synchronize()

    # Timed region: K steps.  Events bracket only the dominant call of each
    # step (recording an event pair between two kernels stalls the queue for
    # a few microseconds, so bracketing every call would slow the step).
    hev = HipEvents()
    sh = stream.cuda_stream
    record = hev.record_fn
    names = [call.name for call in wl.calls]
    dom_idx = [names.index(name) for name in wl.dominant]
    ev = {j: [(hev.create(), hev.create()) for _ in range(K)] for j in dom_idx}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        for j, p in enumerate(plans[W + k]):
            if j in ev:
                record(ev[j][k][0], sh)
                p()
                record(ev[j][k][1], sh)
            else:
                p()
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / K
    step_bytes = sum(call.nbytes for call in wl.calls)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom_durs = {j: [hev.elapsed_ms(a, b) for a, b in ev[j]] for j in dom_idx}
    for evs in ev.values():
        for a, b in evs:
            hev.destroy(a)
            hev.destroy(b)

    # Per-call breakdown (not part of the timed region): a short pass with an
    # event pair around every call.
    kb = min(K, 50)
    durs = time_calls(hev, sh, plans, wl.calls, W, kb)
    per_call = {c.name: call_entry(c, durs[c.name], committed_traffic(wl, c.name))
                for c in wl.calls}
    dom_bytes = float(np.mean([wl.calls[j].nbytes for j in dom_idx]))
    dom_us = 1e3 * float(np.mean([np.mean(dom_durs[j]) for j in dom_idx]))
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = committed_traffic(wl, wl.dominant[0])

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.name != "rows1000" else "f32,bf16,f16",
        "data": "synthetic",
        "config": dict({"workload": "%s: %s" % (wl.name, wl.desc)}, **wl.config),
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": wl.calls[dom_idx[0]].kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": dom_bytes, "mean_launch_us": round(dom_us, 3)},
        "per_call": per_call,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", None),
                   "hbm_gib": round(props.total_memory / 2**30, 1),
                   "hip": getattr(torch.version, "hip", None), "torch": torch.__version__},
    }
    del plans

    if name == "vec1g" and not args.no_configs:
        ks, ws = min(K, 30), min(W, 5)
        x_dev = wl.device_inputs[0]
        log("read-only ceiling over the 2^30 + 7 vector")
        ceiling = {"vec1g": read_ceiling(torch, hev, sh, x_dev, [], ks, ws,
                                         props.multi_processor_count)}
        n16 = workloads.N_VEC16M
        small = x_dev[:n16]
        copies = [small.clone() for _ in range(16)]
        log("read-only ceiling over 2^24 elements (17 cold copies)")
        ceiling["vec16m"] = read_ceiling(torch, hev, sh, small, copies, ks, ws,
                                         props.multi_processor_count)
        del copies
        # The sizes of the column and row tiles: 128 MiB (the 16-bit tiles)
        # and 256 MiB (the fp32 tiles and the 65536 x 1000 rows), each read
        # from disjoint slices of the long vector in turn so that no call
        # finds its bytes in the 256 MB last-level cache.
        for label, lg, nslices in (("128MiB", 25, 8), ("256MiB", 26, 4)):
            m = 1 << lg
            parts = [x_dev[k * m:(k + 1) * m] for k in range(nslices)]
            log("read-only ceiling over %s (%d disjoint slices)" % (label, nslices))
            ceiling[label] = read_ceiling(torch, hev, sh, parts[0], parts[1:], ks, ws,
                                          props.multi_processor_count)
        line["read_ceiling"] = ceiling
        per_config = {}
        for name in PER_CONFIG:
            log("per_config: %s" % name)
            per_config[name] = measure_workload(torch, red, orc, name, ks, ws, hev, sh)
            torch.cuda.empty_cache()
        for entry in per_call.values():
            against_ceiling(entry, ceiling)
        for cfg in per_config.values():
            for entry in cfg["calls"].values():
                against_ceiling(entry, ceiling)
        line["per_config"] = per_config

    if args.cpu_seconds > 0:
        log("timing the CPU oracle (~%.0f s per mode, %d threads)"
            % (args.cpu_seconds, cpu_threads()))
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
