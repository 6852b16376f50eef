"""Build libreduce.so for gfx950 with hipcc, in-tree.

    python fp32_reductions_amd/build.py

(Run it as a file, or load it by path: importing the package would first
load the library being rebuilt.)

Each translation unit under csrc/ compiles to an object in csrc/_build/
(in parallel), and the objects link into fp32_reductions_amd/libreduce.so.
The library is rebuilt on every call.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(CSRC, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libreduce.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "reduce1d.hip", "rows.hip", "colprod.hip"]
# Measurement only (the benchmark's read-only streaming ceiling): a library
# of its own.
CALIB_SOURCES = ["calib_read.hip"]
CALIB_LIBRARY = os.path.join(PKG, "libreduce_calib.so")

ARCH = "gfx950"
HIPFLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Keep subnormals (no flush to zero) and strict IEEE arithmetic.
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off",
    # Packed fp32 VALU forms are disabled: plain v_add / v_mul / v_max3 are
    # used throughout (the kernels are HBM-bound with VALU to spare).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Let float atomicAdd lower to the hardware global_atomic_add_f32.
    "-munsafe-fp-atomics",
    # Preload the first kernel arguments into SGPRs at wave launch (gfx940+
    # kernarg preload), so a kernel's first loads need not wait for a
    # kernel-argument fetch.  The code object keeps the compatible prologue
    # that fetches them itself where the firmware does not preload.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I" + INCLUDE,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s"
                           % (src, " ".join(cmd), res.stdout + res.stderr))
    return obj


def _link(objs, library: str) -> None:
    tmp = library + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd),
                                                     res.stdout + res.stderr))
    os.replace(tmp, library)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950; link libreduce.so and the
    measurement library libreduce_calib.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with concurrent.futures.ThreadPoolExecutor(len(srcs)) as pool:
        objs = dict(zip(srcs, pool.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIBRARY)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIBRARY)
    if verbose:
        print("built", LIBRARY, "and", CALIB_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
