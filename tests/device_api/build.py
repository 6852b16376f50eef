"""Build the test kernels for include/reduce_device.hpp (test support).

    python tests/device_api/build.py

Compiles device_api_test.hip for gfx950 into libdevapitest.so beside it,
with the library's own code-generation flags.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBRARY = os.path.join(HERE, "libdevapitest.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "device_api_test.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), res.stdout + res.stderr))
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print("built", build())
    sys.exit(0)
