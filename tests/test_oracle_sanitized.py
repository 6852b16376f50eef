"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle.c is rebuilt with gcc's ASan and UBSan (no recovery: the first
report aborts) into a temporary directory, and every pin is run against
that build in a child Python process that preloads the ASan runtime.  A
stray read past a row or tile, a signed overflow in an integer product or a
misaligned access in the oracle fails the test even where the pins' values
would not notice it.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))

SAN_FLAGS = ["-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
             "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import PINS
o = oracle.Oracle({lib!r})
for pin in PINS:
    pin(o)
print("pins passed:", len(PINS))
"""


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's ASan runtime is not installed")
    lib = os.path.join(str(tmp_path), "liboracle_san.so")
    res = subprocess.run(["gcc", *SAN_FLAGS, oracle.SOURCE, "-o", lib, "-lm"],
                         capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("gcc cannot build with the sanitizers here: " + res.stderr[-300:])
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    # CPython itself is not built for leak checking; memory errors and UB
    # still abort the child.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = CHILD.format(root=ROOT, tests=TESTS, lib=lib)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          env=env, timeout=600)
    assert proc.returncode == 0, proc.stdout[-2000:] + proc.stderr[-4000:]
    assert "pins passed" in proc.stdout
