"""Helpers shared by the GPU parity tests: device upload, tolerance checks,
and flushed progress lines naming each case before it runs on the GPU."""
from __future__ import annotations

import math
import sys

import numpy as np

# Tolerances (fixed by the stated contract of each operation):
SUM_TOL = 1e-6          # |gpu - S| <= SUM_TOL * A, A = sum of |terms|
COLPROD_F32_TOL = 4e-4  # relative, R <= 4096 (any order is within (R-1)*2^-24)
COLPROD_16_TOL = 2e-2   # relative, f16 / bf16 with one final rounding


def say(msg: str) -> None:
    """Print and flush a line naming the case about to run on the GPU."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f32bits(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


def check_sum(got: float, s: float, a: float, what: str, tol: float = SUM_TOL):
    if math.isnan(s) or math.isinf(s):
        if math.isnan(s):
            assert math.isnan(got), (what, got, s)
        else:
            assert got == s, (what, got, s)
        return
    err = abs(float(got) - s)
    assert err <= tol * a, "%s: |%r - %r| = %g > %g * %g" % (what, float(got), s, err, tol, a)


def check_exact(got, want, what: str):
    """Bit-exact float equality, except that a zero may carry either sign
    when the extreme is a zero (either zero is a correct max / min)."""
    g, w = np.float32(got), np.float32(want)
    if math.isnan(w):
        assert math.isnan(g), (what, g, w)
        return
    if w == 0 and g == 0:
        return
    assert f32bits(g) == f32bits(w), (what, float(g), float(w))


def check_rel(got: np.ndarray, want: np.ndarray, tol: float, what: str):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    zero = want == 0
    assert (got[zero] == 0).all(), what
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, "%s: max relative error %g > %g" % (what, worst, tol)
    return worst
