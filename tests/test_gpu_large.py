"""Index arithmetic past 2^32 elements.

Each case allocates one operand of more than 2^32 elements (16 GiB for
fp32; an MI355X holds 288 GB), fills it with constants on the device,
plants a few distinct values near the far end, and checks results that
hold in closed form at any size: integer-valued sums that every
evaluation order gets within the tolerance (or exactly), the planted
extremes for max / min, and products of ones and powers of two, which are
exact in any order.  A kernel that truncated an index to 32 bits would
miss or misplace the planted values."""
import numpy as np
import pytest

from gpu_helpers import SUM_TOL, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BIG = (1 << 32) + 9  # elements of the 1-D case


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(autouse=True)
def release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def need(gib: float):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * 2**30 * 1.1:
        pytest.skip("needs %.0f GiB of free device memory" % gib)


def test_vector_past_2_32(red):
    need(16.2)
    say("1-D n=2^32+9: planted values past 2^32")
    x = torch.full((BIG,), 0.5, dtype=torch.float32, device="cuda")
    x[5] = 3.0
    x[(1 << 32) + 3] = -9.0
    x[BIG - 1] = 7.0
    s_exact = 0.5 * (BIG - 3) + 3.0 - 9.0 + 7.0
    a_exact = 0.5 * (BIG - 3) + 3.0 + 9.0 + 7.0
    out = torch.zeros(3, dtype=torch.float32, device="cuda")
    red.sum_f32(x, out[0:1])
    red.max_f32(x, out[1:2])
    red.min_f32(x, out[2:3])
    got = host(out)
    assert abs(float(got[0]) - s_exact) <= SUM_TOL * a_exact, (float(got[0]), s_exact)
    assert got[1] == 7.0 and got[2] == -9.0, got
    fused = torch.zeros(3, dtype=torch.float32, device="cuda")
    red.sum_max_min_f32(x, fused)
    assert (host(fused).view(np.uint32) == got.view(np.uint32)).all()
    del x


def test_rows_past_2_32(red):
    need(16.1)
    rows, n = (1 << 22) + 1, 1024
    say("rows %d x %d (2^32 + 1024 elements): last row planted" % (rows, n))
    x = torch.ones((rows, n), dtype=torch.float32, device="cuda")
    x[-1] = 2.0
    x[-1, 17] = 5.0
    out = torch.zeros(rows, dtype=torch.float32, device="cuda")
    red.sum_rows_f32(x, out)
    assert bool((out[:-1] == float(n)).all())
    assert float(out[-1]) == 2.0 * (n - 1) + 5.0
    red.max_rows_f32(x, out)
    assert bool((out[:-1] == 1.0).all()) and float(out[-1]) == 5.0
    del x


def test_short_rows_past_2_32(red):
    need(16.1)
    rows, n = (1 << 26) + 3, 64
    say("rows %d x %d (thread per row, 2^32 + 192 elements)" % (rows, n))
    x = torch.ones((rows, n), dtype=torch.float32, device="cuda")
    x[-1] = 0.25
    x[-2, 63] = -3.0
    out = torch.zeros(rows, dtype=torch.float32, device="cuda")
    red.sum_rows_f32(x, out)
    assert bool((out[:-2] == 64.0).all())
    assert float(out[-2]) == 63.0 - 3.0 and float(out[-1]) == 16.0
    red.min_rows_f32(x, out)
    assert bool((out[:-2] == 1.0).all())
    assert float(out[-2]) == -3.0 and float(out[-1]) == 0.25
    del x


def test_columns_past_2_32(red):
    need(16.1)
    R, C = 65537, 65536
    say("tile %d x %d f32 (2^32 + 65536 elements): colprod and column sum / min" % (R, C))
    t = torch.ones((R, C), dtype=torch.float32, device="cuda")
    t[-1] = 2.0
    t[-2, 7] = 0.5
    out = torch.zeros(C, dtype=torch.float32, device="cuda")
    red.colprod_f32(t, out)
    want = torch.full((C,), 2.0, device="cuda")
    want[7] = 1.0
    assert bool((out == want).all())
    red.sum_cols_f32(t, out)
    want = torch.full((C,), float(R - 2) + 1.0 + 2.0, device="cuda")
    want[7] = float(R - 2) + 0.5 + 2.0
    assert bool((out == want).all())
    red.min_cols_f32(t, out)
    want = torch.ones(C, device="cuda")
    want[7] = 0.5
    assert bool((out == want).all())
    del t


def test_int_columns_past_2_32(red):
    need(16.1)
    R, C = 65537, 65536
    say("tile %d x %d i32: products 3 and -3 from the last rows" % (R, C))
    t = torch.ones((R, C), dtype=torch.int32, device="cuda")
    t[-1] = 3
    t[-2, 7] = -1
    out = torch.zeros(C, dtype=torch.int32, device="cuda")
    red.colprod_i32(t, out)
    want = torch.full((C,), 3, dtype=torch.int32, device="cuda")
    want[7] = -3
    assert bool((out == want).all())
    del t


def test_bf16_columns_past_2_32(red):
    need(8.1)
    R, C = 65537, 65536
    say("tile %d x %d bf16: product 2 from the last row" % (R, C))
    t = torch.ones((R, C), dtype=torch.bfloat16, device="cuda")
    t[-1] = 2.0
    t[-3, C - 1] = 0.25
    out = torch.zeros(C, dtype=torch.bfloat16, device="cuda")
    red.colprod_bf16(t, out)
    want = torch.full((C,), 2.0, dtype=torch.bfloat16, device="cuda")
    want[C - 1] = 0.5
    assert bool((out == want).all())
    del t
