"""The seeded generators: chunked draws equal one monolithic draw, shapes,
dtypes, value ranges.  CPU only, small sizes."""
import numpy as np

import workloads


def test_chunked_equals_monolithic(monkeypatch):
    n = 10007
    rng = np.random.default_rng(3)
    xm = rng.standard_normal(n, dtype=np.float32)
    m = rng.random(n) < 0.01
    xm[m] *= np.float32(1e6)
    monkeypatch.setattr(workloads, "CHUNK", 1000)
    xc = workloads.vec1g(n)
    assert np.array_equal(xm.view(np.uint32), xc.view(np.uint32))
    rng = np.random.default_rng(7)
    um = rng.uniform(-1, 1, n).astype(np.float32)
    uc = workloads.uniform_f32(7, n)
    assert np.array_equal(um, uc)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5,
                  1.0 + 2**-8 + 2**-20], np.float32)
    b = workloads.to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6);
    # 1+2^-9 rounds down; just above a tie rounds up.
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x3F81]


def test_small_workload_shapes():
    a, t = workloads.rows32()
    assert a.shape == (4096, 32) and a.dtype == np.float32
    assert t.shape == (16, 16) and (t >= 0.5).all() and (t <= 1.5).all()
    assert (np.abs(a) <= 1).all()
    o = workloads.odd_i32_tile(64, 32)
    assert set(np.unique(o).tolist()) <= {-3, -1, 1, 3}
