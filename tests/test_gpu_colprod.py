"""GPU parity of the column products (TCOLPROD) against the CPU oracle:
the 16 x 16 example tile, the full 4096 x 16384 f32 / i32 tiles (plus an
odd-valued i32 tile whose products do not vanish mod 2^32), the
2048 x 32768 bf16 / f16 tiles, and ragged, padded and misaligned shapes."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (COLPROD_16_TOL, COLPROD_F32_TOL, check_rel, dev, host,
                         say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


TORCH_T = {"f32": "float32", "f16": "float16", "bf16": "bfloat16", "i32": "int32"}


def to_dev(kind, a):
    """Upload a host tile: f16 / bf16 arrive as uint16 bit patterns."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = dev(a)
    if kind in ("f16", "bf16"):
        t = t.view(torch.int16).view(getattr(torch, TORCH_T[kind]))
    return t


def run(red, kind, sd, C, fill=0):
    dt = getattr(torch, TORCH_T[kind])
    out = torch.full((C,), fill, dtype=dt, device="cuda") if C else \
        torch.zeros(1, dtype=dt, device="cuda")
    getattr(red, "colprod_" + kind)(sd, out, C=C)
    o = host(out.view(torch.int16) if kind in ("f16", "bf16") else out)
    return o.view(np.uint16) if kind in ("f16", "bf16") else o


def decode(kind, bits):
    if kind == "f16":
        return bits.view(np.float16).astype(np.float64)
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def check(orc, kind, src, R, C, ld, got, what):
    if kind == "i32":
        want = orc.colprod_i32(src, R, C, ld)
        bad = np.nonzero(got[:C] != want)[0]
        assert bad.size == 0, "%s: column %d got %d want %d" % (
            what, bad[0], got[bad[0]], want[bad[0]])
        return 0.0
    if kind == "f32":
        want = orc.colprod_f32(src, R, C, ld)
        return check_rel(got[:C], want, COLPROD_F32_TOL, what)
    fn = orc.colprod_f16 if kind == "f16" else orc.colprod_bf16
    want = fn(src, R, C, ld)
    return check_rel(decode(kind, got[:C]), want, COLPROD_16_TOL, what)


def test_tile16_example(red, orc):
    """The 16 x 16 -> 1 x 16 fp32 example shape (uniform[0.5, 1.5))."""
    say("colprod 16x16 tile")
    _, t = workloads.rows32()
    got = run(red, "f32", dev(t), 16)
    check(orc, "f32", t, 16, 16, 16, got, "tile16")


@pytest.fixture(scope="module")
def tiles4k():
    say("generate 4096 x 16384 f32 / i32 tiles (seed 2)")
    f, i = workloads.colprod4k_f32_i32()
    return f, i


@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_tiles4k(red, orc, tiles4k, kind):
    f, i = tiles4k
    src = f if kind == "f32" else i
    say("colprod 4096x16384 %s" % kind)
    got = run(red, kind, to_dev(kind, src), 16384)
    worst = check(orc, kind, src, 4096, 16384, 16384, got, "tiles4k " + kind)
    if kind == "f32":
        say("colprod 4096x16384 f32: worst relative error %.3g (tolerance 4e-4)" % worst)
        assert worst <= 4095 * 2.0 ** -24  # the order-free bound


def test_tiles4k_i32_odd(red, orc):
    """Odd values only: products stay nonzero mod 2^32, so the bit-exact
    comparison means something (the {-3..3} tile's products are all 0)."""
    say("colprod 4096x16384 odd i32")
    t = workloads.odd_i32_tile()
    got = run(red, "i32", dev(t), 16384)
    assert (got != 0).all()
    check(orc, "i32", t, 4096, 16384, 16384, got, "odd i32")


@pytest.fixture(scope="module")
def tiles16bit():
    say("generate 2048 x 32768 bf16 / f16 tiles (seed 4)")
    _, b, h = workloads.rows1000()
    return b, h


@pytest.mark.parametrize("kind", ["bf16", "f16"])
def test_tiles16bit(red, orc, tiles16bit, kind):
    b, h = tiles16bit
    src = b if kind == "bf16" else h
    say("colprod 2048x32768 %s" % kind)
    got = run(red, kind, to_dev(kind, src), 32768)
    worst = check(orc, kind, src, 2048, 32768, 32768, got, "tiles16bit " + kind)
    say("colprod 2048x32768 %s: worst relative error %.3g (tolerance 2e-2)" % (kind, worst))


SHAPES = [  # (R, C, ld, element offset of the base pointer)
    (1, 1, 1, 0), (1, 37, 37, 0), (16, 16, 16, 0), (37, 1, 1, 0),
    (5, 3, 4, 1), (100, 259, 260, 0), (257, 515, 515, 0), (64, 4, 8, 0),
    (33, 1024, 1024, 3), (129, 513, 520, 0), (1000, 130, 136, 2),
    (4096, 300, 304, 0), (8191, 72, 72, 0), (3000, 2049, 2049, 1),
]


@pytest.mark.parametrize("kind", ["f32", "i32", "f16", "bf16"])
@pytest.mark.parametrize("R,C,ld,off", SHAPES)
def test_shapes(red, orc, kind, R, C, ld, off):
    say("colprod shape %s R=%d C=%d ld=%d off=%d" % (kind, R, C, ld, off))
    n = R * ld + off + 8
    if kind == "i32":
        flat = workloads.integers_i32(40, n, -(2 ** 31), 2 ** 31)
        flat[off:off + R * ld].reshape(R, ld)[:, C:] = 0
    else:
        lo, hi = (0.99, 1.01) if R > 64 else (0.5, 1.5)
        vals = workloads.uniform_f32(41, n, lo, hi)
        vals[off:off + R * ld].reshape(R, ld)[:, C:] = np.nan  # padding
        if kind == "f32":
            flat = vals
        elif kind == "f16":
            flat = workloads.to_f16_bits(vals)
        else:
            flat = workloads.to_bf16_bits(vals)
    fd = to_dev(kind, flat)
    src = flat[off:off + R * ld].reshape(R, ld)
    sd = fd[off:off + R * ld].view(R, ld)
    got = run(red, kind, sd, C)
    check(orc, kind, src, R, C, ld, got, "%s R=%d C=%d ld=%d off=%d" % (kind, R, C, ld, off))


def test_closed_forms(red):
    say("colprod closed forms")
    # ones -> exactly 1; powers of two -> exact; zero -> signed zero
    ones = torch.ones((3000, 70), dtype=torch.float32, device="cuda")
    assert (run(red, "f32", ones, 70) == 1.0).all()
    rng = np.random.default_rng(42)
    e = rng.integers(-1, 2, (200, 300))
    p2 = np.ldexp(1.0, e).astype(np.float32) * rng.choice([-1, 1], (200, 300)).astype(np.float32)
    got = run(red, "f32", dev(p2), 300)
    want = np.prod(p2.astype(np.float64), axis=0)
    assert (got.astype(np.float64) == want).all()
    z = np.ones((100, 5), np.float32)
    z[50, 1] = 0.0
    z[3, 1] = -1.0
    z[7, 3] = -0.0
    got = run(red, "f32", dev(z), 5)
    assert got[1] == 0 and math.copysign(1, got[1]) == -1
    assert got[3] == 0 and math.copysign(1, got[3]) == -1
    assert (got[[0, 2, 4]] == 1).all()
    # i32: (-1)^R, 3^R mod 2^32
    m1 = torch.full((4097, 9), -1, dtype=torch.int32, device="cuda")
    assert (run(red, "i32", m1, 9) == -1).all()
    t3 = torch.full((4096, 5), 3, dtype=torch.int32, device="cuda")
    p = pow(3, 4096, 1 << 32)
    assert (run(red, "i32", t3, 5) == (p - (1 << 32) if p >= 1 << 31 else p)).all()


def test_empty_untouched(red):
    """R == 0 or C == 0: TCOLPROD's early return; dst keeps its contents."""
    say("colprod empty")
    for kind in ("f32", "i32", "f16", "bf16"):
        dt = getattr(torch, TORCH_T[kind])
        src = torch.ones((0, 8), dtype=dt, device="cuda")
        out = torch.full((8,), 7, dtype=dt, device="cuda")
        getattr(red, "colprod_" + kind)(src, out)
        assert (out.cpu().float() == 7).all()
        src = torch.ones((4, 8), dtype=dt, device="cuda")
        getattr(red, "colprod_" + kind)(src, out, C=0)
        assert (out.cpu().float() == 7).all()


def test_deterministic(red, tiles4k):
    say("colprod determinism")
    f, _ = tiles4k
    fd = dev(f)
    ref = run(red, "f32", fd, 16384)
    for _ in range(2):
        assert run(red, "f32", fd, 16384).tobytes() == ref.tobytes()


# ---------------------------------------------------------------------------
# int16 / uint16 / uint32 (bit-exact modulo 2^16 / 2^32)
# ---------------------------------------------------------------------------

INT_KINDS = {  # kind: (host storage, torch storage, binding, oracle)
    "i16": (np.int16, torch.int16, "colprod_i16", "colprod_u16"),
    "u16": (np.uint16, torch.int16, "colprod_u16", "colprod_u16"),
    "u32": (np.uint32, torch.int32, "colprod_u32", "colprod_u32"),
}


def run_int(red, kind, src_host_2d, C, off=0):
    """Upload src (with an element offset), run, return the result bits."""
    hdt, tdt, fn, _ = INT_KINDS[kind]
    R, ld = src_host_2d.shape
    flat = np.zeros(R * ld + off + 8, hdt)
    flat[off:off + R * ld] = src_host_2d.reshape(-1)
    signed = np.int16 if tdt == torch.int16 else np.int32
    fd = dev(flat.view(signed))
    sd = fd[off:off + R * ld].view(R, ld)
    out = torch.zeros(max(C, 1), dtype=tdt, device="cuda")
    getattr(red, fn)(sd, out, C=C)
    return host(out).view(np.uint16 if tdt == torch.int16 else np.uint32)[:C]


def want_int(orc, kind, src_host_2d, C):
    R, ld = src_host_2d.shape
    bits = src_host_2d.view(np.uint16) if kind in ("i16", "u16") else src_host_2d.view(np.uint32)
    return getattr(orc, INT_KINDS[kind][3])(bits, R, C, ld)


@pytest.mark.parametrize("kind", ["i16", "u16", "u32"])
@pytest.mark.parametrize("R,C,ld,off", SHAPES)
def test_int_shapes(red, orc, kind, R, C, ld, off):
    say("colprod int shape %s R=%d C=%d ld=%d off=%d" % (kind, R, C, ld, off))
    hdt = INT_KINDS[kind][0]
    hi = 1 << (8 * np.dtype(hdt).itemsize)
    rng = np.random.default_rng(50)
    src = rng.integers(0, hi, (R, ld), dtype=np.uint64)
    src = (src | 1).astype(np.uint64)  # odd: products stay nonzero
    src = src.astype(np.uint16 if hi == 1 << 16 else np.uint32).view(hdt)
    got = run_int(red, kind, src, C, off)
    want = want_int(orc, kind, src, C)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: column %d got %d want %d" % (kind, bad[0], got[bad[0]], want[bad[0]])


# Short, wide 16-bit tiles of 4 row groups per block with a ragged last
# block beside whole ones in the last workgroup (the 2-byte layout whose
# combine places most values of a block from threads that read another).
@pytest.mark.parametrize("kind", ["i16", "u16"])
@pytest.mark.parametrize("R,C,ld", [(2, 236_272, 236_272), (5, 256_356, 256_360),
                                    (1, 518_552, 518_552)])
def test_int_wide_ragged(red, orc, kind, R, C, ld):
    say("colprod int wide ragged %s R=%d C=%d ld=%d" % (kind, R, C, ld))
    rng = np.random.default_rng(51)
    src = (rng.integers(0, 1 << 16, (R, ld), dtype=np.uint64) | 1).astype(np.uint16)
    src = src.view(INT_KINDS[kind][0])
    got = run_int(red, kind, src, C)
    want = want_int(orc, kind, src, C)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: column %d got %d want %d" % (kind, bad[0], got[bad[0]], want[bad[0]])


@pytest.mark.parametrize("kind,R,C", [("u32", 4096, 16384), ("i16", 2048, 32768),
                                      ("u16", 2048, 32768)])
def test_int_large(red, orc, kind, R, C):
    """Full-size tiles of odd values (whose products do not vanish)."""
    say("colprod int large %s %dx%d" % (kind, R, C))
    hdt = INT_KINDS[kind][0]
    vals = workloads.odd_i32_tile(R, C, seed=51)  # {-3, -1, 1, 3}
    src = vals.astype(hdt)
    got = run_int(red, kind, src, C)
    want = want_int(orc, kind, src, C)
    assert (got == want).all()
    assert (want != 0).all()


def test_int_closed_forms(red):
    say("colprod int closed forms")
    m1 = np.full((4097, 5), -1, np.int16)
    assert (run_int(red, "i16", m1, 5) == 0xFFFF).all()          # (-1)^odd
    t3 = np.full((2048, 3), 3, np.uint16)
    assert (run_int(red, "u16", t3, 3) == pow(3, 2048, 1 << 16)).all()
    t2 = np.full((16, 3), 2, np.uint16)
    assert (run_int(red, "u16", t2, 3) == 0).all()
    big = np.full((3, 2), 0xFFFFFFFF, np.uint32)                   # (2^32-1)^3
    assert (run_int(red, "u32", big, 2) == pow(2**32 - 1, 3, 1 << 32)).all()
