"""Pins of the CPU oracle to facts outside the oracle itself.

Each pin is a function ``pin(o)`` that raises AssertionError when the oracle
``o`` disagrees with something the pages or the mathematics fix: exact sums
and products with ``fractions.Fraction`` or Python integers on small inputs,
closed forms, the worked examples in ``tests/golden/`` (derived by hand from
the TVM TIRx page "reduction -> sm100_packed", section "Algorithm"),
special values, and exhaustive checks of the 16-bit decoders against numpy's
binary16 and torch's bfloat16.

The same pins run against the real oracle (test_oracle.py) and against
deliberately broken copies of it (test_oracle_mutants.py), which shows each
plausible mistake fails at least one of them.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 1 << 32


def f32(v) -> np.float32:
    return np.float32(v)


def bits(v) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def exact_sum(values) -> Fraction:
    return sum((Fraction(float(v)) for v in values), Fraction(0))


def exact_prod(values) -> Fraction:
    p = Fraction(1)
    for v in values:
        p *= Fraction(float(v))
    return p


def load_page_order_cases():
    """Parse tests/golden/page_order_sum.txt into dict records."""
    cases = []
    with open(os.path.join(GOLDEN, "page_order_sum.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, n, entries, accum, old, expected, why = (
                p.strip() for p in line.split(";", 6))
            x = np.zeros(int(n), np.float32)
            for e in entries.split():
                i, v = e.split("=")
                x[int(i)] = np.float32(float(v))
            cases.append(dict(name=name, x=x, accum=bool(int(accum)),
                              old=float(old), expected=np.float32(float(expected)),
                              why=why))
    return cases


# ---------------------------------------------------------------------------
# sum
# ---------------------------------------------------------------------------

def pin_sum_bruteforce(o):
    """S and A against exact rational sums on small random inputs."""
    rng = np.random.default_rng(11)
    for n in (1, 2, 3, 7, 8, 9, 31, 32, 33, 64, 257):
        mag = 10.0 ** rng.uniform(-3, 3, n)
        x = (rng.uniform(-1, 1, n) * mag).astype(np.float32)
        old = float(np.float32(rng.uniform(-10, 10)))
        for accum in (False, True):
            terms = list(x) + ([np.float32(old)] if accum else [])
            ex = exact_sum(terms)
            ab = sum((abs(Fraction(float(v))) for v in terms), Fraction(0))
            s, a = o.sum_f32(x, accum, old)
            assert abs(Fraction(s) - ex) <= Fraction(1, 10**15) * ab, (n, s, ex)
            assert abs(Fraction(a) - ab) <= Fraction(1, 10**15) * ab, (n, a, ab)


def pin_sum_integer_exact(o):
    """Integer-valued inputs: every partial sum is exact, so S is exact."""
    rng = np.random.default_rng(12)
    x = rng.integers(-1000, 1001, 5000).astype(np.float32)
    s, a = o.sum_f32(x)
    assert s == float(np.sum(x.astype(np.int64)))
    assert a == float(np.sum(np.abs(x.astype(np.int64))))


def pin_sum_arithmetic_series(o):
    """1 + 2 + ... + n = n (n + 1) / 2."""
    for n in (1, 8, 32, 4096, 100000):
        x = np.arange(1, n + 1, dtype=np.float32)
        s, a = o.sum_f32(x)
        assert s == n * (n + 1) / 2 and a == s, (n, s)


def pin_sum_cancellation(o):
    """The compensation must recover a term a plain double sum loses."""
    big = float(2 ** 60)
    for x in ([big, 1.0, -big], [1.0, big, -big], [-big, 1.0, big]):
        s, a = o.sum_f32(np.array(x, np.float32))
        assert s == 1.0, (x, s)
        assert a == 2 * big + 1.0 or a == 2 * big  # A needs no compensation


def pin_sum_accum(o):
    """accum folds the old dst into the result and into A."""
    s, a = o.sum_f32(np.array([1.0, 2.0], np.float32), True, 3.25)
    assert (s, a) == (6.25, 6.25)
    s, a = o.sum_f32(np.array([1.0, 2.0], np.float32), True, -3.25)
    assert (s, a) == (-0.25, 6.25)
    s, a = o.sum_f32(np.array([1.0, 2.0], np.float32), False, 100.0)
    assert (s, a) == (3.0, 3.0)


def pin_sum_empty(o):
    """An empty vector computes nothing, even under accum."""
    assert o.sum_f32(np.zeros(0, np.float32)) is None
    assert o.sum_f32(np.zeros(0, np.float32), True, 3.25) is None


def pin_sum_nonfinite(o):
    """IEEE classes propagate: inf + 1 = inf, inf + -inf = NaN."""
    inf = float("inf")
    assert o.sum_f32(np.array([inf, 1], np.float32))[0] == inf
    assert o.sum_f32(np.array([-inf, 5], np.float32))[0] == -inf
    assert math.isnan(o.sum_f32(np.array([inf, -inf], np.float32))[0])
    assert math.isnan(o.sum_f32(np.array([float("nan"), 1], np.float32))[0])


def pin_sum_subnormal(o):
    """Subnormals are not flushed: 2^-149 + 2^-149 + 2^-148 = 2^-147."""
    x = np.array([2.0 ** -149, 2.0 ** -149, 2.0 ** -148], np.float32)
    assert x[0] != 0
    s, _ = o.sum_f32(x)
    assert s == 2.0 ** -147


def _ieee_seq_sum(terms) -> float:
    """IEEE-754 double addition from the additive identity -0.0, term by
    term (Python floats are IEEE doubles, round to nearest even)."""
    acc = -0.0
    for v in terms:
        acc = acc + float(v)
    return acc


def pin_sum_signed_zero(o):
    """A sum that is exactly zero is -0 when every term is -0 and +0
    otherwise (IEEE-754 addition in round-to-nearest; the same in any
    order).  Checked against sequential IEEE addition and by hand."""
    nz, pz = np.float32(-0.0), np.float32(0.0)
    cases = [
        ([nz] * 1, False, 0.0, -1), ([nz] * 7, False, 0.0, -1),
        ([nz] * 33, False, 0.0, -1), ([pz] * 8, False, 0.0, 1),
        ([nz, pz], False, 0.0, 1), ([pz, nz, nz], False, 0.0, 1),
        ([1.0, -1.0], False, 0.0, 1), ([-2.5, nz, 2.5], False, 0.0, 1),
        ([nz] * 3, True, -0.0, -1), ([nz] * 3, True, 0.0, 1),
        ([pz] * 3, True, -0.0, 1), ([nz] * 3, False, 0.0, -1),
        ([0.75, -0.5], True, -0.25, 1),
    ]
    for terms, accum, old, sign in cases:
        x = np.array(terms, np.float32)
        s, a = o.sum_f32(x, accum, old)
        ref = _ieee_seq_sum(([old] if accum else []) + list(x))
        assert s == 0 and ref == 0, (terms, s, ref)
        assert math.copysign(1.0, s) == sign == math.copysign(1.0, ref), (terms, accum, old, s)
    # rows and columns follow the same rule, row by row / column by column
    m = np.array([[nz, nz, nz], [nz, pz, nz], [1.0, nz, -1.0]], np.float32)
    s, _ = o.rows_sum_f32(m, 3, 3, 3)
    assert [math.copysign(1.0, v) for v in s] == [-1.0, 1.0, 1.0], s
    s, _ = o.cols_sum_f32(m.T.copy(), 3, 3, 3)
    assert [math.copysign(1.0, v) for v in s] == [-1.0, 1.0, 1.0], s
    old = np.array([-0.0, 0.0, -0.0], np.float32)
    s, _ = o.rows_sum_f32(np.full((3, 2), nz, np.float32), 3, 2, 2, True, old)
    assert [math.copysign(1.0, v) for v in s] == [-1.0, 1.0, -1.0], s


# ---------------------------------------------------------------------------
# max / min
# ---------------------------------------------------------------------------

def pin_maxmin_bruteforce(o):
    """Against Python's max / min, with the extreme at the ends and inside."""
    rng = np.random.default_rng(13)
    for n in (1, 2, 7, 8, 9, 33, 1000):
        for where in {0, n // 2, n - 1}:
            x = rng.uniform(-1, 1, n).astype(np.float32)
            x[where] = 7.5
            assert o.max_f32(x) == max(x.tolist()) == 7.5
            x[where] = -7.5
            assert o.min_f32(x) == min(x.tolist()) == -7.5
            y = rng.uniform(-1, 1, n).astype(np.float32)
            assert o.max_f32(y) == max(y.tolist())
            assert o.min_f32(y) == min(y.tolist())


def pin_maxmin_nan_policy(o):
    """maxNum / minNum: NaN is ignored unless every operand is NaN."""
    nan = float("nan")
    assert o.max_f32(np.array([nan, 1, nan], np.float32)) == 1
    assert o.min_f32(np.array([1, nan, -3], np.float32)) == -3
    assert o.max_f32(np.array([nan, -2], np.float32)) == -2
    assert math.isnan(o.max_f32(np.array([nan, nan], np.float32)))
    assert math.isnan(o.min_f32(np.array([nan], np.float32)))
    assert o.max_f32(np.array([nan], np.float32), True, 2.0) == 2
    assert o.min_f32(np.array([4.0], np.float32), True, nan) == 4


def pin_maxmin_accum(o):
    """accum includes the old dst: max(3.25, x) over x in [-1, 1] is 3.25."""
    rng = np.random.default_rng(14)
    x = rng.uniform(-1, 1, 100).astype(np.float32)
    assert o.max_f32(x, True, 3.25) == np.float32(3.25)
    assert o.min_f32(x, True, 3.25) == min(x.tolist())
    assert o.min_f32(x, True, -5.0) == -5.0
    assert o.max_f32(x, False, 3.25) == max(x.tolist())


def pin_maxmin_empty(o):
    """n == 0 leaves the destination untouched, even under accum."""
    e = np.zeros(0, np.float32)
    assert o.max_f32(e, False, 42.0) == 42.0
    assert o.min_f32(e, True, -42.0) == -42.0


def pin_maxmin_special(o):
    """Subnormals survive bit-exactly; infinities order normally."""
    t = 2.0 ** -149
    x = np.array([t, -t, 0.0], np.float32)
    assert bits(o.max_f32(x)) == bits(t)
    assert bits(o.min_f32(x)) == bits(-t)
    inf = float("inf")
    x = np.array([-inf, 1, 0.5], np.float32)
    assert o.max_f32(x) == 1 and o.min_f32(x) == -inf
    assert o.max_f32(np.array([inf], np.float32)) == inf
    assert o.max_f32(np.array([0.25], np.float32)) == np.float32(0.25)


# ---------------------------------------------------------------------------
# the page's single-precision summation order
# ---------------------------------------------------------------------------

def pin_page_sum_golden(o):
    """Hand-derived worked examples of the page's order (tests/golden)."""
    for c in load_page_order_cases():
        got = o.page_sum_f32(c["x"], c["accum"], c["old"])
        assert bits(got) == bits(c["expected"]), (c["name"], got, c["expected"])


def pin_page_sum_integer_exact(o):
    """Small integers: every order is exact, so the result is the exact sum."""
    rng = np.random.default_rng(15)
    for n in (1, 5, 8, 9, 16, 17, 31, 32, 33, 100, 1000):
        x = rng.integers(-100, 101, n).astype(np.float32)
        assert o.page_sum_f32(x) == float(np.sum(x.astype(np.int64))), n
        assert o.page_sum_f32(x, True, 7.0) == 7.0 + float(np.sum(x.astype(np.int64)))


def pin_page_sum_error_bound(o):
    """Random data: within the worst-case bound of an order of depth n/8 + 4."""
    rng = np.random.default_rng(16)
    for n in (8, 9, 15, 64, 100, 1000, 4099):
        x = rng.uniform(-1, 1, n).astype(np.float32)
        ex = exact_sum(x)
        ab = sum(abs(Fraction(float(v))) for v in x)
        depth = n // 8 + 4
        got = o.page_sum_f32(x)
        assert abs(Fraction(float(got)) - ex) <= depth * Fraction(1, 2**24) * ab


# ---------------------------------------------------------------------------
# rows
# ---------------------------------------------------------------------------

def pin_rows_bruteforce(o):
    """Each row of an ld-padded matrix reduces to its own brute-force value;
    the NaN padding between n and ld never enters."""
    rng = np.random.default_rng(17)
    rows, n, ld = 5, 13, 16
    m = np.full((rows, ld), np.nan, np.float32)
    m[:, :n] = rng.uniform(-1, 1, (rows, n)).astype(np.float32)
    old = rng.uniform(-1, 1, rows).astype(np.float32)
    s, a = o.rows_sum_f32(m, rows, n, ld)
    s2, _ = o.rows_sum_f32(m, rows, n, ld, True, old)
    mx = o.rows_max_f32(m, rows, n, ld)
    mn = o.rows_min_f32(m, rows, n, ld, True, old)
    for r in range(rows):
        row = m[r, :n]
        ex = exact_sum(row)
        ab = sum(abs(Fraction(float(v))) for v in row)
        assert abs(Fraction(s[r]) - ex) <= Fraction(1, 10**15) * ab
        assert abs(Fraction(a[r]) - ab) <= Fraction(1, 10**15) * ab
        ex2 = ex + Fraction(float(old[r]))
        assert abs(Fraction(s2[r]) - ex2) <= Fraction(1, 10**14) * (ab + 1)
        assert mx[r] == max(row.tolist())
        assert mn[r] == min(row.tolist() + [float(old[r])])


def pin_rows_page_golden(o):
    """Rows reproduce the golden page-order cases row by row, with ld > n."""
    cases = [c for c in load_page_order_cases() if c["x"].size == 8
             and not c["accum"]]
    ld = 11
    m = np.full((len(cases), ld), np.nan, np.float32)
    for r, c in enumerate(cases):
        m[r, :8] = c["x"]
    got = o.rows_page_sum_f32(m, len(cases), 8, ld)
    for r, c in enumerate(cases):
        assert bits(got[r]) == bits(c["expected"]), c["name"]


def pin_rows_empty(o):
    """rows == 0 or n == 0 leaves every destination untouched."""
    m = np.ones((3, 4), np.float32)
    sentinel = np.full(3, 9.5, np.float32)
    assert o.rows_sum_f32(m, 3, 0, 4) is None
    assert o.rows_sum_f32(m, 0, 4, 4) is None
    assert (o.rows_max_f32(m, 3, 0, 4, dst=sentinel) == 9.5).all()
    assert (o.rows_min_f32(m, 3, 0, 4, True, dst=sentinel) == 9.5).all()
    assert (o.rows_page_sum_f32(m, 3, 0, 4, dst=sentinel) == 9.5).all()


# ---------------------------------------------------------------------------
# colprod
# ---------------------------------------------------------------------------

def pin_colprod_f32_bruteforce(o):
    """The TCOLPROD example shape (16 x 16 -> 1 x 16) against exact products,
    plus a non-square ld-padded tile (R != C catches a transposed index)."""
    rng = np.random.default_rng(18)
    t = rng.uniform(0.5, 1.5, (16, 16)).astype(np.float32)
    got = o.colprod_f32(t, 16, 16, 16)
    for j in range(16):
        ex = exact_prod(t[:, j])
        assert abs(Fraction(got[j]) - ex) <= Fraction(1, 10**14) * abs(ex)
    R, C, ld = 5, 7, 9
    m = np.full((R, ld), np.nan, np.float32)
    m[:, :C] = rng.uniform(-2, 2, (R, C)).astype(np.float32)
    got = o.colprod_f32(m, R, C, ld)
    for j in range(C):
        ex = exact_prod(m[:, j])
        assert abs(Fraction(got[j]) - ex) <= Fraction(1, 10**14) * abs(ex)


def pin_colprod_f32_closed_forms(o):
    """Ones give exactly 1; powers of two are exact; zeros carry the XOR of
    the signs."""
    assert (o.colprod_f32(np.ones((100, 3), np.float32), 100, 3, 3) == 1).all()
    e = np.array([[2.0, 0.5, -4.0], [2.0, 0.25, 8.0], [-2.0, 4.0, 0.125]],
                 np.float32)
    assert o.colprod_f32(e, 3, 3, 3).tolist() == [-8.0, 0.5, -4.0]
    z = np.array([[-1.0, -1.0], [0.0, -0.0], [2.0, 3.0]], np.float32)
    got = o.colprod_f32(z, 3, 2, 2)
    assert got[0] == 0 and math.copysign(1, got[0]) == -1
    assert got[1] == 0 and math.copysign(1, got[1]) == 1


def pin_colprod_empty(o):
    """R == 0 or C == 0: early return, dst untouched (no empty product 1)."""
    t = np.ones((4, 4), np.float32)
    for (R, C) in ((0, 4), (4, 0), (0, 0)):
        d = o.colprod_f32(t, R, C, 4, dst=np.full(4, 7.0))
        assert (d == 7.0).all(), (R, C)
        d = o.colprod_i32(t.astype(np.int32), R, C, 4,
                          dst=np.full(4, 7, np.int32))
        assert (d == 7).all(), (R, C)
        h = t.astype(np.float16).view(np.uint16)
        assert (o.colprod_f16(h, R, C, 4, dst=np.full(4, 7.0)) == 7.0).all()
        assert (o.colprod_bf16(h, R, C, 4, dst=np.full(4, 7.0)) == 7.0).all()


def _same_float(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def pin_f16_decode_exhaustive(o):
    """All 65536 binary16 patterns decode as numpy's float16 does."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    for b in range(0, 65536):
        assert _same_float(o.f16_to_f64(b), float(ref[b])), hex(b)


def pin_bf16_decode_exhaustive(o):
    """All 65536 bfloat16 patterns decode as torch's bfloat16 does, and a
    few values known from the format's definition."""
    import torch
    allbits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = allbits.view(torch.bfloat16).to(torch.float64).tolist()
    for b in range(0, 65536):
        assert _same_float(o.bf16_to_f64(b), ref[b]), hex(b)
    known = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0000: 0.0,
             0x7F80: float("inf"), 0x0001: 2.0 ** -133,
             0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127}
    for b, v in known.items():
        assert o.bf16_to_f64(b) == v, hex(b)


def pin_colprod_16bit_bruteforce(o):
    """fp16 / bf16 tiles against exact products of independently decoded
    values (numpy float16, torch bfloat16)."""
    import torch
    rng = np.random.default_rng(19)
    v = rng.uniform(0.5, 1.5, (16, 16)).astype(np.float32)
    h = v.astype(np.float16)
    got = o.colprod_f16(h.view(np.uint16), 16, 16, 16)
    for j in range(16):
        ex = exact_prod(h[:, j].astype(np.float64))
        assert abs(Fraction(got[j]) - ex) <= Fraction(1, 10**14) * abs(ex)
    b = torch.from_numpy(v).to(torch.bfloat16)
    bb = b.view(torch.int16).numpy().view(np.uint16)
    got = o.colprod_bf16(bb, 16, 16, 16)
    bd = b.to(torch.float64).numpy()
    for j in range(16):
        ex = exact_prod(bd[:, j])
        assert abs(Fraction(got[j]) - ex) <= Fraction(1, 10**14) * abs(ex)


def _i32(v: int) -> int:
    v %= U32
    return v - U32 if v >= 1 << 31 else v


def pin_colprod_i32_bruteforce(o):
    """Full-range int32 against Python big-int products modulo 2^32."""
    rng = np.random.default_rng(20)
    R, C, ld = 16, 13, 16
    t = rng.integers(-2**31, 2**31, (R, ld), dtype=np.int64).astype(np.int32)
    got = o.colprod_i32(t, R, C, ld)
    for j in range(C):
        p = 1
        for i in range(R):
            p *= int(t[i, j])
        assert int(got[j]) == _i32(p), j


def pin_colprod_i32_closed_forms(o):
    """(-1)^R, 3^R mod 2^32, 2^R = 0 for R >= 32, INT_MIN * -1 = INT_MIN."""
    for R in (7, 8):
        got = o.colprod_i32(np.full((R, 2), -1, np.int32), R, 2, 2)
        assert got.tolist() == [(-1) ** R] * 2
    got = o.colprod_i32(np.full((4096, 3), 3, np.int32), 4096, 3, 3)
    assert got.tolist() == [_i32(pow(3, 4096, U32))] * 3
    got = o.colprod_i32(np.full((40, 1), 2, np.int32), 40, 1, 1)
    assert got.tolist() == [0]
    got = o.colprod_i32(np.array([[-2**31], [-1]], np.int32), 2, 1, 1)
    assert got.tolist() == [-2**31]


def pin_colprod_u32_bruteforce(o):
    """uint32 against Python big-int products modulo 2^32."""
    rng = np.random.default_rng(21)
    R, C, ld = 16, 11, 13
    t = rng.integers(0, 2**32, (R, ld), dtype=np.uint64).astype(np.uint32)
    got = o.colprod_u32(t, R, C, ld)
    for j in range(C):
        p = 1
        for i in range(R):
            p *= int(t[i, j])
        assert int(got[j]) == p % U32, j
    got = o.colprod_u32(np.full((4096, 2), 3, np.uint32), 4096, 2, 2)
    assert got.tolist() == [pow(3, 4096, U32)] * 2
    assert (o.colprod_u32(np.ones((3, 3), np.uint32), 0, 3, 3,
                          dst=np.full(3, 5, np.uint32)) == 5).all()


def pin_colprod_u16_bruteforce(o):
    """16-bit patterns against Python big-int products modulo 2^16, read
    both as uint16 and as int16; closed forms (-1)^R, 3^R, 2^R."""
    rng = np.random.default_rng(22)
    R, C, ld = 16, 9, 12
    t = rng.integers(0, 2**16, (R, ld), dtype=np.int64).astype(np.uint16)
    got = o.colprod_u16(t, R, C, ld)
    for j in range(C):
        pu, ps = 1, 1
        for i in range(R):
            pu *= int(t[i, j])
            ps *= int(t[i, j].astype(np.int16))
        assert int(got[j]) == pu % (1 << 16) == ps % (1 << 16), j
    m1 = np.full((7, 1), 0xFFFF, np.uint16)          # int16 -1
    assert o.colprod_u16(m1, 7, 1, 1).tolist() == [0xFFFF]
    assert o.colprod_u16(m1[:6], 6, 1, 1).tolist() == [1]
    t3 = np.full((2048, 1), 3, np.uint16)
    assert o.colprod_u16(t3, 2048, 1, 1).tolist() == [pow(3, 2048, 1 << 16)]
    t2 = np.full((16, 1), 2, np.uint16)
    assert o.colprod_u16(t2, 16, 1, 1).tolist() == [0]
    assert o.colprod_u16(t2[:15], 15, 1, 1).tolist() == [1 << 15]
    assert (o.colprod_u16(t3, 2048, 0, 1, dst=np.full(1, 9, np.uint16)) == 9).all()


def pin_cols_bruteforce(o):
    """Column sum / max / min of an ld-padded tile against exact sums and
    Python's max / min per column (R != C catches a transposed index); the
    NaN padding never enters; accum folds old[j]."""
    rng = np.random.default_rng(23)
    R, C, ld = 11, 6, 9
    m = np.full((R, ld), np.nan, np.float32)
    m[:, :C] = rng.uniform(-5, 5, (R, C)).astype(np.float32)
    old = rng.uniform(-1, 1, C).astype(np.float32)
    s, a = o.cols_sum_f32(m, R, C, ld)
    s2, a2 = o.cols_sum_f32(m, R, C, ld, True, old)
    mx = o.cols_max_f32(m, R, C, ld)
    mn = o.cols_min_f32(m, R, C, ld, True, old)
    for j in range(C):
        col = m[:R, j]
        ex = exact_sum(col)
        ab = sum(abs(Fraction(float(v))) for v in col)
        assert abs(Fraction(s[j]) - ex) <= Fraction(1, 10**15) * ab
        assert abs(Fraction(a[j]) - ab) <= Fraction(1, 10**15) * ab
        ex2 = ex + Fraction(float(old[j]))
        assert abs(Fraction(s2[j]) - ex2) <= Fraction(1, 10**14) * (ab + 1)
        assert mx[j] == max(col.tolist())
        assert mn[j] == min(col.tolist() + [float(old[j])])


def pin_cols_closed_forms(o):
    """Ones sum to R; 1..R sums to R(R+1)/2; NaN policy; empty untouched."""
    R = 1000
    s, a = o.cols_sum_f32(np.ones((R, 3), np.float32), R, 3, 3)
    assert (s == R).all() and (a == R).all()
    ar = np.repeat(np.arange(1, R + 1, dtype=np.float32)[:, None], 2, axis=1)
    s, _ = o.cols_sum_f32(ar, R, 2, 2)
    assert (s == R * (R + 1) / 2).all()
    assert (o.cols_max_f32(ar, R, 2, 2) == R).all()
    assert (o.cols_min_f32(ar, R, 2, 2) == 1).all()
    nan = float("nan")
    t = np.array([[nan, 1.0], [2.0, nan], [nan, nan]], np.float32)
    assert o.cols_max_f32(t, 3, 2, 2).tolist() == [2.0, 1.0]
    assert math.isnan(o.cols_max_f32(t[2:], 1, 2, 2)[0])
    assert o.cols_sum_f32(t, 0, 2, 2) is None
    assert (o.cols_min_f32(t, 3, 0, 2, dst=np.full(2, 4.0)) == 4.0).all()


# ---------------------------------------------------------------------------
# threaded forms
# ---------------------------------------------------------------------------

THREADS = (1, 2, 3, 7, 16)


def pin_mt_sum(o):
    """Threaded sums against exact rational sums, for thread counts that do
    and do not divide n and exceed it; the signed-zero rule; empty input."""
    rng = np.random.default_rng(81)
    for n in (1, 5, 33, 1000):
        x = (rng.uniform(-1, 1, n) * 10.0 ** rng.uniform(-3, 3, n)).astype(np.float32)
        for t in THREADS + (n + 3,):
            for accum, old in ((False, 0.0), (True, -7.5)):
                terms = list(x) + ([np.float32(old)] if accum else [])
                ex = exact_sum(terms)
                ab = sum((abs(Fraction(float(v))) for v in terms), Fraction(0))
                s, a = o.sum_f32_mt(x, t, accum, old)
                assert abs(Fraction(s) - ex) <= Fraction(1, 10**14) * ab, (n, t, s, ex)
                assert abs(Fraction(a) - ab) <= Fraction(1, 10**14) * ab, (n, t, a, ab)
    x = rng.integers(-1000, 1001, 100001).astype(np.float32)
    assert o.sum_f32_mt(x, 16)[0] == float(np.sum(x.astype(np.int64)))
    nz = np.full(9, -0.0, np.float32)
    assert math.copysign(1.0, o.sum_f32_mt(nz, 4)[0]) == -1.0
    nz[5] = 0.0
    assert math.copysign(1.0, o.sum_f32_mt(nz, 4)[0]) == 1.0
    assert o.sum_f32_mt(np.zeros(0, np.float32), 4) is None


def pin_mt_extremes(o):
    """Threaded max / min against Python's max / min, with accum and NaN."""
    rng = np.random.default_rng(82)
    for n in (1, 6, 100, 4099):
        x = rng.standard_normal(n).astype(np.float32)
        for t in THREADS + (n + 1,):
            assert o.max_f32_mt(x, t) == max(x.tolist()), (n, t)
            assert o.min_f32_mt(x, t) == min(x.tolist()), (n, t)
            assert o.max_f32_mt(x, t, True, 50.0) == np.float32(50.0)
            assert o.min_f32_mt(x, t, True, -50.0) == np.float32(-50.0)
    x = np.array([np.nan, 2.0, np.nan, np.nan, -1.0, np.nan], np.float32)
    assert o.max_f32_mt(x, 3) == 2.0 and o.min_f32_mt(x, 6) == -1.0
    assert math.isnan(o.max_f32_mt(np.full(5, np.nan, np.float32), 2))


def pin_mt_rows(o):
    """Threaded row sums and maxima against exact sums and numpy maxima."""
    rng = np.random.default_rng(83)
    rows, n, ld = 13, 9, 11
    x = rng.uniform(-2, 2, (rows, ld)).astype(np.float32)
    for t in THREADS + (rows + 2,):
        s, a = o.rows_sum_f32_mt(x, rows, n, ld, t)
        m = o.rows_max_f32_mt(x, rows, n, ld, t)
        for r in range(rows):
            ex = exact_sum(x[r, :n])
            assert abs(Fraction(s[r]) - ex) <= Fraction(1, 10**14) * exact_sum(np.abs(x[r, :n]))
            assert a[r] == float(exact_sum(np.abs(x[r, :n].astype(np.float64))))
            assert m[r] == x[r, :n].max(), (r, t)


def pin_mt_colprod(o):
    """Threaded column products against exact products of independently
    decoded values (fp32, numpy float16, bfloat16 as the upper half of a
    binary32) and big-integer products modulo 2^32."""
    rng = np.random.default_rng(84)
    R, C, ld = 7, 19, 21
    v = rng.uniform(0.5, 1.5, (R, ld)).astype(np.float32)
    h = v.astype(np.float16)
    bbits = (v.view(np.uint32) >> 16).astype(np.uint16)
    bvals = (bbits.astype(np.uint32) << 16).view(np.float32)
    iv = rng.integers(-(2 ** 31), 2 ** 31, (R, ld), dtype=np.int64).astype(np.int32)
    for t in THREADS + (C + 4,):
        pf = o.colprod_f32_mt(v, R, C, ld, t)
        ph = o.colprod_f16_mt(h.view(np.uint16), R, C, ld, t)
        pb = o.colprod_bf16_mt(bbits, R, C, ld, t)
        pi = o.colprod_i32_mt(iv, R, C, ld, t)
        for j in range(C):
            for got, col in ((pf[j], v[:, j]), (ph[j], h[:, j]), (pb[j], bvals[:, j])):
                ex = exact_prod(col.astype(np.float64))
                assert abs(Fraction(got) - ex) <= Fraction(1, 10**14) * abs(ex), (t, j)
            p = 1
            for val in iv[:, j].tolist():
                p = (p * val) % U32
            assert pi[j] == _i32(p), (t, j)


PINS = [
    pin_sum_bruteforce, pin_sum_integer_exact, pin_sum_arithmetic_series,
    pin_sum_cancellation, pin_sum_accum, pin_sum_empty, pin_sum_nonfinite,
    pin_sum_subnormal, pin_sum_signed_zero,
    pin_maxmin_bruteforce, pin_maxmin_nan_policy, pin_maxmin_accum,
    pin_maxmin_empty, pin_maxmin_special,
    pin_page_sum_golden, pin_page_sum_integer_exact, pin_page_sum_error_bound,
    pin_rows_bruteforce, pin_rows_page_golden, pin_rows_empty,
    pin_colprod_f32_bruteforce, pin_colprod_f32_closed_forms,
    pin_colprod_empty, pin_f16_decode_exhaustive, pin_bf16_decode_exhaustive,
    pin_colprod_16bit_bruteforce, pin_colprod_i32_bruteforce,
    pin_colprod_i32_closed_forms, pin_colprod_u32_bruteforce,
    pin_colprod_u16_bruteforce, pin_cols_bruteforce, pin_cols_closed_forms,
    pin_mt_sum, pin_mt_extremes, pin_mt_rows, pin_mt_colprod,
]
