"""Seeded random parity sweep over every entry point.

Sizes are drawn log-uniformly so that the cases fall on both sides of
every kernel-selection boundary (1-D: one or many workgroups, partial last
sweep; rows: n up to 16, 64, 128, 256, 512, 1024 and 4096 elements, few and
many rows, split rows; columns: ragged last column block, row splits,
16-byte-aligned and unaligned rows), with random base misalignment, row
padding (filled with NaN, which must never reach a result) and accum.  Every
result is checked against the CPU oracle: bit-exact for max / min, the
page-order sum of rows of at most 64 elements and the integer products;
the stated tolerances otherwise.  The generator seed is fixed, so a
failure names a reproducible case."""
import math

import numpy as np
import pytest

import oracle
from gpu_helpers import (COLPROD_16_TOL, COLPROD_F32_TOL, check_exact, check_extremes,
                         check_rel, check_sum, check_sums, dev, has_both_zeros, host, say,
                         valid_region)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def log_uniform(rng, lo, hi):
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def upload_padded(x2d, off, fill=np.nan):
    """(rows, ld) fp32 host matrix -> device view starting `off` elements
    into a larger buffer."""
    rows, ld = x2d.shape
    flat = np.full(rows * ld + off + 8, fill, np.float32)
    flat[off:off + rows * ld] = x2d.reshape(-1)
    return dev(flat)[off:off + rows * ld].view(rows, ld)


def test_random_1d(red, orc):
    rng = np.random.default_rng(9001)
    for case in range(60):
        n = log_uniform(rng, 1, 3_000_000)
        off = int(rng.integers(0, 4))
        op = ("sum", "max", "min")[case % 3]
        accum = bool(rng.integers(0, 2))
        variant = ("", "_atomic", "fused")[int(rng.integers(0, 3))]
        old = np.float32(rng.uniform(-4, 4))
        x = rng.standard_normal(n).astype(np.float32)
        if rng.random() < 0.2:
            x[rng.integers(0, n, max(1, n // 100))] = np.nan
        what = "1d case %d n=%d off=%d op=%s accum=%s variant=%s" % (case, n, off, op, accum, variant)
        say(what)
        xd = dev(np.concatenate([np.zeros(off, np.float32), x]))[off:]
        if variant == "fused":
            out = dev(np.array([old, old, old], np.float32))
            red.sum_max_min_f32(xd, out, accum=accum)
            got = host(out)[("sum", "max", "min").index(op)]
        else:
            out = dev(np.array([old], np.float32))
            getattr(red, op + "_f32" + variant)(xd, out, accum=accum)
            got = host(out)[0]
        if op == "sum":
            s, a = orc.sum_f32(x, accum, old)
            check_sum(got, s, a, what)
        else:
            check_exact(got, getattr(orc, op + "_f32")(x, accum, old), what,
                        bool(has_both_zeros(x, np.float32(old), accum)))


def test_random_rows(red, orc):
    rng = np.random.default_rng(9002)
    for case in range(60):
        n = log_uniform(rng, 1, 20000)
        rows = max(1, min(log_uniform(rng, 1, 200000), 4_000_000 // max(n, 1)))
        ld = n + int(rng.integers(0, 2)) * int(rng.integers(0, 9))
        off = int(rng.integers(0, 4))
        op = ("sum", "max", "min")[case % 3]
        accum = bool(rng.integers(0, 2))
        what = "rows case %d rows=%d n=%d ld=%d off=%d op=%s accum=%s" % (
            case, rows, n, ld, off, op, accum)
        say(what)
        x = np.full((rows, ld), np.nan, np.float32)
        x[:, :n] = rng.uniform(-1, 1, (rows, n)).astype(np.float32)
        old = rng.uniform(-3, 3, rows).astype(np.float32)
        xd = upload_padded(x, off)
        out = dev(old.copy())
        getattr(red, op + "_rows_f32")(xd, out, n=n, accum=accum)
        got = host(out)
        if op == "sum":
            if n <= 64:
                want = orc.rows_page_sum_f32(x, rows, n, ld, accum, old)
                assert (got.view(np.uint32) == want.view(np.uint32)).all(), what
            s, a = orc.rows_sum_f32(x, rows, n, ld, accum, old)
            check_sums(got, s, a, what)
        else:
            want = getattr(orc, "rows_%s_f32" % op)(x, rows, n, ld, accum, old)
            check_extremes(got, want, has_both_zeros(x[:, :n], old, accum, axis=1), what)


COL_KINDS = ["f32", "bf16", "f16", "i32", "sum", "max", "min"]


def test_random_columns(red, orc):
    rng = np.random.default_rng(9003)
    for case in range(70):
        kind = COL_KINDS[case % len(COL_KINDS)]
        C = log_uniform(rng, 1, 40000)
        # products are held to their tolerance for R <= 4096
        rmax = 20000 if kind in ("i32", "sum", "max", "min") else 4096
        R = max(1, min(log_uniform(rng, 1, rmax), 3_000_000 // C))
        ld = C + int(rng.integers(0, 2)) * int(rng.integers(0, 17))
        off = int(rng.integers(0, 4))
        what = "cols case %d kind=%s R=%d C=%d ld=%d off=%d" % (case, kind, R, C, ld, off)
        say(what)
        if kind == "i32":
            src = rng.integers(-(2 ** 31), 2 ** 31, (R, ld), dtype=np.int64).astype(np.int32)
            flat = np.zeros(R * ld + off + 8, np.int32)
            flat[off:off + R * ld] = src.reshape(-1)
            sd = dev(flat)[off:off + R * ld].view(R, ld)
            out = torch.zeros(C, dtype=torch.int32, device="cuda")
            red.colprod_i32(sd, out, C=C)
            want = orc.colprod_i32(src, R, C, ld)
            assert (host(out) == want).all(), what
            continue
        # factors near 1, so that no product leaves the normal range of fp16
        lo, hi = (0.75, 1.25) if R <= 16 else ((0.99, 1.01) if R <= 2000 else (0.999, 1.001))
        vals = np.full((R, ld), np.nan, np.float32)
        if kind in ("sum", "max", "min"):
            vals[:, :C] = rng.uniform(-1, 1, (R, C)).astype(np.float32)
        else:
            vals[:, :C] = rng.uniform(lo, hi, (R, C)).astype(np.float32)
        if C >= 3 and case % 2 == 0:
            # Signed zeros in three columns: for sum / max / min a column of
            # zeros of random signs, one of -0 only and one of +0 only; for
            # products one -0 factor, one +0 factor and a -0 factor in a
            # column of negated values (the product's sign is the XOR).
            j = rng.choice(C, 3, replace=False)
            if kind in ("sum", "max", "min"):
                vals[:, j[0]] = np.where(rng.random(R) < 0.5, 0.0, -0.0)
                vals[:, j[1]] = -0.0
                vals[:, j[2]] = 0.0
            else:
                vals[rng.integers(0, R), j[0]] = -0.0
                vals[rng.integers(0, R), j[1]] = 0.0
                vals[:, j[2]] = -vals[:, j[2]]
                vals[rng.integers(0, R), j[2]] = -0.0
        if kind in ("f32", "sum", "max", "min"):
            sd = upload_padded(vals, off)
            out = torch.zeros(C, dtype=torch.float32, device="cuda")
            if kind == "f32":
                red.colprod_f32(sd, out, C=C)
                check_rel(host(out), orc.colprod_f32(vals, R, C, ld), COLPROD_F32_TOL, what)
            else:
                accum = bool(rng.integers(0, 2))
                old = rng.uniform(-3, 3, C).astype(np.float32)
                out = dev(old.copy())
                getattr(red, kind + "_cols_f32")(sd, out, C=C, accum=accum)
                got = host(out)
                if kind == "sum":
                    s, a = orc.cols_sum_f32(vals, R, C, ld, accum, old)
                    check_sums(got, s, a, what)
                else:
                    want = getattr(orc, "cols_%s_f32" % kind)(vals, R, C, ld, accum, old)
                    both = has_both_zeros(valid_region(vals, R, C, ld), old, accum, axis=0)
                    check_extremes(got, want, both, what)
        else:
            tdt = torch.bfloat16 if kind == "bf16" else torch.float16
            h = torch.from_numpy(vals).to(tdt)           # exact RNE conversion; NaN padding stays NaN
            bits = h.view(torch.int16).numpy().view(np.uint16)
            flat = np.zeros(R * ld + off + 8, np.uint16)
            flat[off:off + R * ld] = bits.reshape(-1)
            sd = dev(flat.view(np.int16))[off:off + R * ld].view(R, ld).view(tdt)
            out = torch.zeros(C, dtype=tdt, device="cuda")
            getattr(red, "colprod_" + kind)(sd, out, C=C)
            got = host(out.float())
            want = getattr(orc, "colprod_" + kind)(bits, R, C, ld)
            check_rel(got, want, COLPROD_16_TOL, what)


def _at(a, o):
    flat = np.zeros(a.size + o + 8, a.dtype)
    flat[o:o + a.size] = a.reshape(-1)
    return dev(flat)[o:o + a.size].view(*a.shape)


def column_case(red, orc, rng, kind, R, C, ld, off, doff, what):
    """One column call of `kind` on a seeded (R, ld) tile starting `off`
    elements into its buffer, dst `doff` elements in; checked against the
    oracle."""
    if kind == "i32":
        src = rng.integers(-(2 ** 31), 2 ** 31, (R, ld), dtype=np.int64).astype(np.int32) | 1
        out = torch.zeros(C + doff, dtype=torch.int32, device="cuda")[doff:]
        red.colprod_i32(_at(src, off), out, C=C)
        assert (host(out) == orc.colprod_i32(src, R, C, ld)).all(), what
    elif kind in ("i16", "u16", "u32"):
        # odd values: the products modulo 2^16 / 2^32 stay odd, so every row counts
        w = 32 if kind == "u32" else 16
        bits = (rng.integers(0, 1 << w, (R, ld), dtype=np.uint64) | 1).astype(
            np.uint32 if w == 32 else np.uint16)
        signed = np.int32 if w == 32 else np.int16
        out = torch.zeros(C + doff, dtype=torch.int32 if w == 32 else torch.int16,
                          device="cuda")[doff:]
        getattr(red, "colprod_" + kind)(_at(bits.view(signed), off), out, C=C)
        got = host(out).view(np.uint32 if w == 32 else np.uint16)
        want = (orc.colprod_u32 if w == 32 else orc.colprod_u16)(bits, R, C, ld)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "%s: column %d" % (what, bad[0])
    elif kind in ("sum", "max", "min"):
        x = rng.uniform(-1, 1, (R, ld)).astype(np.float32)
        x[:, C:] = np.nan
        accum = bool(rng.integers(0, 2))
        old = rng.uniform(-3, 3, C).astype(np.float32)
        out = _at(old.copy(), doff)
        getattr(red, kind + "_cols_f32")(_at(x, off), out, C=C, accum=accum)
        got = host(out)
        if kind == "sum":
            s, a = orc.cols_sum_f32(x, R, C, ld, accum, old)
            check_sums(got, s, a, what)
        else:
            want = getattr(orc, "cols_%s_f32" % kind)(x, R, C, ld, accum, old)
            check_extremes(got, want, has_both_zeros(x[:, :C], old, accum, axis=0), what)
    else:
        rare = 2e-5 if kind == "f16" else 2e-4
        u = rng.random((R, ld))
        x = np.where(u < rare, 2.0, np.where(u < 2 * rare, 0.5, 1.0))
        x = (x * np.where(rng.random((R, ld)) < 0.5, -1.0, 1.0)).astype(np.float32)
        x[:, C:] = np.nan
        if kind == "f32":
            out = torch.zeros(C + doff, dtype=torch.float32, device="cuda")[doff:]
            red.colprod_f32(_at(x, off), out, C=C)
            check_rel(host(out), orc.colprod_f32(x, R, C, ld), COLPROD_F32_TOL, what)
        else:
            tdt = torch.bfloat16 if kind == "bf16" else torch.float16
            bits = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
            out = torch.zeros(C + doff, dtype=tdt, device="cuda")[doff:]
            getattr(red, "colprod_" + kind)(_at(bits.view(np.int16), off).view(tdt), out, C=C)
            want = getattr(orc, "colprod_" + kind)(bits, R, C, ld)
            check_rel(host(out.float()), want, COLPROD_16_TOL, what)


def test_random_column_paths(red, orc):
    """Column cases drawn per layout class: narrow rows (16-byte vectors or
    elements), short and wide tiles (several blocks per workgroup, wide
    strips), rows shared by several workgroups, and general shapes; with a
    random source and destination offset and, for the column sum / max /
    min, random accum.  Products over long columns use factors +-1 with
    rare +-2 and +-0.5 (exact in any order)."""
    rng = np.random.default_rng(9004)
    kinds = ["f32", "i32", "bf16", "f16", "sum", "max", "min"]
    for case in range(84):
        kind = kinds[case % 7]
        layout = (case // 7) % 4
        if layout == 0:
            C, R = log_uniform(rng, 1, 127), log_uniform(rng, 1, 300000)
        elif layout == 1:
            C, R = log_uniform(rng, 60000, 2_500_000), log_uniform(rng, 1, 24)
        elif layout == 2:
            C, R = log_uniform(rng, 64, 5000), log_uniform(rng, 100, 40000)
        else:
            C, R = log_uniform(rng, 1, 40000), log_uniform(rng, 1, 5000)
        ld = C + int(rng.integers(0, 2)) * int(rng.integers(0, 9))
        R = max(1, min(R, 6_000_000 // ld))
        off = int(rng.integers(0, 2)) * int(rng.integers(0, 4))
        doff = int(rng.integers(0, 2)) * int(rng.integers(0, 3))
        what = "col path case %d kind=%s R=%d C=%d ld=%d off=%d doff=%d" % (
            case, kind, R, C, ld, off, doff)
        say(what)
        column_case(red, orc, rng, kind, R, C, ld, off, doff, what)


def test_random_overrun_tiles(red, orc):
    """Column cases whose workgroups overrun one, two or three multiples of
    256 by at most 64 (blocks of 64 four-byte or 128 two-byte columns, 16
    row groups each), rows on 128-byte lines (strides rounded up to 128
    bytes, offsets of whole lines), row counts from one chunk of 128 to
    many, and random dst offsets and accum."""
    rng = np.random.default_rng(9005)
    kinds = ["f32", "i32", "bf16", "f16", "sum", "max", "min"]
    for case in range(28):
        kind = kinds[case % 7]
        es = 2 if kind in ("bf16", "f16") else 4
        cols = 256 // es
        blocks = 256 * int(rng.integers(1, 4)) + int(rng.integers(1, 65))
        C = (blocks - 1) * cols + int(rng.integers(1, cols + 1))
        line = 128 // es
        ld = -(-C // line) * line + line * int(rng.integers(0, 2))
        R = max(1, min(log_uniform(rng, 1, 3000), 16_000_000 // ld))
        off = line * int(rng.integers(0, 3))
        doff = int(rng.integers(0, 2)) * int(rng.integers(0, 3))
        what = "overrun case %d kind=%s R=%d C=%d (%d blocks) ld=%d off=%d doff=%d" % (
            case, kind, R, C, blocks, ld, off, doff)
        say(what)
        column_case(red, orc, rng, kind, R, C, ld, off, doff, what)


def test_random_multiblock_tiles(red, orc):
    """Short, wide tiles on 16-byte aligned rows whose workgroups hold
    several column blocks (4 row groups each), a row group per block, or
    wide strips, with a ragged last block for every element type: the
    block counts are drawn from 1021 to 20000 (the 4-row-group layout
    below 4081 at 256 CUs), so the last workgroup often holds whole blocks
    beside the ragged one."""
    rng = np.random.default_rng(9006)
    kinds = ["f32", "i32", "bf16", "f16", "i16", "u16", "u32", "sum", "max", "min"]
    for case in range(60):
        kind = kinds[case % len(kinds)]
        es = 2 if kind in ("bf16", "f16", "i16", "u16") else 4
        cols = 256 // es
        blocks = log_uniform(rng, 1021, 20000)
        C = (blocks - 1) * cols + int(rng.integers(1, cols))      # ragged last block
        vec = 16 // es
        ld = -(-C // vec) * vec + vec * int(rng.integers(0, 2))    # rows on 16-byte boundaries
        R = max(1, min(log_uniform(rng, 1, 24), 8_000_000 // ld))
        off = vec * int(rng.integers(0, 2))
        doff = int(rng.integers(0, 2)) * int(rng.integers(0, 3))
        what = "multiblock case %d kind=%s R=%d C=%d (%d blocks) ld=%d off=%d doff=%d" % (
            case, kind, R, C, blocks, ld, off, doff)
        say(what)
        column_case(red, orc, rng, kind, R, C, ld, off, doff, what)


SPECIALS = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 2.0 ** -140, -(2.0 ** -140), 1e30, -1e30],
                    np.float32)


def _special_values(rng, shape, p):
    """Uniform values with a fraction p replaced by NaN, infinities, zeros of
    both signs, subnormals and large values; or zeros only, of random signs;
    or -0 only with a few of those specials."""
    kind = int(rng.integers(0, 3))
    if kind == 1:
        return np.where(rng.random(shape) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    x = (np.full(shape, -0.0, np.float32) if kind == 2
         else rng.uniform(-1, 1, shape).astype(np.float32))
    m = rng.random(shape) < p
    x[m] = SPECIALS[rng.integers(0, SPECIALS.size, int(m.sum()))]
    return x


def test_random_special_values(red, orc, monkeypatch):
    """Special values through random shapes of the row and column
    reductions, the column products and every 1-D entry point, under the
    launch plans of random device sizes (RED_TEST_CUS from 1 to 4096, or
    the device's own count), each checked strictly: NaN for NaN, the same
    infinity, the sign of every zero (sums: -0 only when every term is -0;
    products: the XOR of the factors' signs; max / min: either zero only
    when both occur)."""
    rng = np.random.default_rng(9007)
    for case in range(90):
        if rng.random() < 0.5:
            monkeypatch.delenv("RED_TEST_CUS", raising=False)
            cus = 0
        else:
            cus = log_uniform(rng, 1, 4096)
            monkeypatch.setenv("RED_TEST_CUS", str(cus))
        p = float(np.exp(rng.uniform(np.log(1e-5), np.log(0.05))))
        part = case % 3
        if part == 0:  # rows
            op = ("sum", "max", "min")[(case // 3) % 3]
            n = log_uniform(rng, 1, 5000)
            ld = n + int(rng.integers(0, 2)) * int(rng.integers(0, 9))
            rows = max(1, min(log_uniform(rng, 1, 200_000), 4_000_000 // ld))
            off = int(rng.integers(0, 4))
            accum = bool(rng.integers(0, 2))
            x = np.full((rows, ld), np.nan, np.float32)
            x[:, :n] = _special_values(rng, (rows, n), p)
            old = _special_values(rng, rows, 0.2)
            what = "special rows case %d %s rows=%d n=%d ld=%d off=%d accum=%d p=%.1e cus=%d" % (
                case, op, rows, n, ld, off, accum, p, cus)
            say(what)
            out = dev(old.copy())
            getattr(red, op + "_rows_f32")(upload_padded(x, off), out, n=n, accum=accum)
            got = host(out)
            if op == "sum":
                s, a = orc.rows_sum_f32(x, rows, n, ld, accum, old)
                check_sums(got, s, a, what)
            else:
                want = getattr(orc, "rows_%s_f32" % op)(x, rows, n, ld, accum, old)
                both = has_both_zeros(valid_region(x, rows, n, ld), old, accum, axis=1)
                check_extremes(got, want, both, what)
        elif part == 1:  # columns
            kind = ("f32", "bf16", "f16", "sum", "max", "min")[(case // 3) % 6]
            C = log_uniform(rng, 1, 300_000)
            ld = C + int(rng.integers(0, 2)) * int(rng.integers(0, 9))
            R = max(1, min(log_uniform(rng, 1, 4000), 4_000_000 // ld))
            off = int(rng.integers(0, 2)) * int(rng.integers(0, 4))
            what = "special cols case %d %s R=%d C=%d ld=%d off=%d p=%.1e cus=%d" % (
                case, kind, R, C, ld, off, p, cus)
            say(what)
            if kind in ("sum", "max", "min"):
                x = _special_values(rng, (R, ld), p)
                accum = bool(rng.integers(0, 2))
                old = _special_values(rng, C, 0.2)
                out = dev(old.copy())
                getattr(red, kind + "_cols_f32")(_at(x, off), out, C=C, accum=accum)
                got = host(out)
                if kind == "sum":
                    s, a = orc.cols_sum_f32(x, R, C, ld, accum, old)
                    check_sums(got, s, a, what)
                else:
                    want = getattr(orc, "cols_%s_f32" % kind)(x, R, C, ld, accum, old)
                    both = has_both_zeros(valid_region(x, R, C, ld), old, accum, axis=0)
                    check_extremes(got, want, both, what)
            else:
                # +-1 with rare +-2 / +-0.5, and +-0, NaN, +-inf: every order
                # gives the same product, bit for bit
                u = rng.random((R, ld))
                x = np.where(u < 2e-4, 2.0, np.where(u < 4e-4, 0.5, 1.0))
                x = (x * np.where(rng.random((R, ld)) < 0.5, -1.0, 1.0)).astype(np.float32)
                m = rng.random((R, ld)) < p
                sp = np.array([0.0, -0.0, np.nan, np.inf, -np.inf], np.float32)
                x[m] = sp[rng.integers(0, sp.size, int(m.sum()))]
                if kind == "f32":
                    out = torch.zeros(C, dtype=torch.float32, device="cuda")
                    red.colprod_f32(_at(x, off), out, C=C)
                    got, want = host(out), orc.colprod_f32(x, R, C, ld)
                else:
                    tdt = torch.bfloat16 if kind == "bf16" else torch.float16
                    bits = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
                    out = torch.zeros(C, dtype=tdt, device="cuda")
                    getattr(red, "colprod_" + kind)(_at(bits.view(np.int16), off).view(tdt), out, C=C)
                    got = host(out.float())
                    want = np.asarray(getattr(orc, "colprod_" + kind)(bits, R, C, ld), np.float32)
                g, w = np.asarray(got, np.float32), np.asarray(want, np.float32)
                same = (g.view(np.uint32) == w.view(np.uint32)) | (np.isnan(g) & np.isnan(w))
                assert same.all(), "%s: column %d got %r want %r" % (
                    what, int(np.nonzero(~same)[0][0]), g[~same][0], w[~same][0])
        else:  # 1-D
            n = log_uniform(rng, 1, 4_000_000)
            off = int(rng.integers(0, 4))
            accum = bool(rng.integers(0, 2))
            x = _special_values(rng, n, p)
            old = np.float32(SPECIALS[rng.integers(0, SPECIALS.size)] if rng.random() < 0.3
                             else rng.uniform(-3, 3))
            what = "special 1-D case %d n=%d off=%d accum=%d p=%.1e old=%r cus=%d" % (
                case, n, off, accum, p, float(old), cus)
            say(what)
            xd = upload_padded(x.reshape(1, n), off).view(n)
            s, a = orc.sum_f32(x, accum, float(old))
            both = bool(has_both_zeros(x, np.array([old]), accum))
            res = {}
            for op in ("sum", "max", "min"):
                out = dev(np.array([old], np.float32))
                getattr(red, op + "_f32")(xd, out, accum=accum)
                res[op] = host(out)[0]
            check_sum(res["sum"], s, a, what + " sum")
            check_exact(res["max"], orc.max_f32(x, accum, float(old)), what + " max", both)
            check_exact(res["min"], orc.min_f32(x, accum, float(old)), what + " min", both)
            want3 = np.array([res["sum"], res["max"], res["min"]], np.float32)
            for fn in ("sum_max_min_f32", "sum_max_min_f32_noalloc"):
                out3 = dev(np.array([old, old, old], np.float32))
                try:
                    getattr(red, fn)(xd, out3, accum=accum)
                except red.ReduceError as e:  # partials past the static buffer
                    assert fn.endswith("noalloc") and e.status == red.RED_ERR_SCRATCH and cus > 1365, what
                    continue
                g = host(out3)
                same = (g.view(np.uint32) == want3.view(np.uint32)) | (np.isnan(g) & np.isnan(want3))
                assert same.all(), (what, fn, g, want3)
            for op in ("sum", "max", "min"):
                out = dev(np.array([old], np.float32))
                getattr(red, op + "_f32_atomic")(xd, out, accum=accum)
                got = host(out)[0]
                if op == "sum":
                    check_sum(got, s, a, what + " atomic sum")
                else:
                    check_exact(got, getattr(orc, op + "_f32")(x, accum, float(old)),
                                what + " atomic " + op, both)
