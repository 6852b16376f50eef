"""GPU parity of the column reductions on narrow rows, on short and wide
tiles, and of the second pass over many row slices.

Rows narrower than 256 bytes take the narrow-row kernel: a workgroup
reads whole rows (W units per row, 256 / W rows per step) and walks its
sweeps grid-stride.  The unit is a 16-byte vector when the start, stride
and valid width are multiples of 16 bytes, else one element.  The cases
cover every vector width W from 1 to 15 for 4-byte and 2-byte elements,
element rows of 1 to 127 elements with misaligned starts, padding past C
(filled with NaN, never read), row counts that end inside a step and
inside a sweep, and counts large enough for hundreds of workgroups and a
second pass.  Products over long columns use factors +-1 with rare +-2
and +-0.5, so that the exact product stays in range and every order of
multiplication gives it exactly.

Tiles whose workgroups (one per 16-row-group block, or per four blocks of
4 row groups) overrun a multiple of the 256 CUs by at most a quarter of it
and whose rows lie on 128-byte lines split their rows into 6 shares and
take the second pass, so that the last round of workgroups is short; each
share needs at least one 32 KiB chunk per workgroup.  The cases cover block counts just over one, two and three
multiples of 256 and over 1024 (4 row groups per block), 6 to 24 chunks,
ragged last blocks, unaligned destinations and accum, and tiles that miss
one of the conditions and keep one share.

Rows that are not 16-byte aligned (an odd stride, a stride of 2 or 3
elements past a multiple of four, a misaligned start) meet each column
block at an offset within a 16-byte vector that depends on the row (on
every fourth or eighth row the same).  The cases cover every such offset
for 4-byte and 2-byte elements, ragged last blocks, a block count of one,
leftover rows, row splits, NaN padding, accum and misaligned
destinations.

Short, wide tiles (thousands of 256-byte column blocks) give a workgroup
several adjacent column blocks with 4 or 1 row groups each, and with
more blocks still a wide strip in which each lane reads 2, 4 or 8
vectors of a row; the cases cover each, with a block count that leaves
the last workgroup part empty, a ragged last block, unaligned rows, and
aligned and misaligned destinations.

The second pass spreads each column's S partial rows over the threads of
a workgroup; the cases below put S from 2 to a few hundred against column
counts from 1 to a few thousand on the column-block and narrow-row
kernels."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (COLPROD_16_TOL, COLPROD_F32_TOL, check_extremes, check_rel, check_sums,
                         dev, has_both_zeros, host, say, valid_region)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def pow2_factors(seed, shape, rare):
    """+-1 with rare +-2 and +-0.5 (probability `rare` each)."""
    rng = np.random.default_rng(seed)
    u = rng.random(shape)
    v = np.where(u < rare, 2.0, np.where(u < 2 * rare, 0.5, 1.0))
    v = v * np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    return v.astype(np.float32)


def tile_f32(seed, R, C, ld, kind, rare=2e-4):
    x = np.full((R, ld), np.nan, np.float32)
    if kind == "prod":
        x[:, :C] = pow2_factors(seed, (R, C), rare)
    else:
        x[:, :C] = workloads.uniform_f32(seed, R * C).reshape(R, C)
    return x


def dev_at(a, off):
    """Upload a host tile so that it starts `off` elements into a larger
    device buffer (off = 0: the buffer's own 256-byte-aligned start)."""
    flat = np.zeros(a.size + off, a.dtype)
    flat[off:] = a.reshape(-1)
    return dev(flat)[off:].view(*a.shape)


def colprod_case(red, orc, kind, R, C, ld, seed, off=0, dst_off=0):
    what = "colprod %s R=%d C=%d ld=%d off=%d dst_off=%d" % (kind, R, C, ld, off, dst_off)
    say(what)
    if kind == "i32":
        # odd factors: the product mod 2^32 stays odd, so every row counts
        src = workloads.integers_i32(seed, R * ld, -(2 ** 31), 2 ** 31).reshape(R, ld) | 1
        out = torch.zeros(C + dst_off, dtype=torch.int32, device="cuda")[dst_off:]
        red.colprod_i32(dev_at(src, off), out, C=C)
        got = host(out)
        want = orc.colprod_i32(src, R, C, ld)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "%s: column %d" % (what, bad[0])
        return
    # binary16 keeps exponents -14..15: long columns get rarer powers of two
    rare = 2e-5 if kind == "f16" and R > 4096 else 2e-4
    x = tile_f32(seed, R, C, ld, "prod", rare)
    if kind == "f32":
        out = torch.zeros(C + dst_off, dtype=torch.float32, device="cuda")[dst_off:]
        red.colprod_f32(dev_at(x, off), out, C=C)
        check_rel(host(out), orc.colprod_f32(x, R, C, ld), COLPROD_F32_TOL, what)
        return
    bits = (workloads.to_f16_bits if kind == "f16" else workloads.to_bf16_bits)(x.reshape(-1))
    bits = bits.reshape(R, ld)
    tdt = torch.float16 if kind == "f16" else torch.bfloat16
    out = torch.zeros(C + dst_off, dtype=tdt, device="cuda")[dst_off:]
    getattr(red, "colprod_" + kind)(dev_at(bits.view(np.int16), off).view(tdt), out, C=C)
    want = (orc.colprod_f16 if kind == "f16" else orc.colprod_bf16)(bits, R, C, ld)
    check_rel(host(out.float()), want, COLPROD_16_TOL, what)


def cols_case(red, orc, op, R, C, ld, accum, seed, off=0, dst_off=0):
    what = "cols %s R=%d C=%d ld=%d accum=%d off=%d dst_off=%d" % (op, R, C, ld, accum, off, dst_off)
    say(what)
    x = tile_f32(seed, R, C, ld, op)
    old = workloads.uniform_f32(seed + 1, C, -3.0, 3.0)
    out = dev_at(old.copy(), dst_off)
    getattr(red, op + "_cols_f32")(dev_at(x, off), out, C=C, accum=accum)
    got = host(out)
    if op == "sum":
        s, a = orc.cols_sum_f32(x, R, C, ld, accum, old)
        check_sums(got, s, a, what)
    else:
        want = getattr(orc, "cols_%s_f32" % op)(x, R, C, ld, accum, old)
        check_extremes(got, want, has_both_zeros(valid_region(x, R, C, ld), old, accum, axis=0),
                       what)


# (W vectors per row, valid vectors, rows): rows end inside a step, inside
# a sweep, and after many sweeps (S up to twice the compute units).
NARROW = [
    (1, 1, 1), (1, 1, 255), (1, 1, 2049), (1, 1, 600_000),
    (2, 2, 130), (2, 1, 40_000),
    (3, 3, 85), (3, 2, 3 * 2048 + 5),
    (4, 4, 64 * 8 + 63), (4, 3, 200_000),
    (5, 5, 51 * 8 * 3 + 50), (6, 6, 42 * 8 * 7), (6, 1, 70_000),
    (7, 7, 36 * 8 * 5 + 1), (8, 8, 100_001), (8, 5, 9),
    (9, 9, 28 * 8 * 3 + 27), (10, 10, 25 * 8 + 24), (11, 7, 23 * 8 * 2 + 1),
    (12, 12, 21 * 8 * 9 + 20), (13, 13, 19 * 8 * 4 + 3), (14, 14, 40_000),
    (15, 15, 17 * 8 * 11 + 16), (15, 2, 17),
]


@pytest.mark.parametrize("kind", ["f32", "i32"])
@pytest.mark.parametrize("W,valid,R", NARROW)
def test_narrow_4byte(red, orc, kind, W, valid, R):
    colprod_case(red, orc, kind, R, 4 * valid, 4 * W, 500 + W)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("W,valid,R", NARROW)
def test_narrow_2byte(red, orc, kind, W, valid, R):
    colprod_case(red, orc, kind, min(R, 60_000), 8 * valid, 8 * W, 600 + W)


@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("W,valid,R", [(1, 1, 300_001), (4, 4, 5000), (5, 3, 70_000),
                                       (8, 8, 63), (15, 15, 100_000)])
@pytest.mark.parametrize("accum", [0, 1])
def test_narrow_cols(red, orc, op, W, valid, R, accum):
    cols_case(red, orc, op, R, 4 * valid, 4 * W, accum, 700 + W)


# Narrow rows read in elements (rows narrower than 256 bytes whose start,
# stride or valid width is not a multiple of 16 bytes): (R, C, ld, off).
NARROW_ELEM = [
    (1, 1, 1, 0), (100_000, 15, 15, 0), (70_000, 1, 3, 0), (5000, 63, 63, 1),
    (3001, 33, 40, 3), (40_000, 16, 16, 2), (20_000, 30, 32, 0), (257, 7, 9, 1),
    (300_000, 2, 2, 0), (12_345, 40, 60, 0),
]


@pytest.mark.parametrize("kind", ["f32", "i32", "f16", "bf16"])
@pytest.mark.parametrize("R,C,ld,off", NARROW_ELEM)
def test_narrow_elements(red, orc, kind, R, C, ld, off):
    colprod_case(red, orc, kind, min(R, 60_000) if kind in ("f16", "bf16") else R,
                 C, ld, 1300 + C, off)


NARROW16_ELEM = [(9999, 127, 127, 0), (4000, 100, 120, 1), (50_000, 9, 9, 0)]


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("R,C,ld,off", NARROW16_ELEM)
def test_narrow_elements_2byte(red, orc, kind, R, C, ld, off):
    colprod_case(red, orc, kind, R, C, ld, 1400 + C, off)


@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("R,C,ld,off", [(100_000, 15, 15, 0), (5000, 63, 63, 1),
                                        (3001, 33, 40, 3), (300_000, 2, 2, 0)])
@pytest.mark.parametrize("accum", [0, 1])
def test_narrow_elements_cols(red, orc, op, R, C, ld, off, accum):
    cols_case(red, orc, op, R, C, ld, accum, 1500 + C, off)


# Second pass: (R, C, ld) on the column-block kernel (rows of 256 bytes or
# more) and on both forms of the narrow-row kernel, spanning S from 2 to a
# few hundred and column counts on both sides of each power of two.
FINISH = [
    (4096, 1, 1), (100_000, 1, 3), (50_000, 3, 5), (70_000, 17, 17),
    (40_000, 64, 65), (20_000, 255, 255), (8192, 257, 257), (5000, 1000, 1001),
    (3000, 4099, 4099), (100_000, 16, 16), (60_000, 64, 64),
]


@pytest.mark.parametrize("R,C,ld", FINISH)
@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_second_pass_products(red, orc, kind, R, C, ld):
    colprod_case(red, orc, kind, R, C, ld, 800 + C)


@pytest.mark.parametrize("R,C,ld", FINISH)
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_second_pass_cols(red, orc, op, R, C, ld):
    cols_case(red, orc, op, R, C, ld, 1, 900 + C)


# Short, wide tiles: (R, C, ld).  For 4-byte elements, 1021 or more
# column blocks give 4 row groups per block, 4081 or more give 1; with
# 16-byte aligned rows, 256 strips of 32, 64 or 128 whole blocks (8 K, 16 K
# or 32 K blocks) give the wide-strip kernel 2, 4 or 8 vectors per lane,
# the remaining blocks going to one row group per block.
WIDE = [
    (37, 65536, 65536), (5, 131172, 131172), (7, 70001, 70002), (33, 80000, 80001),
    (3, 300_000, 300_000), (16, 262_144, 262_144), (1, 1_000_003, 1_000_004),
    (9, 300_001, 300_005), (2, 400_000, 400_001),
    (3, 2_100_001, 2_100_004), (5, 1_048_576, 1_048_576), (2, 1_600_000, 1_600_000),
    (17, 600_000, 600_000),
]


@pytest.mark.parametrize("R,C,ld", WIDE)
@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_wide_4byte(red, orc, kind, R, C, ld):
    colprod_case(red, orc, kind, R, C, ld, 1000 + R)


# 2-byte elements: the same block counts, of 128 columns: 1021 or more
# give 4 row groups per block, 4081 or more give 1, and 256 strips of
# 32, 64 or 128 whole blocks (8 K, 16 K or 32 K blocks) the wide-strip
# kernel.
WIDE16 = [(20, 262_144, 262_144), (6, 270_000, 270_003), (4, 1_100_000, 1_100_008),
          (11, 1_050_001, 1_050_001), (3, 4_200_005, 4_200_008), (2, 2_400_000, 2_400_000),
          (5, 600_000, 600_000)]

# 4 row groups per block on 16-byte aligned rows with a ragged last block
# (read in elements) in a workgroup whose other blocks are whole (read in
# vectors).  A workgroup of 2-byte elements combines 4 x 128 values on 256
# threads, so most of a block's values are combined by threads that read
# another block; each must place them by that block's layout.  (Block
# counts 1846, 4052, 2003, 1094, 3002: 2, 4, 3, 2 and 2 blocks in the last
# workgroup.)
WIDE16_RAGGED = [(2, 236_272, 236_272), (1, 518_552, 518_552), (7, 256_356, 256_360),
                 (33, 140_000, 140_000), (3, 384_192, 384_192)]


@pytest.mark.parametrize("R,C,ld", WIDE16)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_wide_2byte(red, orc, kind, R, C, ld):
    colprod_case(red, orc, kind, R, C, ld, 1100 + R)


@pytest.mark.parametrize("R,C,ld", WIDE16_RAGGED)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("dst_off", [0, 2])
def test_wide_2byte_ragged(red, orc, kind, R, C, ld, dst_off):
    colprod_case(red, orc, kind, R, C, ld, 1150 + R, 0, dst_off)


@pytest.mark.parametrize("R,C,ld", [(37, 65536, 65536), (7, 70001, 70002),
                                    (3, 300_000, 300_000), (9, 300_001, 300_005),
                                    (3, 2_100_001, 2_100_004), (2, 1_600_000, 1_600_000)])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("accum", [0, 1])
def test_wide_cols(red, orc, op, R, C, ld, accum):
    cols_case(red, orc, op, R, C, ld, accum, 1200 + R)


# The wide-strip kernel stores whole 16-byte vectors when dst is 16-byte
# aligned and single elements otherwise: both, with and without accum.
@pytest.mark.parametrize("dst_off", [0, 1, 3])
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16", "f16"])
def test_wide_dst_alignment(red, orc, kind, dst_off):
    R, C, ld = (3, 2_100_001, 2_100_004) if kind in ("f32", "i32") else (3, 4_200_005, 4_200_008)
    colprod_case(red, orc, kind, R, C, ld, 1600, 0, dst_off)


@pytest.mark.parametrize("dst_off", [0, 1])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("accum", [0, 1])
def test_wide_cols_dst_alignment(red, orc, op, accum, dst_off):
    cols_case(red, orc, op, 5, 1_048_576, 1_048_576, accum, 1700, 0, dst_off)


# (rows, columns, stride): 257 to 769 blocks of 64 (4-byte) columns on
# 128-byte lines, with rows spanning 6 to 24 chunks and ragged last blocks;
# 1100 and 2100 blocks of 4 row groups; then tiles that keep one share:
# fewer than six chunks, unaligned rows, a last round more than a quarter
# full.
OVERRUN = [
    (1000, 16448, 16448), (800, 17405, 17408), (1500, 33000, 33024), (3000, 36800, 36800),
    (770, 49153, 49184), (200, 70400, 70400), (300, 134390, 134400),
    (129, 20032, 20032), (64, 19008, 19008), (2, 49216, 49216),
    (1000, 16448, 16451), (127, 25000, 25001), (400, 24640, 24640), (2, 65000, 65024),
]


@pytest.mark.parametrize("R,C,ld", OVERRUN)
@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_overrun_4byte(red, orc, kind, R, C, ld):
    colprod_case(red, orc, kind, R, C, ld, 1800 + R)


# 2-byte elements: 257 to 782 blocks of 128 columns on 128-byte lines, 1100
# blocks of 4 row groups, and one unaligned tile.
OVERRUN16 = [(1000, 32896, 32896), (777, 40000, 40000), (3000, 70001, 70016),
             (3, 100000, 100032), (300, 140800, 140800), (500, 40000, 40001)]


@pytest.mark.parametrize("R,C,ld", OVERRUN16)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_overrun_2byte(red, orc, kind, R, C, ld):
    colprod_case(red, orc, kind, R, C, ld, 1900 + R)


# off = 32 keeps 128-byte lines; off = 1 moves the rows off them.
@pytest.mark.parametrize("R,C,ld,off", [(1000, 16448, 16448, 0), (800, 17405, 17408, 32),
                                        (1500, 33000, 33024, 0), (2, 49216, 49216, 0),
                                        (3000, 36800, 36800, 0), (770, 49153, 49184, 1),
                                        (200, 70400, 70400, 0)])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("accum", [0, 1])
def test_overrun_cols(red, orc, op, R, C, ld, off, accum):
    cols_case(red, orc, op, R, C, ld, accum, 2000 + R, off)


@pytest.mark.parametrize("dst_off", [1, 3])
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16", "f16"])
def test_overrun_dst_alignment(red, orc, kind, dst_off):
    R, C, ld = (700, 20000, 20000) if kind in ("f32", "i32") else (700, 40000, 40000)
    colprod_case(red, orc, kind, R, C, ld, 2100, 0, dst_off)


@pytest.mark.parametrize("dst_off", [0, 1])
@pytest.mark.parametrize("accum", [0, 1])
def test_overrun_cols_dst_alignment(red, orc, accum, dst_off):
    cols_case(red, orc, "sum", 1000, 16448, 16448, accum, 2200, 0, dst_off)


# (rows, columns, stride, offset in elements): strides of every residue mod
# 4, starts of every residue, ragged last blocks, one to 256 blocks.
ROWOFF4 = [
    (1000, 16383, 16383, 0), (777, 16384, 16385, 0), (300, 16384, 16386, 0),
    (129, 1000, 1001, 1), (128, 1001, 1003, 2), (17, 255, 255, 3), (5000, 130, 130, 1),
    (16, 65, 67, 3), (1, 100, 101, 1), (3, 64, 64, 1), (250, 4097, 4097, 0),
    (2049, 333, 335, 2), (40000, 70, 71, 0),
]


@pytest.mark.parametrize("R,C,ld,off", ROWOFF4)
@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_row_offsets_4byte(red, orc, kind, R, C, ld, off):
    colprod_case(red, orc, kind, R, C, ld, 2300 + R, off)


# 2-byte elements: strides of every residue mod 8, starts of every residue.
ROWOFF2 = [
    (1000, 32767, 32767, 0), (500, 32768, 32769, 0), (500, 32768, 32771, 0),
    (500, 32768, 32773, 0), (300, 1000, 1002, 1), (129, 1001, 1006, 3), (17, 255, 255, 5),
    (5000, 200, 203, 7), (1, 129, 131, 1), (250, 4097, 4097, 2), (2049, 333, 340, 6),
    (64, 4000, 4004, 4),
]


@pytest.mark.parametrize("R,C,ld,off", ROWOFF2)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_row_offsets_2byte(red, orc, kind, R, C, ld, off):
    colprod_case(red, orc, kind, R, C, ld, 2400 + R, off)


@pytest.mark.parametrize("R,C,ld,off", [(1000, 16383, 16383, 0), (129, 1000, 1001, 1),
                                        (5000, 130, 130, 1), (16, 65, 67, 3),
                                        (2049, 333, 335, 2), (40000, 70, 71, 0)])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("accum", [0, 1])
def test_row_offsets_cols(red, orc, op, R, C, ld, off, accum):
    cols_case(red, orc, op, R, C, ld, accum, 2500 + R, off)


@pytest.mark.parametrize("dst_off", [1, 3])
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16", "f16"])
def test_row_offsets_dst_alignment(red, orc, kind, dst_off):
    colprod_case(red, orc, kind, 700, 5001, 5003, 2600, 1, dst_off)
