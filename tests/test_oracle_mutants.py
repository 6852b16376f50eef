"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a copy of oracle/oracle.c with one plausible slip (a dropped
term, a wrong sign or index, a transposed operand, a lost accum, a wrong
identity, a wrong decoder shift), compiled with gcc into a temporary
directory.  The real oracle is never modified.  CPU only.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("sum_drops_last_term",
     "for (size_t i = 0; i < n; i++)\n        neumaier_add(&st, (double)x[i]);",
     "for (size_t i = 0; i + 1 < n; i++)\n        neumaier_add(&st, (double)x[i]);"),
    ("sum_compensation_sign",
     "st->c += (st->s - t) + v;", "st->c += (st->s - t) - v;"),
    ("sum_ignores_accum",
     "if (accum)\n        neumaier_add(&st, (double)old);", ""),
    ("sum_abs_without_fabs", "st->a += fabs(v);", "st->a += v;"),
    ("sum_starts_at_positive_zero",
     "neumaier_t st = {-0.0, 0.0, 0.0, 0};", "neumaier_t st = {0.0, 0.0, 0.0, 0};"),
    ("sum_adds_zero_correction",
     "return st->c == 0.0 ? st->s : st->s + st->c;", "return st->s + st->c;"),
    ("sum_computes_empty",
     "    if (n == 0)\n        return 0;\n    neumaier_t st",
     "    neumaier_t st"),
    ("max_compare_reversed", "return (b > a) ? b : a;", "return (b < a) ? b : a;"),
    ("min_compare_reversed", "return (b < a) ? b : a;", "return (b > a) ? b : a;"),
    ("max_ignores_accum",
     "    float r = accum ? *dst : NAN;\n    for (size_t i = 0; i < n; i++)\n        r = max_num(r, x[i]);",
     "    float r = NAN;\n    for (size_t i = 0; i < n; i++)\n        r = max_num(r, x[i]);"),
    ("maxnum_keeps_nan",
     "static float max_num(float a, float b)\n{\n    if (isnan(a))\n        return b;",
     "static float max_num(float a, float b)\n{\n    if (isnan(a))\n        return a;"),
    ("page_tree_pairs_neighbours",
     "slot[0] = slot[0] + slot[2];\n    slot[1] = slot[1] + slot[3];",
     "slot[0] = slot[0] + slot[1];\n    slot[1] = slot[2] + slot[3];"),
    ("page_tree_halving",
     "slot[0] = slot[0] + slot[2];\n    slot[1] = slot[1] + slot[3];\n"
     "    slot[4] = slot[4] + slot[6];\n    slot[5] = slot[5] + slot[7];",
     "slot[0] = slot[0] + slot[4];\n    slot[1] = slot[1] + slot[5];\n"
     "    slot[4] = slot[2] + slot[6];\n    slot[5] = slot[3] + slot[7];"),
    ("page_remainder_to_slot0",
     "slot[i % 8] = slot[i % 8] + x[i];", "slot[0] = slot[0] + x[i];"),
    ("page_identity_positive_zero", ": -0.0f;", ": 0.0f;"),
    ("page_accum_after_tree",
     "    if (accum)\n        slot[0] = slot[0] + *dst;\n", ""),
    ("page_chunks_restart_at_zero", "size_t c = 8;", "size_t c = 0;"),
    ("rows_stride_n_not_ld",
     "oracle_max_f32(x + r * ld, n, accum, &dst[r]);",
     "oracle_max_f32(x + r * n, n, accum, &dst[r]);"),
    ("colprod_f32_transposed",
     "p *= (double)src[i * ld + j];", "p *= (double)src[j * ld + i];"),
    ("colprod_f32_drops_last_row",
     "        double p = 1.0;\n        for (size_t i = 0; i < R; i++)\n            p *= (double)src[i * ld + j];",
     "        double p = 1.0;\n        for (size_t i = 0; i + 1 < R; i++)\n            p *= (double)src[i * ld + j];"),
    ("colprod_f32_writes_empty",
     "int oracle_colprod_f32(const float* src, size_t R, size_t C, size_t ld,\n                       double* dst)\n{\n    if (R == 0 || C == 0)",
     "int oracle_colprod_f32(const float* src, size_t R, size_t C, size_t ld,\n                       double* dst)\n{\n    if (R == 0 && C == 0)"),
    ("f16_exponent_bias", "ldexp((double)(1024 + f), e - 25)",
     "ldexp((double)(1024 + f), e - 24)"),
    ("f16_subnormal_scale", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("bf16_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("i32_adds", "p *= v;", "p += v;"),
    ("u16_keeps_high_bits", "dst[j] = (uint16_t)(p & 0xffffu);",
     "dst[j] = (uint16_t)((p >> 1) & 0xffffu);"),
    ("u32_starts_at_zero",
     "        uint32_t p = 1u;\n        for (size_t i = 0; i < R; i++)\n            p *= src[i * ld + j];",
     "        uint32_t p = 0u;\n        for (size_t i = 0; i < R; i++)\n            p *= src[i * ld + j];"),
    ("cols_sum_transposed",
     "            neumaier_add(&st, (double)src[i * ld + j]);",
     "            neumaier_add(&st, (double)src[j * ld + i]);"),
    ("cols_max_is_min",
     "            r = max_num(r, src[i * ld + j]);",
     "            r = min_num(r, src[i * ld + j]);"),
    ("mt_pieces_drop_remainder",
     "*len = base + ((size_t)i < extra ? 1 : 0);", "*len = base;"),
    ("mt_sum_skips_first_piece",
     "    for (int i = 0; i < k; i++) {\n        if (!p[i].ok)\n            continue;",
     "    for (int i = 1; i < k; i++) {\n        if (!p[i].ok)\n            continue;"),
    ("mt_extreme_ignores_accum",
     "    float r = accum ? *dst : NAN;\n    for (int i = 0; i < k; i++)",
     "    float r = NAN;\n    for (int i = 0; i < k; i++)"),
    ("mt_colprod_offset_in_elements_not_bytes",
     "(const char*)src + f * elem", "(const char*)src + f"),
    ("mt_rows_offset_ignores_stride",
     "p[i] = mt_piece(MT_ROWS_SUM, x + f * ld,", "p[i] = mt_piece(MT_ROWS_SUM, x + f * n,"),
    ("i32_signed_read",
     "uint32_t v;\n            memcpy(&v, &src[i * ld + j], sizeof v);",
     "uint32_t v = (uint32_t)(src[i * ld + j] & 0x7fffffff);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(oracle.SOURCE) as fh:
        src = fh.read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new, 1)
    assert mutated != src
    cpath = os.path.join(tmp_path, "mutant.c")
    with open(cpath, "w") as fh:
        fh.write(mutated)
    lib = oracle.build(cpath, os.path.join(tmp_path, "libmutant.so"))
    mut = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(mut)
        except Exception:  # a failed assertion, or a pin that cannot even run
            failed.append(pin.__name__)
    assert failed, "no pin catches mutant " + name
