/*
 * oracle.c -- plain, slow CPU oracle for dense-array reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file.  Its only users are the tests under tests/, the smoke check
 * in __graft_entry__.py and the cpu_baseline leg of bench.py.  It shares no
 * code, header, table or constant with the HIP library, and it includes
 * nothing from it.
 *
 * Each function is the definition of one reduction written out as directly
 * as possible, in double precision where the result is floating point:
 *
 *   sum   -- TVM TIRx docs, "reduction -> sm100_packed", introduction and the
 *            table "How inputs change the algorithm": a 1-D fp32 vector is
 *            reduced to one scalar; with accum the old dst value takes part.
 *   max / min -- same page and sections (the max / min operators).
 *   page-order sum -- same page, section "Algorithm": the 8-slot fp32
 *            accumulator, the chunk-of-8 fold, the scalar remainder and the
 *            8 -> 4 -> 2 -> 1 tree, replayed in single precision.
 *   column sum / max / min -- the TVM page's reduction taken along the rows
 *            of a 2-D source (the 2-D case its fast path hands to a generic
 *            fallback, "How inputs change the algorithm").
 *   colprod -- PTO ISA "TCOLPROD", sections "Math Interpretation" (the
 *            per-column product over the R valid rows) and "Constraints"
 *            (early return for zero valid rows or columns; supported element
 *            types half, float, bfloat16, int16, uint16, int32, uint32).
 *
 * Readings where the pages are silent:
 *   - n == 0 (1-D and rows) is treated like TCOLPROD's empty tile: nothing
 *     is written, not even under accum.
 *   - max / min follow IEEE-754-2008 maxNum / minNum: a NaN operand is
 *     ignored; the result is NaN only when every operand is NaN.
 *   - accum folds the old dst into the first accumulator slot before any
 *     element; for the exact definitions the position does not matter.
 *   - int32 / uint32 products wrap modulo 2^32, int16 / uint16 products
 *     modulo 2^16 (computed in uint32_t).
 *   - half / bfloat16 are decoded exactly from their bit definitions.
 *
 * Every function here is pinned by tests/test_oracle.py (brute force with
 * exact rationals or big integers, closed forms, a worked example derived by
 * hand from the page's algorithm, and exhaustive checks of the decoders).
 * No function is "parity unpinned".
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* sum                                                                 */
/* ------------------------------------------------------------------ */

/* Neumaier's compensated summation in double: the running sum s plus a
 * separate correction c that collects the low-order bits each addition
 * loses.  For fp32 inputs this reproduces the exact sum to within about
 * one double rounding, far below any fp32 tolerance. */
typedef struct {
    double s;      /* running sum */
    double c;      /* accumulated rounding corrections */
    double a;      /* running sum of absolute values */
    int nonfinite; /* an inf or NaN term was seen */
} neumaier_t;

static void neumaier_add(neumaier_t* st, double v)
{
    if (!isfinite(v))
        st->nonfinite = 1;
    double t = st->s + v;
    if (fabs(st->s) >= fabs(v))
        st->c += (st->s - t) + v;
    else
        st->c += (v - t) + st->s;
    st->s = t;
    st->a += fabs(v);
}

static double neumaier_result(const neumaier_t* st)
{
    /* With an inf or NaN term the compensation is meaningless; the plain
     * IEEE sum carries the right class (inf, -inf or NaN). */
    return st->nonfinite ? st->s : st->s + st->c;
}

/* S = [old if accum] + sum_{i<n} x[i], and A = sum of the absolute values of
 * the same terms.  Returns 0 and writes nothing when n == 0. */
int oracle_sum_f32(const float* x, size_t n, int accum, float old,
                   double* s_out, double* a_out)
{
    if (n == 0)
        return 0;
    neumaier_t st = {0.0, 0.0, 0.0, 0};
    if (accum)
        neumaier_add(&st, (double)old);
    for (size_t i = 0; i < n; i++)
        neumaier_add(&st, (double)x[i]);
    *s_out = neumaier_result(&st);
    *a_out = st.a;
    return 1;
}

/* ------------------------------------------------------------------ */
/* max / min under maxNum / minNum                                     */
/* ------------------------------------------------------------------ */

static float max_num(float a, float b)
{
    if (isnan(a))
        return b;
    if (isnan(b))
        return a;
    return (b > a) ? b : a;
}

static float min_num(float a, float b)
{
    if (isnan(a))
        return b;
    if (isnan(b))
        return a;
    return (b < a) ? b : a;
}

/* *dst = max over x[0..n) (and the old *dst under accum).  A quiet NaN is
 * the identity of maxNum, so the fold starts from NaN.  n == 0: untouched. */
int oracle_max_f32(const float* x, size_t n, int accum, float* dst)
{
    if (n == 0)
        return 0;
    float r = accum ? *dst : NAN;
    for (size_t i = 0; i < n; i++)
        r = max_num(r, x[i]);
    *dst = r;
    return 1;
}

int oracle_min_f32(const float* x, size_t n, int accum, float* dst)
{
    if (n == 0)
        return 0;
    float r = accum ? *dst : NAN;
    for (size_t i = 0; i < n; i++)
        r = min_num(r, x[i]);
    *dst = r;
    return 1;
}

/* ------------------------------------------------------------------ */
/* The page's own single-precision summation order                      */
/* ------------------------------------------------------------------ */

/* TVM TIRx "reduction -> sm100_packed", section "Algorithm" (sum): an
 * 8-wide fp32 accumulator takes the first 8 elements; every further full
 * chunk of 8 is added slot by slot; the remaining n mod 8 elements are added
 * one at a time (reading: element i goes to slot i mod 8); the accumulator
 * then collapses pairwise exactly as the page's tree shows:
 *     slots (0,1) += slots (2,3);  slots (4,5) += slots (6,7);
 *     slots (0,1) += slots (4,5);  result = slot 0 + slot 1.
 * accum (section "How inputs change the algorithm") adds the old dst into
 * slot 0 before any chunk is folded.  The page requires n >= 8; for
 * 1 <= n < 8 the unused slots hold the additive identity -0.0 (reading).
 * All arithmetic is IEEE single precision, round to nearest even, with no
 * flush of subnormals.  n == 0: nothing written. */
int oracle_page_sum_f32(const float* x, size_t n, int accum, float* dst)
{
    if (n == 0)
        return 0;
    float slot[8];
    for (size_t k = 0; k < 8; k++)
        slot[k] = (k < n) ? x[k] : -0.0f;
    if (accum)
        slot[0] = slot[0] + *dst;
    size_t c = 8;
    for (; c + 8 <= n; c += 8)
        for (size_t k = 0; k < 8; k++)
            slot[k] = slot[k] + x[c + k];
    for (size_t i = c; i < n; i++)
        slot[i % 8] = slot[i % 8] + x[i];
    slot[0] = slot[0] + slot[2];
    slot[1] = slot[1] + slot[3];
    slot[4] = slot[4] + slot[6];
    slot[5] = slot[5] + slot[7];
    slot[0] = slot[0] + slot[4];
    slot[1] = slot[1] + slot[5];
    *dst = slot[0] + slot[1];
    return 1;
}

/* ------------------------------------------------------------------ */
/* Segmented rows: the 1-D definitions applied to each row              */
/* ------------------------------------------------------------------ */

/* Row r is x[r*ld .. r*ld + n).  Under accum, row r folds old[r]. */
int oracle_rows_sum_f32(const float* x, size_t rows, size_t n, size_t ld,
                        int accum, const float* old, double* s_out,
                        double* a_out)
{
    if (rows == 0 || n == 0)
        return 0;
    for (size_t r = 0; r < rows; r++)
        oracle_sum_f32(x + r * ld, n, accum, accum ? old[r] : 0.0f,
                       &s_out[r], &a_out[r]);
    return 1;
}

int oracle_rows_max_f32(const float* x, size_t rows, size_t n, size_t ld,
                        int accum, float* dst)
{
    if (rows == 0 || n == 0)
        return 0;
    for (size_t r = 0; r < rows; r++)
        oracle_max_f32(x + r * ld, n, accum, &dst[r]);
    return 1;
}

int oracle_rows_min_f32(const float* x, size_t rows, size_t n, size_t ld,
                        int accum, float* dst)
{
    if (rows == 0 || n == 0)
        return 0;
    for (size_t r = 0; r < rows; r++)
        oracle_min_f32(x + r * ld, n, accum, &dst[r]);
    return 1;
}

int oracle_rows_page_sum_f32(const float* x, size_t rows, size_t n,
                             size_t ld, int accum, float* dst)
{
    if (rows == 0 || n == 0)
        return 0;
    for (size_t r = 0; r < rows; r++)
        oracle_page_sum_f32(x + r * ld, n, accum, &dst[r]);
    return 1;
}

/* ------------------------------------------------------------------ */
/* 16-bit float decoding, from the bit definitions                      */
/* ------------------------------------------------------------------ */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 encodes zero and subnormals (fraction * 2^-24);
 * exponent 31 encodes inf (fraction 0) and NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE-754 binary32 bit pattern. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* Column product (TCOLPROD)                                            */
/* ------------------------------------------------------------------ */

/* dst[j] = prod_{i<R} src[i*ld + j] for j < C, in double.  R == 0 or
 * C == 0: return early, dst untouched (the empty product 1 is NOT written). */
int oracle_colprod_f32(const float* src, size_t R, size_t C, size_t ld,
                       double* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        double p = 1.0;
        for (size_t i = 0; i < R; i++)
            p *= (double)src[i * ld + j];
        dst[j] = p;
    }
    return 1;
}

int oracle_colprod_f16(const uint16_t* src, size_t R, size_t C, size_t ld,
                       double* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        double p = 1.0;
        for (size_t i = 0; i < R; i++)
            p *= oracle_f16_to_f64(src[i * ld + j]);
        dst[j] = p;
    }
    return 1;
}

int oracle_colprod_bf16(const uint16_t* src, size_t R, size_t C, size_t ld,
                        double* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        double p = 1.0;
        for (size_t i = 0; i < R; i++)
            p *= oracle_bf16_to_f64(src[i * ld + j]);
        dst[j] = p;
    }
    return 1;
}

/* int32: the product modulo 2^32, read back as two's complement. */
int oracle_colprod_i32(const int32_t* src, size_t R, size_t C, size_t ld,
                       int32_t* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        uint32_t p = 1u;
        for (size_t i = 0; i < R; i++) {
            uint32_t v;
            memcpy(&v, &src[i * ld + j], sizeof v);
            p *= v;
        }
        memcpy(&dst[j], &p, sizeof p);
    }
    return 1;
}

/* uint32: the product modulo 2^32. */
int oracle_colprod_u32(const uint32_t* src, size_t R, size_t C, size_t ld,
                       uint32_t* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        uint32_t p = 1u;
        for (size_t i = 0; i < R; i++)
            p *= src[i * ld + j];
        dst[j] = p;
    }
    return 1;
}

/* int16 / uint16 (given as 16-bit patterns): the product modulo 2^16.  It is
 * computed modulo 2^32 and truncated: reduction modulo 2^16 commutes with
 * multiplication, so the low 16 bits are those of the exact product for
 * signed and unsigned readings alike. */
int oracle_colprod_u16(const uint16_t* src, size_t R, size_t C, size_t ld,
                       uint16_t* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        uint32_t p = 1u;
        for (size_t i = 0; i < R; i++)
            p *= (uint32_t)src[i * ld + j];
        dst[j] = (uint16_t)(p & 0xffffu);
    }
    return 1;
}

/* ------------------------------------------------------------------ */
/* Column sum / max / min of a row-major fp32 tile                      */
/* ------------------------------------------------------------------ */

/* The 1-D definitions applied to each column j < C of the R x C valid
 * region (row stride ld): the reduction the TVM page's primitive performs,
 * taken along the first axis of a 2-D source instead of over a whole
 * vector.  Under accum, column j folds old[j].  R == 0 or C == 0: nothing
 * written. */
int oracle_cols_sum_f32(const float* src, size_t R, size_t C, size_t ld,
                        int accum, const float* old, double* s_out,
                        double* a_out)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        neumaier_t st = {0.0, 0.0, 0.0, 0};
        if (accum)
            neumaier_add(&st, (double)old[j]);
        for (size_t i = 0; i < R; i++)
            neumaier_add(&st, (double)src[i * ld + j]);
        s_out[j] = neumaier_result(&st);
        a_out[j] = st.a;
    }
    return 1;
}

int oracle_cols_max_f32(const float* src, size_t R, size_t C, size_t ld,
                        int accum, float* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        float r = accum ? dst[j] : NAN;
        for (size_t i = 0; i < R; i++)
            r = max_num(r, src[i * ld + j]);
        dst[j] = r;
    }
    return 1;
}

int oracle_cols_min_f32(const float* src, size_t R, size_t C, size_t ld,
                        int accum, float* dst)
{
    if (R == 0 || C == 0)
        return 0;
    for (size_t j = 0; j < C; j++) {
        float r = accum ? dst[j] : NAN;
        for (size_t i = 0; i < R; i++)
            r = min_num(r, src[i * ld + j]);
        dst[j] = r;
    }
    return 1;
}
