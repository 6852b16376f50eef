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
 * Threaded forms (suffix _mt) run the same functions on contiguous pieces
 * of the input on several host threads and combine the pieces' results in
 * piece order; they exist to time the oracle on a multi-core host.
 *
 * Every function here is pinned by tests/test_oracle.py (brute force with
 * exact rationals or big integers, closed forms, a worked example derived by
 * hand from the page's algorithm, and exhaustive checks of the decoders).
 * No function is "parity unpinned".
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* sum                                                                 */
/* ------------------------------------------------------------------ */

/* Neumaier's compensated summation in double: the running sum s plus a
 * separate correction c that collects the low-order bits each addition
 * loses.  For fp32 inputs this reproduces the exact sum to within about
 * one double rounding, far below any fp32 tolerance.
 *
 * Sign of a zero sum (reading; the pages are silent): IEEE-754 addition in
 * round-to-nearest gives -0 only for two negative zeros, and +0 for any
 * other pair whose exact sum is zero.  So a sum that is exactly zero is -0
 * when every term is -0 and +0 otherwise, in every order of evaluation.
 * The running sum starts at -0.0 (the IEEE additive identity, x + -0 = x
 * for every x) so that the double sum follows the same rule. */
typedef struct {
    double s;      /* running sum; starts at -0.0, the additive identity */
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
    if (st->nonfinite)
        return st->s;
    /* A zero correction leaves the running sum as it is: adding a +0
     * correction would turn the -0 sum of negative zeros into +0. */
    return st->c == 0.0 ? st->s : st->s + st->c;
}

/* S = [old if accum] + sum_{i<n} x[i], and A = sum of the absolute values of
 * the same terms.  Returns 0 and writes nothing when n == 0. */
int oracle_sum_f32(const float* x, size_t n, int accum, float old,
                   double* s_out, double* a_out)
{
    if (n == 0)
        return 0;
    neumaier_t st = {-0.0, 0.0, 0.0, 0};
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
        neumaier_t st = {-0.0, 0.0, 0.0, 0};
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

/* ------------------------------------------------------------------ */
/* Threaded forms (timing the oracle on several host cores)             */
/* ------------------------------------------------------------------ */

/* The same definitions spread over `threads` host threads, for timing the
 * oracle as a CPU baseline: the work is cut into `threads` contiguous
 * pieces of nearly equal size (elements of a vector, rows of a row
 * reduction, columns of a column product), each piece is computed by the
 * single-threaded function above on a thread of its own, and the pieces'
 * results are combined on the calling thread in piece order.  Rows and
 * columns are independent, so those results are identical to the
 * single-threaded ones; max / min are exact in any order; the sum adds the
 * pieces' double-precision sums with the same compensated summation.
 * Each returns what its single-threaded form returns, or -1 (nothing
 * written) when a thread could not be started. */
#define MT_MAX_THREADS 256

enum mt_kind { MT_SUM, MT_MAX, MT_MIN, MT_ROWS_SUM, MT_ROWS_MAX, MT_COLPROD_F32,
               MT_COLPROD_F16, MT_COLPROD_BF16, MT_COLPROD_I32 };

typedef struct {
    enum mt_kind kind;
    const void* src; /* the piece's first element, row or column */
    size_t count;    /* elements (1-D), rows (rows) or columns (colprod) */
    size_t n;        /* row length (rows) or row count R (colprod) */
    size_t ld;       /* row stride in elements */
    void* out;       /* the piece's first output */
    void* out2;      /* row sums: the piece's first sum of |x| */
    double s, a;     /* 1-D sum: the piece's S and A */
    float e;         /* 1-D max / min: the piece's extreme */
    int ok;          /* the single-threaded function's return value */
} mt_piece_t;

static void* mt_run(void* arg)
{
    mt_piece_t* p = (mt_piece_t*)arg;
    const float* xf = (const float*)p->src;
    const uint16_t* xh = (const uint16_t*)p->src;
    switch (p->kind) {
    case MT_SUM:
        p->ok = oracle_sum_f32(xf, p->count, 0, 0.0f, &p->s, &p->a);
        break;
    case MT_MAX:
        p->ok = oracle_max_f32(xf, p->count, 0, &p->e);
        break;
    case MT_MIN:
        p->ok = oracle_min_f32(xf, p->count, 0, &p->e);
        break;
    case MT_ROWS_SUM:
        p->ok = oracle_rows_sum_f32(xf, p->count, p->n, p->ld, 0, NULL,
                                    (double*)p->out, (double*)p->out2);
        break;
    case MT_ROWS_MAX:
        p->ok = oracle_rows_max_f32(xf, p->count, p->n, p->ld, 0, (float*)p->out);
        break;
    case MT_COLPROD_F32:
        p->ok = oracle_colprod_f32(xf, p->n, p->count, p->ld, (double*)p->out);
        break;
    case MT_COLPROD_F16:
        p->ok = oracle_colprod_f16(xh, p->n, p->count, p->ld, (double*)p->out);
        break;
    case MT_COLPROD_BF16:
        p->ok = oracle_colprod_bf16(xh, p->n, p->count, p->ld, (double*)p->out);
        break;
    case MT_COLPROD_I32:
        p->ok = oracle_colprod_i32((const int32_t*)p->src, p->n, p->count, p->ld,
                                   (int32_t*)p->out);
        break;
    }
    return NULL;
}

/* Runs pieces[0..k) on k threads (piece 0 on the caller).  Returns 0 if a
 * thread could not be started; every started thread is joined first. */
static int mt_execute(mt_piece_t* pieces, int k)
{
    pthread_t tid[MT_MAX_THREADS];
    int started = 0, ok = 1;
    for (int i = 1; i < k; i++) {
        if (pthread_create(&tid[i], NULL, mt_run, &pieces[i]) != 0) {
            ok = 0;
            break;
        }
        started = i;
    }
    if (ok)
        mt_run(&pieces[0]);
    for (int i = 1; i <= started; i++)
        pthread_join(tid[i], NULL);
    return ok;
}

/* Piece i of `count` items cut into k nearly equal contiguous pieces. */
static void mt_range(size_t count, int k, int i, size_t* first, size_t* len)
{
    size_t base = count / (size_t)k, extra = count % (size_t)k;
    *first = (size_t)i * base + ((size_t)i < extra ? (size_t)i : extra);
    *len = base + ((size_t)i < extra ? 1 : 0);
}

static int mt_clamp(int threads)
{
    return threads < 1 ? 1 : (threads > MT_MAX_THREADS ? MT_MAX_THREADS : threads);
}

static mt_piece_t mt_piece(enum mt_kind kind, const void* src, size_t count,
                           size_t n, size_t ld, void* out, void* out2)
{
    mt_piece_t p;
    memset(&p, 0, sizeof p);
    p.kind = kind;
    p.src = src;
    p.count = count;
    p.n = n;
    p.ld = ld;
    p.out = out;
    p.out2 = out2;
    return p;
}

int oracle_sum_f32_mt(const float* x, size_t n, int accum, float old,
                      int threads, double* s_out, double* a_out)
{
    if (n == 0)
        return 0;
    const int k = mt_clamp(threads);
    mt_piece_t p[MT_MAX_THREADS];
    for (int i = 0; i < k; i++) {
        size_t f, len;
        mt_range(n, k, i, &f, &len);
        p[i] = mt_piece(MT_SUM, x + f, len, 0, 0, NULL, NULL);
    }
    if (!mt_execute(p, k))
        return -1;
    neumaier_t st = {-0.0, 0.0, 0.0, 0};
    if (accum)
        neumaier_add(&st, (double)old);
    double a = st.a;
    for (int i = 0; i < k; i++) {
        if (!p[i].ok)
            continue; /* an empty piece (n < threads) */
        neumaier_add(&st, p[i].s);
        a += p[i].a;
    }
    *s_out = neumaier_result(&st);
    *a_out = a;
    return 1;
}

static int extreme_mt(enum mt_kind kind, const float* x, size_t n, int accum,
                      int threads, float* dst)
{
    if (n == 0)
        return 0;
    const int k = mt_clamp(threads);
    mt_piece_t p[MT_MAX_THREADS];
    for (int i = 0; i < k; i++) {
        size_t f, len;
        mt_range(n, k, i, &f, &len);
        p[i] = mt_piece(kind, x + f, len, 0, 0, NULL, NULL);
    }
    if (!mt_execute(p, k))
        return -1;
    float r = accum ? *dst : NAN;
    for (int i = 0; i < k; i++)
        if (p[i].ok)
            r = (kind == MT_MAX) ? max_num(r, p[i].e) : min_num(r, p[i].e);
    *dst = r;
    return 1;
}

int oracle_max_f32_mt(const float* x, size_t n, int accum, int threads, float* dst)
{
    return extreme_mt(MT_MAX, x, n, accum, threads, dst);
}

int oracle_min_f32_mt(const float* x, size_t n, int accum, int threads, float* dst)
{
    return extreme_mt(MT_MIN, x, n, accum, threads, dst);
}

/* Row sums and row maxima without accum, rows spread over the threads. */
int oracle_rows_sum_f32_mt(const float* x, size_t rows, size_t n, size_t ld,
                           int threads, double* s_out, double* a_out)
{
    if (rows == 0 || n == 0)
        return 0;
    const int k = mt_clamp(threads);
    mt_piece_t p[MT_MAX_THREADS];
    for (int i = 0; i < k; i++) {
        size_t f, len;
        mt_range(rows, k, i, &f, &len);
        p[i] = mt_piece(MT_ROWS_SUM, x + f * ld, len, n, ld, s_out + f, a_out + f);
    }
    return mt_execute(p, k) ? 1 : -1;
}

int oracle_rows_max_f32_mt(const float* x, size_t rows, size_t n, size_t ld,
                           int threads, float* dst)
{
    if (rows == 0 || n == 0)
        return 0;
    const int k = mt_clamp(threads);
    mt_piece_t p[MT_MAX_THREADS];
    for (int i = 0; i < k; i++) {
        size_t f, len;
        mt_range(rows, k, i, &f, &len);
        p[i] = mt_piece(MT_ROWS_MAX, x + f * ld, len, n, ld, dst + f, NULL);
    }
    return mt_execute(p, k) ? 1 : -1;
}

/* Column products with the columns spread over the threads. */
static int colprod_mt(enum mt_kind kind, const void* src, size_t elem, size_t R,
                      size_t C, size_t ld, void* dst, size_t out_elem, int threads)
{
    if (R == 0 || C == 0)
        return 0;
    const int k = mt_clamp(threads);
    mt_piece_t p[MT_MAX_THREADS];
    for (int i = 0; i < k; i++) {
        size_t f, len;
        mt_range(C, k, i, &f, &len);
        p[i] = mt_piece(kind, (const char*)src + f * elem, len, R, ld,
                        (char*)dst + f * out_elem, NULL);
    }
    return mt_execute(p, k) ? 1 : -1;
}

int oracle_colprod_f32_mt(const float* src, size_t R, size_t C, size_t ld,
                          int threads, double* dst)
{
    return colprod_mt(MT_COLPROD_F32, src, 4, R, C, ld, dst, 8, threads);
}

int oracle_colprod_f16_mt(const uint16_t* src, size_t R, size_t C, size_t ld,
                          int threads, double* dst)
{
    return colprod_mt(MT_COLPROD_F16, src, 2, R, C, ld, dst, 8, threads);
}

int oracle_colprod_bf16_mt(const uint16_t* src, size_t R, size_t C, size_t ld,
                           int threads, double* dst)
{
    return colprod_mt(MT_COLPROD_BF16, src, 2, R, C, ld, dst, 8, threads);
}

int oracle_colprod_i32_mt(const int32_t* src, size_t R, size_t C, size_t ld,
                          int threads, int32_t* dst)
{
    return colprod_mt(MT_COLPROD_I32, src, 4, R, C, ld, dst, 4, threads);
}
