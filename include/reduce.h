/*
 * reduce.h -- C ABI of libreduce: dense-array reduction on AMD Instinct
 * MI355X (gfx950).
 *
 * Two families of operations:
 *
 *   1. A 1-D fp32 vector reduced to one scalar by sum, max or min, with an
 *      accum mode that folds the old destination value into the result
 *      (TVM TIRx docs, "reduction -> sm100_packed": introduction, section
 *      "What it accepts" -- a 1-D fp32 source and a one-element
 *      destination -- and the table in "How inputs change the algorithm",
 *      row "accum").  The same reduction applied independently to each row
 *      of a row-major matrix is the segmented ("rows") form.
 *
 *   2. A row-major tile reduced column-wise by product to one row
 *      (PTO ISA "TCOLPROD": "Math Interpretation" -- dst[0,j] is the
 *      product of src[i,j] over the R valid rows, for each of the C valid
 *      columns; "Constraints" -- row-major layout, dst and src share the
 *      element type, the column counts agree, and a tile with zero valid
 *      rows or columns returns early).
 *
 * Conventions shared by every entry point:
 *
 *   - Every pointer is a DEVICE pointer (HBM of the current HIP device).
 *     The caller owns all buffers and must keep them alive until the work
 *     enqueued on `stream` has completed.  The library keeps no pointer
 *     after the call returns.
 *   - Every call is asynchronous with respect to the host: it validates its
 *     arguments, enqueues kernels on `stream` and returns.  `stream` is a
 *     hipStream_t passed as an opaque pointer; NULL means the null stream.
 *     It must belong to the current HIP device, as the buffers must.
 *     Results are visible after the stream is synchronised.
 *   - The return value is a status code (enum red_status).  Errors are
 *     reported synchronously and never abort.  A status other than RED_OK
 *     means nothing was enqueued, except RED_ERR_HIP after a launch, which
 *     reports what hipGetLastError() returned.  Faults raised while a
 *     kernel runs surface at the caller's next synchronisation, as for any
 *     HIP kernel.
 *   - The destination must not overlap the source (not checked).
 *   - Empty input (n == 0, rows == 0, R == 0 or C == 0) returns RED_OK,
 *     enqueues nothing and leaves the destination untouched, also under
 *     accum; for column products this is TCOLPROD's early return, and the
 *     empty product 1 is NOT written.  Pointers are not inspected then.
 *   - Floating point follows IEEE-754 with round to nearest even.
 *     Subnormal inputs and results are kept (no flush to zero).
 *   - max / min are IEEE-754-2008 maxNum / minNum: a quiet NaN operand is
 *     ignored; the result is NaN only if every operand is NaN.  When the
 *     extreme is a zero that occurs with both signs, either zero may be
 *     returned.
 *   - The default (non-atomic) entry points are deterministic: for a given
 *     input, device model and library build the result bits never change
 *     between runs.
 *   - Workspace.  The calls that combine per-workgroup partials in a second
 *     kernel (1-D, fused, column and column-product calls, and row calls
 *     with very long rows or very few rows) keep those partials in a
 *     16 MiB workspace the library allocates on the first such call for a
 *     (device, stream) pair and keeps until red_release_workspace.  For
 *     hipStreamPerThread, which names a different stream in every host
 *     thread, the workspace belongs to (device, calling thread).  A call
 *     holds its workspace while it enqueues its kernels, so calls from
 *     several host threads on one stream are ordered by that stream and
 *     never interleave their kernels.  The first call on a stream allocates
 *     device memory and must not be made under HIP graph capture.
 *   - HIP graphs.  A call captured into a graph uses the workspace of its
 *     capture stream at every replay.  Replays must therefore be ordered
 *     with each other and with the calls made on that stream (replaying
 *     on the capture stream does this), and must end before that stream's
 *     workspace is released.
 *   - Thread safety: any host thread may call any entry point.
 *   - Test hooks, read from the environment and meant to be left unset
 *     outside tests: RED_TEST_FAIL_ALLOC=1 makes the creation of a workspace
 *     fail (RED_ERR_NOMEM); RED_TEST_SCRATCH_LIMIT=<bytes>
 *     lowers the static scratch limit of red_sum_max_min_f32_noalloc;
 *     RED_TEST_CUS=<1..65536> replaces the compute-unit count the launch
 *     plans start from (results then stay correct but may differ in their
 *     last bits from the device's own plan).
 */
#ifndef LIBREDUCE_REDUCE_H
#define LIBREDUCE_REDUCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RED_ABI_VERSION 2

/* A hipStream_t, passed as an opaque pointer (NULL: the null stream). */
typedef void* red_stream_t;

enum red_status {
    RED_OK = 0,
    RED_ERR_INVALID = 1, /* null pointer for non-empty input, ld too small,
                            or a size whose byte extent overflows size_t */
    RED_ERR_ALIGN = 2,   /* a pointer not aligned to its element size */
    RED_ERR_NOMEM = 3,   /* the per-stream workspace could not be allocated */
    RED_ERR_HIP = 4,     /* the HIP runtime reported an error */
    RED_ERR_SCRATCH = 5  /* red_sum_max_min_f32_noalloc: the grid would need
                            more than the static scratch buffer holds */
};

/* ---------------------------------------------------------------------
 * 1-D fp32 vector -> scalar
 *
 * x      : n fp32 values, 4-byte aligned (16-byte alignment not required).
 * n      : number of elements; any n >= 0 (no minimum length).
 * out    : one fp32 value, 4-byte aligned.
 * accum  : 0 -> *out = reduce(x);  nonzero -> *out = old *out (+|max|min)
 *          reduce(x), with the old value folded in first.
 *
 * sum: the fp32 result lies within 1e-6 * (|old| + sum |x_i|) of the exact
 * sum for the sizes this library is built for (n up to 2^31); it is
 * computed with per-thread 8-wide accumulators, a fixed tree and a
 * fixed-order combine of per-workgroup partials.
 * max / min: exact (order cannot change the result).
 * ------------------------------------------------------------------- */
int red_sum_f32(const float* x, size_t n, float* out, int accum,
                red_stream_t stream);
int red_max_f32(const float* x, size_t n, float* out, int accum,
                red_stream_t stream);
int red_min_f32(const float* x, size_t n, float* out, int accum,
                red_stream_t stream);

/* Fused sum, max and min of one vector from a single read of it: out points
 * to three fp32 values, out[0] = sum, out[1] = max, out[2] = min (under
 * accum each folds its own old value first).  The TVM page's reduction
 * offers these three operators on the same 1-D source ("How inputs change
 * the algorithm", row "op"); computing them together reads x once instead
 * of three times.  Each result is bit-identical to the corresponding
 * red_sum_f32 / red_max_f32 / red_min_f32 result.  out must be 4-byte
 * aligned and must not overlap x. */
int red_sum_max_min_f32(const float* x, size_t n, float* out, int accum,
                        red_stream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): red_sum_max_min_f32
 * without any device or host allocation.  Same arguments, results (bit for
 * bit) and errors, and the same two kernels, but the per-workgroup partials
 * (12 bytes per workgroup of the first pass, at most one workgroup per
 * compute unit) live in a 16 KiB static device buffer that the library
 * declares and that each GPU it runs on holds until the process ends.
 * Calls whose grid would need more than 16 KiB of partials (devices of
 * more than 1365 compute units) return RED_ERR_SCRATCH and enqueue nothing.
 * Nothing in the buffer has to start at zero: the first kernel writes
 * every partial the second reads.  Every call on one GPU shares that GPU's
 * buffer, whatever its stream or host thread: calls that overlap in time
 * on one GPU race and give wrong results, so the caller must order them
 * (for example, issue them all on one stream).  The first call on a device
 * looks up the buffer's device address once (hipGetSymbolAddress) and
 * keeps it in a fixed table of 64 devices: on a device of index 64 or more
 * the call returns RED_ERR_HIP and enqueues nothing. */
int red_sum_max_min_f32_noalloc(const float* x, size_t n, float* out, int accum,
                                red_stream_t stream);

/* Single-pass variants: each workgroup folds its partial into *out with
 * one device-scope atomic, as the one-atomic-per-program block reduce in
 * the imxueqiu.com blog post on a Triton vector-sum kernel does (its
 * hand-written C version: warp reduce, shared-memory combine, one atomicAdd
 * by thread 0).  Same arguments and error behaviour as above.  With
 * accum == 0 the library first sets *out to the identity (-0.0 for sum, a
 * quiet NaN for max / min) on `stream`.  sum uses the hardware fp32 atomic
 * add, so its rounding order -- and its last bits -- vary from run to run
 * (same error bound); on gfx950 that atomic keeps subnormal operands and
 * results and the sign of zero, as the other entry points do (a zero sum
 * is -0 only when every term is -0); max / min fold each workgroup's result with one
 * integer atomic max / min on the fp32 bit pattern and are exact (an old
 * NaN under accum is replaced first by compare-and-swap; equal zeros of
 * both signs give +0 for max and -0 for min).  No workspace is used. */
int red_sum_f32_atomic(const float* x, size_t n, float* out, int accum,
                       red_stream_t stream);
int red_max_f32_atomic(const float* x, size_t n, float* out, int accum,
                       red_stream_t stream);
int red_min_f32_atomic(const float* x, size_t n, float* out, int accum,
                       red_stream_t stream);

/* ---------------------------------------------------------------------
 * Segmented rows: out[r] = reduce(x[r*ld .. r*ld + n)) for r < rows
 *
 * x      : row-major fp32 matrix, 4-byte aligned; row r starts at x + r*ld.
 *          Elements between n and ld in a row never affect the result.
 *          Nothing past the last row's n-th element is read; rows of 17
 *          to 64 elements with ld <= 64, or with ld <= 128 and
 *          ld - n <= n / 8, are read as one span, padding included, and
 *          the padding is dropped.
 * rows   : number of rows; n : elements reduced per row; ld : row stride
 *          in elements, ld >= n (RED_ERR_INVALID otherwise).
 * out    : rows fp32 values, 4-byte aligned.
 * accum  : nonzero folds old out[r] into row r's result.
 *
 * Rows of at most 64 elements are reduced one per thread in exactly the
 * single-precision order of the TVM page's "Algorithm" section (8 slots,
 * chunks of 8, leftovers into slot i mod 8, the 8 -> 4 -> 2 -> 1 tree,
 * accum into slot 0 first).  Longer rows are shared by 16, 32 or 64 lanes
 * (up to 1024 elements) or by a wavefront (up to 4096); rows longer still,
 * or too few rows to occupy the device, are cut into chunks reduced by
 * separate workgroups whose partials a second kernel folds in index order
 * (that case uses the stream's workspace).  Every choice depends only on
 * (rows, n, ld, alignment of x) and the device's compute-unit count, so
 * the results are deterministic.  Same tolerances as the 1-D calls.
 * ------------------------------------------------------------------- */
int red_sum_rows_f32(const float* x, size_t rows, size_t n, size_t ld,
                     float* out, int accum, red_stream_t stream);
int red_max_rows_f32(const float* x, size_t rows, size_t n, size_t ld,
                     float* out, int accum, red_stream_t stream);
int red_min_rows_f32(const float* x, size_t rows, size_t n, size_t ld,
                     float* out, int accum, red_stream_t stream);

/* ---------------------------------------------------------------------
 * Column sum / max / min: dst[j] = reduce_{i<R} src[i*ld + j], j < C
 *
 * The reduction of the TVM page ("reduction -> sm100_packed") taken along
 * the rows of a 2-D source -- the case its fast path leaves to a generic
 * fallback ("How inputs change the algorithm", last row).  Layout, ld,
 * alignment, empty-tile early return and errors as for the column product
 * below; accum folds old dst[j] into column j first.  Same identities,
 * NaN policy and tolerances as the 1-D calls: max / min exact, sum within
 * 1e-6 * (|old| + sum |x|) per column.  Deterministic.
 * ------------------------------------------------------------------- */
int red_sum_cols_f32(const float* src, size_t R, size_t C, size_t ld,
                     float* dst, int accum, red_stream_t stream);
int red_max_cols_f32(const float* src, size_t R, size_t C, size_t ld,
                     float* dst, int accum, red_stream_t stream);
int red_min_cols_f32(const float* src, size_t R, size_t C, size_t ld,
                     float* dst, int accum, red_stream_t stream);

/* ---------------------------------------------------------------------
 * Column product (TCOLPROD): dst[j] = prod_{i<R} src[i*ld + j], j < C
 *
 * src    : row-major tile of element type T, aligned to sizeof(T); row i
 *          starts at src + i*ld.  Elements between C and ld are never read.
 * R, C   : valid rows and columns; ld : row stride in elements, ld >= C
 *          (RED_ERR_INVALID otherwise -- the analogue of TCOLPROD's check
 *          that source and destination agree on the valid column count).
 * dst    : C values of the same element type T, aligned to sizeof(T).
 *
 * f32    : products accumulate in fp32; relative error <= (R-1) * 2^-24
 *          whatever the order.
 * f16/bf16 (given as uint16_t bit patterns: IEEE binary16 / bfloat16):
 *          values are widened exactly to fp32, multiplied in fp32, and the
 *          final product is rounded once to T (round to nearest even).
 * i32    : products wrap modulo 2^32 (two's complement); bit-exact.
 *
 * Deterministic: for a given shape, alignment and device, the rows are
 * split over workgroups in a fixed way and the partial products are
 * combined in a fixed order, so repeated calls give identical bits.
 * ------------------------------------------------------------------- */
int red_colprod_f32(const float* src, size_t R, size_t C, size_t ld,
                    float* dst, red_stream_t stream);
int red_colprod_f16(const uint16_t* src, size_t R, size_t C, size_t ld,
                    uint16_t* dst, red_stream_t stream);
int red_colprod_bf16(const uint16_t* src, size_t R, size_t C, size_t ld,
                     uint16_t* dst, red_stream_t stream);
int red_colprod_i32(const int32_t* src, size_t R, size_t C, size_t ld,
                    int32_t* dst, red_stream_t stream);

/* The other integer element types TCOLPROD lists ("Constraints": int16 and
 * int32 on A2A3; int16, uint16, int32, uint32 on A5).  Same arguments,
 * layout and errors as above; products wrap modulo 2^32 (u32) or 2^16 (i16,
 * u16) and are bit-exact.  The low bits of a product depend only on the low
 * bits of its factors, so i16 and u16 give the same bit patterns, and u32
 * the same bits as i32. */
int red_colprod_i16(const int16_t* src, size_t R, size_t C, size_t ld,
                    int16_t* dst, red_stream_t stream);
int red_colprod_u16(const uint16_t* src, size_t R, size_t C, size_t ld,
                    uint16_t* dst, red_stream_t stream);
int red_colprod_u32(const uint32_t* src, size_t R, size_t C, size_t ld,
                    uint32_t* dst, red_stream_t stream);

/* ---------------------------------------------------------------------
 * Utilities
 * ------------------------------------------------------------------- */

/* Waits for the work enqueued on `stream` to finish, then frees the
 * workspace the library holds for (current device, stream) -- for
 * hipStreamPerThread, the calling thread's.  Call it before destroying a
 * stream that library calls used, or before a thread that used
 * hipStreamPerThread exits; a later call on the stream allocates a new
 * workspace.  RED_OK when there is nothing to free; RED_ERR_HIP when the
 * synchronisation or the free fails.  The stream must still exist. */
int red_release_workspace(red_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* red_status_str(int status);

/* RED_ABI_VERSION of the built library. */
int red_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBREDUCE_REDUCE_H */
