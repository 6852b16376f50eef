// rows.hip -- segmented reduction: out[r] = reduce(x[r*ld .. r*ld + n)).
//
// Kernels picked by the host from (rows, n) and the CU count alone, so
// that a given problem on a given device always runs the same code and
// gives the same bits:
//
//  * rows_short (n <= 4): eight rows per thread per step, all their loads
//    issued together, over a grid of a few workgroups per CU; each row in
//    the same order as rows_thread;
//  * rows_thread (4 < n <= 16) / rows_tile (16 < n <= 64): one thread per row
//    (rows of 17 to 64 elements first staged in LDS 128 at a time with
//    coalesced loads), running the thread-scope
//    algorithm of the TVM TIRx page "reduction -> sm100_packed" (section
//    "Algorithm") in exactly its single-precision order: 8 slots take the
//    first 8 elements, each further full chunk of 8 is added slot by slot,
//    leftovers go one by one into slot i mod 8, and the slots collapse
//    (0,1)+=(2,3), (4,5)+=(6,7), (0,1)+=(4,5), result = slot 0 + slot 1.
//    accum adds the old destination into slot 0 first ("How inputs change
//    the algorithm").  max / min use four slots folded with max3 / min3.
//  * rows_seg (64 < n <= 1024): 16, 32 or 64 lanes per row (by n), each
//    lane holding up to two or four non-temporal 16-byte loads of a row, and
//    2 to 16 rows per wave, every load issued before any row is reduced;
//    one multi-wide accumulator per row, a DPP reduction over each lane
//    segment; the segment's last lane stores.  Each workgroup walks a
//    contiguous range of rows.  No LDS, no second pass.
//  * rows_wave (1024 < n <= 4096, at least 8 rows per CU): one row per
//    wave, looping over the row four vectors per lane at a time.
//  * rows_split: rows longer than 4096 elements, or too few rows to give
//    every CU waves: K workgroups share each row, streaming it like the 1-D
//    vector, and a second kernel folds each row's K partials in index order
//    (no second kernel when K = 1).
#include "device.hpp"
#include "internal.hpp"

namespace red {
namespace {

constexpr uint64_t kThreadRowMax = 64; // rows this short go one per thread
#ifndef RED_ROWS_WAVE_MAX
#define RED_ROWS_WAVE_MAX 4096
#endif
// Longest row one wave reduces; longer rows go to the split kernel.
// (Measured on MI355X, 256 MiB of rows from HBM: 8192-element rows 43.4 us
// one wave per row, 41.3 us split; 16384-element rows 50.3 vs 43.0 us.)
constexpr uint64_t kWaveRowMax = RED_ROWS_WAVE_MAX;
#ifndef RED_ROWS_WG_PER_CU
#define RED_ROWS_WG_PER_CU 16
#endif
constexpr uint64_t kRowsWgPerCu = RED_ROWS_WG_PER_CU;

// ---- one thread per row: the page's exact order ---------------------------

// Reads 8 consecutive elements; VEC means p is 16-byte aligned.
template <bool VEC>
__device__ __forceinline__ void load8(const float* __restrict__ p, float v[8])
{
    if constexpr (VEC) {
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = p[k];
    }
}

// The page's collapse of the eight sum slots: (0,1) += (2,3),
// (4,5) += (6,7), (0,1) += (4,5), result = slot 0 + slot 1.
__device__ __forceinline__ float slot_tree(float s[8])
{
    s[0] = s[0] + s[2];
    s[1] = s[1] + s[3];
    s[4] = s[4] + s[6];
    s[5] = s[5] + s[7];
    s[0] = s[0] + s[4];
    s[1] = s[1] + s[5];
    return s[0] + s[1];
}

// The cnt < 8 consecutive elements p[0 .. cnt-1] of global memory into
// v[0 .. cnt-1] (v[k] = 0 for k >= cnt) with at most three loads, of 4, 2
// and 1 elements.  p need only be 4-byte aligned: gfx950 reads unaligned
// multi-dword vectors from global memory.  (One 4-byte load per element,
// each lane on its own row, cost rows of 15 elements 99 us per 256 MiB
// against 51 us for rows of 16.)
__device__ __forceinline__ void load_tail(const float* __restrict__ p, uint32_t cnt,
                                          float v[8])
{
    typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
    typedef float f2u __attribute__((ext_vector_type(2), aligned(4)));
    const uint32_t A = cnt & 4u, B = cnt & 2u;
    f4u a = {0.0f, 0.0f, 0.0f, 0.0f};
    f2u b = {0.0f, 0.0f};
    float c = 0.0f;
    if (A)
        a = *reinterpret_cast<const f4u*>(p);
    if (B)
        b = *reinterpret_cast<const f2u*>(p + A);
    if (cnt & 1u)
        c = p[A + B];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k)
        v[k] = (k < A) ? a[k & 3u] : (k < A + B) ? ((k == A) ? b.x : b.y) : (k < cnt ? c : 0.0f);
}

// GLOBAL: p points to global memory, and the elements past the last full
// chunk of 8 (all of them when n < 8) are read by load_tail.
template <bool VEC, bool GLOBAL = false>
__device__ __forceinline__ float page_sum(const float* __restrict__ p,
                                          uint32_t n, int accum, float old)
{
    float s[8];
    if (n >= 8) {
        load8<VEC>(p, s);
    } else if constexpr (GLOBAL) {
        float v[8];
        load_tail(p, n, v);
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            s[k] = (k < n) ? v[k] : -0.0f;
    } else {
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            s[k] = (k < n) ? p[k] : -0.0f;
    }
    if (accum)
        s[0] = s[0] + old;
    uint32_t c = 8;
    for (; c + 8 <= n; c += 8) {
        float v[8];
        load8<VEC>(p + c, v);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s[k] = s[k] + v[k];
    }
    // Leftovers: element c + k joins slot (c + k) mod 8 == k.
    if constexpr (GLOBAL) {
        if (c < n) {
            float v[8];
            load_tail(p + c, n - c, v);
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k)
                if (c + k < n)
                    s[k] = s[k] + v[k];
        }
    } else {
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            if (c + k < n)
                s[k] = s[k] + p[c + k];
    }
    return slot_tree(s);
}

template <class Op, bool VEC, bool GLOBAL = false>
__device__ __forceinline__ float page_minmax(const float* __restrict__ p,
                                             uint32_t n, int accum, float old)
{
    AccMinMax<Op> acc(accum ? old : Op::identity());
    uint32_t c = 0;
    for (; c + 8 <= n; c += 8) {
        float v[8];
        load8<VEC>(p + c, v);
        acc.fold2(make_float4(v[0], v[1], v[2], v[3]),
                  make_float4(v[4], v[5], v[6], v[7]));
    }
    if constexpr (GLOBAL) {
        if (c < n) {
            float v[8];
            load_tail(p + c, n - c, v);
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k)
                if (c + k < n)
                    acc.fold_scalar(v[k]);
        }
    } else {
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            if (c + k < n)
                acc.fold_scalar(p[c + k]);
    }
    return acc.collapse();
}

template <class Op, bool VEC>
__global__ __launch_bounds__(kBlock) void rows_thread_kernel(
    const float* __restrict__ x, uint64_t rows, uint32_t n, uint64_t ld,
    float* __restrict__ out, int accum)
{
    const uint64_t stride = (uint64_t)gridDim.x * kBlock;
    for (uint64_t r = (uint64_t)blockIdx.x * kBlock + threadIdx.x; r < rows;
         r += stride) {
        const float* __restrict__ p = x + r * ld;
        const float old = accum ? out[r] : 0.0f;
        if constexpr (__is_same(Op, OpSum))
            out[r] = page_sum<VEC, true>(p, n, accum, old);
        else
            out[r] = page_minmax<Op, VEC, true>(p, n, accum, old);
    }
}

// Rows of N < 8 elements, already in registers: the arithmetic page_sum
// and page_minmax apply to such rows.  Each element sits alone in its
// slot (slot 0 also takes the old value under accum) before the slot tree;
// max / min fold the elements one by one.
template <class Op, int N, bool ACC>
__device__ __forceinline__ float short_row(const float v[N], float old)
{
    if constexpr (__is_same(Op, OpSum)) {
        float s[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s[k] = (k < N) ? v[k < N ? k : 0] : -0.0f;
        if (ACC)
            s[0] = s[0] + old;
        return slot_tree(s);
    } else {
        AccMinMax<Op> acc(ACC ? old : Op::identity());
#pragma unroll
        for (int k = 0; k < N; ++k)
            acc.fold_scalar(v[k]);
        return acc.collapse();
    }
}

#ifndef RED_ROWS_SHORT_PER_THREAD
#define RED_ROWS_SHORT_PER_THREAD 8
#endif
#ifndef RED_ROWS_SHORT_WG_PER_CU
#define RED_ROWS_SHORT_WG_PER_CU 8
#endif
constexpr int kShortRowsPerThread = RED_ROWS_SHORT_PER_THREAD;
constexpr uint64_t kShortWgPerCu = RED_ROWS_SHORT_WG_PER_CU;
constexpr uint64_t kShortRowMax = 4; // rows this short take the short-row kernel

// Rows of N = 1 to 4 elements.  One row per thread would give each
// workgroup a few KiB to read and the grid hundreds of thousands of
// workgroups; instead each thread takes kShortRowsPerThread rows per step
// (rows base, base + 256, ..., so that every load instruction of a wave
// reads 64 neighbouring rows), requests all their elements (and, under
// accum, their old values) before reducing any, and a grid of a few
// workgroups per CU walks the steps grid-stride.  N and accum are template
// parameters, so that the loads of a step form one straight run.
// (Measured on MI355X, row sums over 256 MiB from HBM: 1-element rows
// 80 us instead of 175 us one row per thread, 2 to 4 elements 55-65 us
// instead of 69-99 us; 5 to 7 elements were ~2 us slower this way than one
// row per thread, so they stay with rows_thread.  4 and 16 rows per thread,
// and 2 or 4 workgroups per CU, were no faster.)
template <class Op, int N, bool ACC>
__global__ __launch_bounds__(kBlock) void rows_short_kernel(
    const float* __restrict__ x, uint64_t rows, uint64_t ld,
    float* __restrict__ out)
{
    constexpr int RPT = kShortRowsPerThread;
    const uint64_t span = (uint64_t)kBlock * RPT;
    for (uint64_t base = (uint64_t)blockIdx.x * span + threadIdx.x; base < rows;
         base += (uint64_t)gridDim.x * span) {
        float v[RPT][N];
        float old[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const uint64_t r = base + (uint64_t)j * kBlock;
            const uint64_t rr = r < rows ? r : base; // a row that exists
            const float* __restrict__ p = x + rr * ld;
#pragma unroll
            for (int k = 0; k < N; ++k)
                v[j][k] = __builtin_nontemporal_load(p + k);
            old[j] = ACC ? out[rr] : 0.0f;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const uint64_t r = base + (uint64_t)j * kBlock;
            if (r < rows)
                out[r] = short_row<Op, N, ACC>(v[j], old[j]);
        }
    }
}

constexpr uint32_t kTileThreads = 128; // threads of the tile kernel
constexpr uint32_t kTileRows = 128;    // rows staged in LDS per step
constexpr int kTileBatch = 8;          // loads in flight per thread while staging
constexpr uint64_t kDirectRowMax = 16; // rows this short are read by their thread directly

// Rows of 17 to 64 elements: the workgroup copies TR rows at a time into
// LDS with coalesced loads, each row at an odd stride so that the threads'
// row reads hit distinct banks; then thread t reduces rows t, t + 128, ...
// of the tile, each in the page's order.  With a short row stride (span,
// below) the tile is read as one contiguous run, from its first
// row's first element to its last row's last valid element, in 16-byte
// non-temporal loads at any 4-byte alignment (gfx950 reads unaligned
// multi-dword vectors from global memory); longer strides read each row's
// whole vectors and then its last n % 4 elements.  (Measured on MI355X, 256 MiB of rows from
// HBM: 31-element rows 260 us read directly by their thread, 52 us staged;
// 33- to 64-element rows 84-204 us direct, 47-57 us staged.  Rows of up to
// 16 elements are faster read directly: 51.5 us against 58.3 at n = 16.)
// floor(e / d) for d = ld or n / 4 is computed as (e * inv_d) >> 32 with
// inv_d = ceil(2^32 / d), exact for e < 2^14 and d <= 128 (checked
// exhaustively).
// Staging reads the whole span, padding included, when the row stride is
// at most 64 elements, or at most 128 with padding of at most an eighth of
// the row.  (Measured on MI355X, 256 MiB of 64-element rows: stride 65
// read element by element 80.9 us, stride 68 75.5 us, against 52.0 us for
// contiguous rows.)
__host__ inline bool rows_span(uint64_t n, uint64_t ld)
{
    return ld <= kThreadRowMax || (ld <= 2 * kThreadRowMax && (ld - n) * 8 <= n);
}

// The tile's row stride: odd, so that the threads' row reads hit distinct
// LDS banks.  A span of odd stride goes to LDS unchanged, padding and all
// (copied, never read), at its own stride.  A span of even stride keeps
// its padding at stride ld + 1 when the padding is at most an eighth of
// the row, which spares the copy a padding test per element; otherwise
// the padding is dropped and the stride is n | 1.  (Measured on MI355X,
// 256 MiB of rows, padding dropped -> kept: 17 of stride 33 52.0 -> 47.2
// us; 64 of stride 68 61.9 -> 54.5 us, 64 of stride 72 61.8 -> 54.1 us;
// but 50 of stride 64 51.1 -> 55.1 us.)
__host__ __device__ inline uint32_t tile_stride(uint64_t n, uint64_t ld, int span)
{
    if (!span)
        return (uint32_t)(n | 1u);
    if (ld & 1u)
        return (uint32_t)ld;
    return (ld - n) * 8 <= n ? (uint32_t)(ld + 1) : (uint32_t)(n | 1u);
}

// Copies the span of T rows of stride L <= 128 (from the first element to
// the last row's n-th) into the LDS tile, span row i at tile + i * stride,
// in 16-byte loads at any 4-byte alignment.  PAD: the L - n padding
// elements of each row are dropped (stride >= n); otherwise every element
// is copied (stride > L).  PIECE = 4 (L a multiple of 4): no 16-byte
// vector of the span crosses a row, so each goes to one row at one
// offset; PIECE = 2 (L even): each half of a vector stays in one row;
// PIECE = 1: elements one at a time, moving to the next row at its end.
// (Measured on MI355X, 256 MiB of rows, elements one at a time -> PIECE 4:
// contiguous 64-element rows 52.2 -> 44.3 us, 60 of stride 64 52.9 -> 45.2
// us.)
template <bool PAD, int PIECE>
__device__ __forceinline__ void stage_span(const float* __restrict__ x, uint32_t T,
                                           uint32_t n, uint32_t L, uint64_t inv_ld,
                                           float* __restrict__ tile, uint32_t stride)
{
    typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
    const uint32_t t = threadIdx.x;
    const f4u* __restrict__ src = reinterpret_cast<const f4u*>(x);
    const uint32_t run = (T - 1) * L + n; // elements of the span
    const uint32_t nv = run / 4;
    for (uint32_t f0 = 0; f0 < nv; f0 += kTileBatch * kTileThreads) {
        // Unconditional loads (past the end: vector 0 again, not stored) so
        // that the whole batch is in flight at once.
        f4u v[kTileBatch];
#pragma unroll
        for (int b = 0; b < kTileBatch; ++b) {
            const uint32_t f = f0 + b * kTileThreads + t;
            v[b] = __builtin_nontemporal_load(src + (f < nv ? f : 0));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < kTileBatch; ++b) {
            const uint32_t f = f0 + b * kTileThreads + t;
            if (f < nv) {
                const uint32_t e = 4 * f;
                uint32_t row = (uint32_t)(((uint64_t)e * inv_ld) >> 32);
                uint32_t col = e - row * L;
                if constexpr (PIECE == 4) {
                    float* __restrict__ d = tile + row * stride + col;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (!PAD || col + c < n)
                            d[c] = v[b][c];
                } else if constexpr (PIECE == 2) {
#pragma unroll
                    for (int h = 0; h < 4; h += 2) {
                        if (h == 2) {
                            col += 2;
                            if (col == L) {
                                col = 0;
                                ++row;
                            }
                        }
                        float* __restrict__ d = tile + row * stride + col;
                        if (!PAD || col < n)
                            d[0] = v[b][h];
                        if (!PAD || col + 1 < n)
                            d[1] = v[b][h + 1];
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (!PAD || col < n)
                            tile[row * stride + col] = v[b][c];
                        if (++col == L) {
                            col = 0;
                            ++row;
                        }
                    }
                }
            }
        }
    }
    for (uint32_t e = 4 * nv + t; e < run; e += kTileThreads) {
        const uint32_t row = (uint32_t)(((uint64_t)e * inv_ld) >> 32);
        const uint32_t col = e - row * L;
        if (!PAD || col < n)
            tile[row * stride + col] = x[e];
    }
}

// The span copied as it stands, when the row stride L is odd and serves as
// the tile's row stride too: element e of the span lands at tile[e], so
// whole 16-byte vectors go to LDS unchanged (the padding between rows is
// copied and never read).  (Measured on MI355X, 256 MiB of rows: 63
// elements 54.5 -> 45.4 us, 64 of stride 65 68.6 -> 52.1 us.)
__device__ __forceinline__ void stage_span_direct(const float* __restrict__ x, uint32_t T,
                                                  uint32_t n, uint32_t L,
                                                  float* __restrict__ tile)
{
    typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    const uint32_t t = threadIdx.x;
    const f4u* __restrict__ src = reinterpret_cast<const f4u*>(x);
    f4* __restrict__ dstv = reinterpret_cast<f4*>(tile);
    const uint32_t run = (T - 1) * L + n;
    const uint32_t nv = run / 4;
    for (uint32_t f0 = 0; f0 < nv; f0 += kTileBatch * kTileThreads) {
        f4u v[kTileBatch];
#pragma unroll
        for (int b = 0; b < kTileBatch; ++b) {
            const uint32_t f = f0 + b * kTileThreads + t;
            v[b] = __builtin_nontemporal_load(src + (f < nv ? f : 0));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < kTileBatch; ++b) {
            const uint32_t f = f0 + b * kTileThreads + t;
            if (f < nv)
                dstv[f] = v[b];
        }
    }
    for (uint32_t e = 4 * nv + t; e < run; e += kTileThreads)
        tile[e] = x[e];
}

// stage_span with the widest piece the row stride allows (ld is even here:
// odd strides go to LDS unchanged).
template <bool PAD>
__device__ __forceinline__ void span_copy(const float* __restrict__ x, uint32_t T,
                                          uint32_t n, uint32_t L, uint64_t inv_ld,
                                          float* __restrict__ tile, uint32_t stride)
{
    if (L % 4 == 0)
        stage_span<PAD, 4>(x, T, n, L, inv_ld, tile, stride);
    else if (L % 2 == 0)
        stage_span<PAD, 2>(x, T, n, L, inv_ld, tile, stride);
    else
        stage_span<PAD, 1>(x, T, n, L, inv_ld, tile, stride);
}

// Rows too far apart for a span: each row's whole 16-byte vectors (n / 4
// of them, at any 4-byte alignment) and then its n % 4 last elements one
// at a time, so nothing past a row's n-th element is read.  (Measured on
// MI355X, 256 MiB of rows, element loads -> vectors: 64 of stride 80 77.0
// -> 45.0 us, 48 of stride 100 43.5 -> 35.1 us.)
__device__ __forceinline__ void stage_rows(const float* __restrict__ x, uint32_t T,
                                           uint32_t n, uint64_t ld,
                                           float* __restrict__ tile, uint32_t stride)
{
    typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
    const uint32_t t = threadIdx.x;
    const uint32_t nw = n / 4; // at least 4: n > 16
    const uint64_t inv_nw = ((1ull << 32) + nw - 1) / nw;
    const uint32_t units = T * nw;
    // The last n % 4 elements of each row (T * (n % 4) <= 3 * kTileThreads
    // of them): requested first, stored after the vectors.
    static_assert(kTileRows <= kTileThreads, "three leftover elements per thread at most");
    const uint32_t rem = n - 4 * nw;
    float rv[3];
    uint32_t rdst[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const uint32_t e = t + (uint32_t)k * kTileThreads;
        const bool ok = e < T * rem;
        const uint32_t row = rem == 1 ? e : (rem == 2 ? e >> 1 : (e * 43691u) >> 17); // e / rem, e < 2^15
        const uint32_t col = 4 * nw + (e - row * rem);
        rv[k] = x[ok ? row * ld + col : 0];
        rdst[k] = ok ? row * stride + col : ~0u;
    }
    for (uint32_t u0 = 0; u0 < units; u0 += kTileBatch * kTileThreads) {
        f4u v[kTileBatch];
#pragma unroll
        for (int b = 0; b < kTileBatch; ++b) {
            const uint32_t u = u0 + b * kTileThreads + t;
            const uint32_t uc = u < units ? u : 0; // past the end: vector 0 again
            const uint32_t row = (uint32_t)(((uint64_t)uc * inv_nw) >> 32);
            const uint32_t j = uc - row * nw;
            v[b] = __builtin_nontemporal_load(
                reinterpret_cast<const f4u*>(x + row * ld + 4 * j));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < kTileBatch; ++b) {
            const uint32_t u = u0 + b * kTileThreads + t;
            if (u < units) {
                const uint32_t row = (uint32_t)(((uint64_t)u * inv_nw) >> 32);
                const uint32_t j = u - row * nw;
                float* __restrict__ d = tile + row * stride + 4 * j;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    d[c] = v[b][c];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (rdst[k] != ~0u)
            tile[rdst[k]] = rv[k];
}

template <class Op>
__global__ __launch_bounds__(kTileThreads) void rows_tile_kernel(
    const float* __restrict__ x, uint64_t rows, uint32_t n, uint64_t ld,
    float* __restrict__ out, int accum, int span, uint64_t inv_ld,
    uint32_t TR)
{
    extern __shared__ __align__(16) float tile[];
    const uint32_t stride = tile_stride(n, ld, span);
    const uint32_t t = threadIdx.x;
    for (uint64_t r0 = (uint64_t)blockIdx.x * TR; r0 < rows; r0 += (uint64_t)gridDim.x * TR) {
        const uint32_t T = (rows - r0 < TR) ? (uint32_t)(rows - r0) : TR;
        if (span) {
            if (stride == ld)
                stage_span_direct(x + r0 * ld, T, n, (uint32_t)ld, tile);
            else if (stride == (ld | 1u))
                span_copy<false>(x + r0 * ld, T, n, (uint32_t)ld, inv_ld, tile, stride);
            else
                span_copy<true>(x + r0 * ld, T, n, (uint32_t)ld, inv_ld, tile, stride);
        } else {
            stage_rows(x + r0 * ld, T, n, ld, tile, stride);
        }
        __syncthreads();
        for (uint32_t i = t; i < T; i += kTileThreads) {
            const uint64_t r = r0 + i;
            const float* p = tile + i * stride;
            const float old = accum ? out[r] : 0.0f;
            if constexpr (__is_same(Op, OpSum))
                out[r] = page_sum<false>(p, n, accum, old);
            else
                out[r] = page_minmax<Op, false>(p, n, accum, old);
        }
        __syncthreads(); // the next tile overwrites the LDS
    }
}

// ---- one wave per row -----------------------------------------------------

constexpr int kRowUnroll = 4; // float4 loads in flight per lane

// A lane's share of the row p[0..n): vectors lane, lane + L, ... with
// L = lanes; scalars before the first 16-byte boundary and after the last
// whole vector go to the lowest lanes.
template <class Op, int LANES>
__device__ __forceinline__ float row_lane_part(const float* __restrict__ p,
                                               uint64_t n, uint32_t lane,
                                               float first)
{
    const uint32_t head = head_count(p, n);
    const uint64_t nvec = (n - head) / 4;
    const float4* __restrict__ pv = reinterpret_cast<const float4*>(p + head);
    Acc<Op> acc(first);
    for (uint64_t base = lane; base < nvec; base += (uint64_t)LANES * kRowUnroll) {
        // Every lane loads kRowUnroll vectors (past the end it reloads
        // vector `base`, then folds the identity instead), so all loads are
        // issued before the first fold.
        float4 v[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const uint64_t idx = base + (uint64_t)u * LANES;
            v[u] = load_stream(pv + (idx < nvec ? idx : base));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u)
            if (base + (uint64_t)u * LANES >= nvec)
                v[u] = identity4<Op>();
#pragma unroll
        for (int u = 0; u < kRowUnroll; u += 2)
            acc.fold2(v[u], v[u + 1]);
    }
    if (lane < head)
        acc.fold_scalar(p[lane]);
    const uint64_t tail = head + 4 * nvec;
    if (tail + lane < n)
        acc.fold_scalar(p[tail + lane]);
    return acc.collapse();
}

// Rows of at most kPairRowMax elements go to the segmented kernel below.
constexpr uint64_t kPairRowMax = (uint64_t)kWave * kRowUnroll * 4; // 1024 elements

template <class Op>
__global__ __launch_bounds__(kBlock) void rows_wave_kernel(
    const float* __restrict__ x, uint64_t rows, uint64_t n, uint64_t ld,
    float* __restrict__ out, int accum)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t stride = (uint64_t)gridDim.x * kWaves;
    // r is uniform across the wave, so every lane runs every iteration.
    for (uint64_t r = (uint64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
         r < rows; r += stride) {
        const float first = (lane == 0 && accum) ? out[r] : Op::identity();
        const float v = row_lane_part<Op, kWave>(x + r * ld, n, lane, first);
        const float total = wave_reduce<Op>(v);
        if (lane == 0)
            out[r] = total;
    }
}

// Reduction over segments of G consecutive lanes (G = 16, 32 or 64) with the
// DPP steps of the wave reduction: the row shifts total each 16-lane row,
// row_bcast:15 joins rows (0,1) and (2,3), row_bcast:31 joins the halves.
// The segment's total lands in its last lane.
template <class Op, int G>
__device__ __forceinline__ float segment_reduce(float v)
{
    static_assert(G == 16 || G == 32 || G == 64, "segments of 16, 32 or 64 lanes");
    v = red_dev::dpp_fold<Op, 0x111, 0xf>(v); // row_shr:1
    v = red_dev::dpp_fold<Op, 0x112, 0xf>(v); // row_shr:2
    v = red_dev::dpp_fold<Op, 0x114, 0xf>(v); // row_shr:4
    v = red_dev::dpp_fold<Op, 0x118, 0xf>(v); // row_shr:8
    if constexpr (G >= 32)
        v = red_dev::dpp_fold<Op, 0x142, 0xa>(v); // row_bcast:15 -> rows 1, 3
    if constexpr (G == 64)
        v = red_dev::dpp_fold<Op, 0x143, 0xc>(v); // row_bcast:31 -> rows 2, 3
    return v;
}

// Rows of at most kPairRowMax elements.  G lanes share a row (G = 16 for
// n <= 256, 32 for n <= 512, 64 above), each holding up to U 16-byte
// vectors of it; a wave covers 64 / G rows per pass and P passes per step.
// Every load of a step -- vectors, and the scalars before the row's first
// 16-byte boundary and after its last whole vector -- is issued before any
// row is reduced.  Each workgroup owns a contiguous range of rows, a
// multiple of the rows its four waves cover in one step.  Lane 0 of a
// segment carries the old value under accum; the segment's last lane
// stores.
template <class Op, int G, int U, int P>
__global__ __launch_bounds__(kBlock) void rows_seg_kernel(
    const float* __restrict__ x, uint64_t rows, uint64_t n, uint64_t ld,
    float* __restrict__ out, int accum, uint64_t rows_per_wg)
{
    static_assert(U % 2 == 0, "vectors are folded in pairs");
    constexpr int kSegs = kWave / G;         // rows per pass of a wave
    constexpr int kRowsPerWave = kSegs * P;  // rows per step of a wave
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t seg = lane / G;
    const uint32_t q = lane % G;
    const uint64_t b0 = (uint64_t)blockIdx.x * rows_per_wg;
    const uint64_t b1 = (b0 + rows_per_wg < rows) ? b0 + rows_per_wg : rows;
    for (uint64_t base = b0 + (uint64_t)(threadIdx.x / kWave) * kRowsPerWave; base < b1;
         base += (uint64_t)kWaves * kRowsPerWave) {
        float4 v[P][U];
        float hv[P], tv[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const uint64_t r = base + (uint64_t)p * kSegs + seg;
            const bool valid = r < b1;
            const float* __restrict__ row = x + (valid ? r : base) * ld;
            const uint32_t h = head_count(row, n);
            const uint64_t nv = (n - h) / 4;
            const uint64_t tail = h + 4 * nv + q;
            const float4* __restrict__ rv = reinterpret_cast<const float4*>(row + h);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t idx = q + (uint64_t)u * G;
                v[p][u] = (valid && idx < nv) ? load_stream(rv + idx) : identity4<Op>();
            }
            hv[p] = (valid && q < h) ? row[q] : Op::identity();
            tv[p] = (valid && tail < n) ? row[tail] : Op::identity();
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const uint64_t r = base + (uint64_t)p * kSegs + seg;
            const bool valid = r < b1;
            Acc<Op> acc((q == 0 && accum && valid) ? out[r] : Op::identity());
#pragma unroll
            for (int u = 0; u < U; u += 2)
                acc.fold2(v[p][u], v[p][u + 1]);
            acc.fold_scalar(hv[p]); // the identity where a lane has none
            acc.fold_scalar(tv[p]);
            const float t = segment_reduce<Op, G>(acc.collapse());
            if (valid && q == G - 1)
                out[r] = t;
        }
    }
}

// Long rows, or too few rows to fill the GPU one wave per row: K
// workgroups share row r's sweeps in grid-stride order (workgroup k takes
// sweeps k, k + K, ...), streaming exactly as the 1-D kernel streams a
// vector.  With K = 1
// the workgroup writes out[r] itself (the old value folded first under
// accum); otherwise it writes partials[r * K + k] and rows_split_finish
// folds each row's K partials in index order.
template <class Op>
__global__ __launch_bounds__(kBlock) void rows_split_kernel(
    const float* __restrict__ x, uint64_t rows, uint64_t n, uint64_t ld,
    float* __restrict__ out, int accum, uint32_t K,
    float* __restrict__ partials)
{
    __shared__ float lds[kWaves];
    const uint64_t units = rows * K;
    for (uint64_t b = blockIdx.x; b < units; b += gridDim.x) {
        const uint64_t r = b / K;
        const uint32_t k = (uint32_t)(b % K);
        Acc<Op> acc(Op::identity());
        stream_chunk(x + r * ld, n, k, K, acc);
        const float total = block_reduce<Op>(acc.collapse(), lds);
        if (threadIdx.x == 0) {
            if (K == 1)
                out[r] = accum ? Op::apply(out[r], total) : total;
            else
                partials[b] = total;
        }
        __syncthreads(); // lds is rewritten by the next unit
    }
}

// One workgroup per row: the old value (under accum) first, then the row's
// K partials in index order, combined by the workgroup tree.
template <class Op>
__global__ __launch_bounds__(kBlock) void rows_split_finish_kernel(
    const float* __restrict__ partials, uint64_t rows, uint32_t K,
    float* __restrict__ out, int accum)
{
    __shared__ float lds[kWaves];
    for (uint64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float o = out[r]; // read unconditionally, so it is requested first
        const float v = fold_strided<Op>((threadIdx.x == 0 && accum) ? o : Op::identity(),
                                         partials + r * K, K);
        const float total = block_reduce<Op>(v, lds);
        if (threadIdx.x == 0)
            out[r] = total;
        __syncthreads();
    }
}

// Grid cap for the row kernels: the kernels loop over the remaining rows,
// so any row count stays within the 2^32 work-item limit of a launch.
constexpr uint64_t kMaxRowGrid = 1u << 20;

__host__ inline unsigned cap_grid(uint64_t g)
{
    return (unsigned)(g < kMaxRowGrid ? (g ? g : 1) : kMaxRowGrid);
}

// Contiguous row ranges, a multiple of the rows a workgroup covers in one
// step, for at most kRowsWgPerCu workgroups per CU.  (Measured on MI355X
// for 65536 rows of 1000 from HBM: 39.9 us at 16 per CU, 40.5 at 4, 41.5
// at 8; one workgroup per 8 rows took 41.0 us.)
template <class Op, int G, int U, int P>
void launch_seg(const float* x, uint64_t rows, uint64_t n, uint64_t ld,
                float* out, int accum, const DeviceInfo& dev, hipStream_t stream)
{
    constexpr uint64_t kStepRows = (uint64_t)kWaves * (kWave / G) * P;
    const uint64_t steps = (rows + kStepRows - 1) / kStepRows;
    const uint64_t cap = (uint64_t)dev.cus * kRowsWgPerCu;
    const uint64_t grid = steps < cap ? steps : cap;
    const uint64_t per = (steps + grid - 1) / grid * kStepRows;
    rows_seg_kernel<Op, G, U, P><<<(unsigned)((rows + per - 1) / per), kBlock, 0, stream>>>(
        x, rows, n, ld, out, accum, per);
}

template <class Op>
hipError_t launch_rows_op(const float* x, size_t rows, size_t n, size_t ld,
                          float* out, int accum, const DeviceInfo& dev,
                          const Workspace& ws, hipStream_t stream)
{
    if (n <= kShortRowMax) {
        const uint64_t span = (uint64_t)kBlock * kShortRowsPerThread;
        const uint64_t steps = (rows + span - 1) / span;
        const uint64_t cap = (uint64_t)dev.cus * kShortWgPerCu;
        const unsigned grid = (unsigned)(steps < cap ? steps : cap);
        auto go = [&](auto acc, auto plain) {
            if (accum)
                acc<<<grid, kBlock, 0, stream>>>(x, rows, ld, out);
            else
                plain<<<grid, kBlock, 0, stream>>>(x, rows, ld, out);
        };
        switch (n) {
        case 1: go(rows_short_kernel<Op, 1, true>, rows_short_kernel<Op, 1, false>); break;
        case 2: go(rows_short_kernel<Op, 2, true>, rows_short_kernel<Op, 2, false>); break;
        case 3: go(rows_short_kernel<Op, 3, true>, rows_short_kernel<Op, 3, false>); break;
        default: go(rows_short_kernel<Op, 4, true>, rows_short_kernel<Op, 4, false>); break;
        }
    } else if (n <= kDirectRowMax) {
        const unsigned grid = cap_grid((rows + kBlock - 1) / kBlock);
        const bool vec = (((uintptr_t)x & 15u) == 0) && (ld % 4 == 0);
        if (vec)
            rows_thread_kernel<Op, true><<<grid, kBlock, 0, stream>>>(
                x, rows, (uint32_t)n, ld, out, accum);
        else
            rows_thread_kernel<Op, false><<<grid, kBlock, 0, stream>>>(
                x, rows, (uint32_t)n, ld, out, accum);
    } else if (n <= kThreadRowMax) {
        // A multiple of 4 rows per tile keeps every tile of 16-byte aligned,
        // contiguous rows aligned; TR * ld <= 2^14 keeps the row index
        // arithmetic exact on the span path.
        const uint32_t TR = kTileRows;
        const uint64_t tiles = (rows + TR - 1) / TR;
        const uint64_t cap = (uint64_t)dev.cus * kRowsWgPerCu;
        const unsigned grid = (unsigned)(tiles < cap ? tiles : cap);
        const int span = rows_span(n, ld);
        const uint64_t inv_ld = ((1ull << 32) + ld - 1) / ld;
        const size_t lds = (size_t)TR * tile_stride(n, ld, span) * sizeof(float);
        rows_tile_kernel<Op><<<grid, kTileThreads, lds, stream>>>(
            x, rows, (uint32_t)n, ld, out, accum, span, inv_ld, TR);
    } else if (n <= kPairRowMax) {
        // <G lanes per row, U vectors per lane and row, P rows per segment>:
        // 4 * G * U >= n covers the row; U * P = 8 loads per lane in flight.
        if (n <= 128)
            launch_seg<Op, 16, 2, 4>(x, rows, n, ld, out, accum, dev, stream);
        else if (n <= 256)
            launch_seg<Op, 16, 4, 2>(x, rows, n, ld, out, accum, dev, stream);
        else if (n <= 512)
            launch_seg<Op, 32, 4, 2>(x, rows, n, ld, out, accum, dev, stream);
        else
            launch_seg<Op, 64, 4, 2>(x, rows, n, ld, out, accum, dev, stream);
    } else if (n <= kWaveRowMax && rows >= (size_t)dev.cus * kRowsWavePerCu) {
        const unsigned grid = cap_grid((rows + kWaves - 1) / kWaves);
        rows_wave_kernel<Op><<<grid, kBlock, 0, stream>>>(x, rows, n, ld, out,
                                                          accum);
    } else {
        const uint32_t K = rows_chunks(x, rows, n, dev);
        if (K > 1 && (size_t)rows * K * sizeof(float) > ws.partial_bytes)
            return hipErrorInvalidValue;
        float* partials = static_cast<float*>(ws.partials);
        rows_split_kernel<Op><<<cap_grid(rows * K), kBlock, 0, stream>>>(
            x, rows, n, ld, out, accum, K, partials);
        if (K > 1)
            rows_split_finish_kernel<Op><<<cap_grid(rows), kBlock, 0, stream>>>(
                partials, rows, K, out, accum);
    }
    return hipGetLastError();
}

} // namespace

uint32_t rows_chunks(const float* x, size_t rows, size_t n, const DeviceInfo& dev)
{
    if (n <= kPairRowMax || (n <= kWaveRowMax && rows >= (size_t)dev.cus * kRowsWavePerCu))
        return 0; // not the split kernel
    const uint64_t target = (uint64_t)dev.cus * kStreamWgPerCu;
    if (rows >= target)
        return 1;
    uint64_t K = (target + rows - 1) / rows;
    const uint64_t sweeps = sweep_count(x, n); // the first row's; others differ by < 1
    if (K > sweeps)
        K = sweeps;
    return (uint32_t)(K < 1 ? 1 : K);
}

hipError_t launch_rows(OpKind op, const float* x, size_t rows, size_t n,
                       size_t ld, float* out, int accum, const DeviceInfo& dev,
                       const Workspace& ws, hipStream_t stream)
{
    switch (op) {
    case OpKind::Sum: return launch_rows_op<OpSum>(x, rows, n, ld, out, accum, dev, ws, stream);
    case OpKind::Max: return launch_rows_op<OpMax>(x, rows, n, ld, out, accum, dev, ws, stream);
    case OpKind::Min: return launch_rows_op<OpMin>(x, rows, n, ld, out, accum, dev, ws, stream);
    }
    return hipErrorInvalidValue;
}

} // namespace red
