// rows.hip -- segmented reduction: out[r] = reduce(x[r*ld .. r*ld + n)).
//
// Three kernels, picked by the host from (rows, n) alone so that a given
// problem always runs the same code and gives the same bits:
//
//  * rows_thread (n <= 64): one thread per row, running the thread-scope
//    algorithm of the TVM TIRx page "reduction -> sm100_packed" (section
//    "Algorithm") in exactly its single-precision order: 8 slots take the
//    first 8 elements, each further full chunk of 8 is added slot by slot,
//    leftovers go one by one into slot i mod 8, and the slots collapse
//    (0,1)+=(2,3), (4,5)+=(6,7), (0,1)+=(4,5), result = slot 0 + slot 1.
//    accum adds the old destination into slot 0 first ("How inputs change
//    the algorithm").  max / min use four slots folded with max3 / min3.
//  * rows_wave2 (64 < n <= 1024): one wave64 per pair of rows; each lane
//    issues its four non-temporal 16-byte loads of both rows, keeps one
//    multi-wide accumulator per row, then two DPP wave reduces; lane 0
//    stores.  Each workgroup walks a contiguous range of rows.  No LDS, no
//    second pass.
//  * rows_wave: the same with one row per wave and any n, looping over the
//    row four vectors per lane at a time.
//  * rows_block: one 256-thread workgroup per row, for few very long rows.
#include "device.hpp"
#include "internal.hpp"

namespace red {
namespace {

constexpr uint64_t kThreadRowMax = 64; // rows this short go one per thread
constexpr uint64_t kWaveRowMax = 16384;
#ifndef RED_ROWS_WG_PER_CU
#define RED_ROWS_WG_PER_CU 16
#endif
constexpr uint64_t kRowsWgPerCu = RED_ROWS_WG_PER_CU;

__device__ __forceinline__ uint32_t head_count(const float* p, uint64_t n)
{
    const uint32_t mis = (uint32_t)(((uintptr_t)p >> 2) & 3u);
    const uint64_t h = (4u - mis) & 3u;
    return (uint32_t)(h < n ? h : n);
}

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

template <bool VEC>
__device__ __forceinline__ float page_sum(const float* __restrict__ p,
                                          uint32_t n, int accum, float old)
{
    float s[8];
    if (n >= 8) {
        load8<VEC>(p, s);
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
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k)
        if (c + k < n)
            s[k] = s[k] + p[c + k];
    s[0] = s[0] + s[2];
    s[1] = s[1] + s[3];
    s[4] = s[4] + s[6];
    s[5] = s[5] + s[7];
    s[0] = s[0] + s[4];
    s[1] = s[1] + s[5];
    return s[0] + s[1];
}

template <class Op, bool VEC>
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
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k)
        if (c + k < n)
            acc.fold_scalar(p[c + k]);
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
            out[r] = page_sum<VEC>(p, n, accum, old);
        else
            out[r] = page_minmax<Op, VEC>(p, n, accum, old);
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
        float4 v[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const uint64_t idx = base + (uint64_t)u * LANES;
            v[u] = idx < nvec ? load_stream(pv + idx) : identity4<Op>();
        }
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

// Two rows per wave at a time when both are short enough for one sweep:
// all of both rows' loads are issued before either row is reduced.
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

// Rows of at most kPairRowMax elements: each workgroup owns a contiguous
// range of rows (a multiple of 8), and in every step its four waves take
// the next eight rows, two consecutive rows per wave, loading both before
// reducing either.
template <class Op>
__global__ __launch_bounds__(kBlock) void rows_wave2_kernel(
    const float* __restrict__ x, uint64_t rows, uint64_t n, uint64_t ld,
    float* __restrict__ out, int accum, uint64_t rows_per_wg)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t b0 = (uint64_t)blockIdx.x * rows_per_wg;
    const uint64_t b1 = (b0 + rows_per_wg < rows) ? b0 + rows_per_wg : rows;
    for (uint64_t r = b0 + 2 * (threadIdx.x / kWave); r < b1; r += 2 * kWaves) {
        const bool second = r + 1 < b1; // uniform across the wave
        const float* __restrict__ p0 = x + r * ld;
        const float* __restrict__ p1 = second ? p0 + ld : p0;
        const uint32_t h0 = head_count(p0, n), h1 = head_count(p1, n);
        const uint64_t nv0 = (n - h0) / 4, nv1 = (n - h1) / 4;
        const float4* __restrict__ v0 = reinterpret_cast<const float4*>(p0 + h0);
        const float4* __restrict__ v1 = reinterpret_cast<const float4*>(p1 + h1);
        float4 a[kRowUnroll], b[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const uint64_t idx = lane + (uint64_t)u * kWave;
            a[u] = idx < nv0 ? load_stream(v0 + idx) : identity4<Op>();
            b[u] = (second && idx < nv1) ? load_stream(v1 + idx) : identity4<Op>();
        }
        Acc<Op> acc0((lane == 0 && accum) ? out[r] : Op::identity());
        Acc<Op> acc1((lane == 0 && accum && second) ? out[r + 1] : Op::identity());
#pragma unroll
        for (int u = 0; u < kRowUnroll; u += 2) {
            acc0.fold2(a[u], a[u + 1]);
            acc1.fold2(b[u], b[u + 1]);
        }
        if (lane < h0)
            acc0.fold_scalar(p0[lane]);
        if (lane < h1)
            acc1.fold_scalar(p1[lane]);
        if (h0 + 4 * nv0 + lane < n)
            acc0.fold_scalar(p0[h0 + 4 * nv0 + lane]);
        if (h1 + 4 * nv1 + lane < n)
            acc1.fold_scalar(p1[h1 + 4 * nv1 + lane]);
        const float t0 = wave_reduce<Op>(acc0.collapse());
        const float t1 = wave_reduce<Op>(acc1.collapse());
        if (lane == 0) {
            out[r] = t0;
            if (second)
                out[r + 1] = t1;
        }
    }
}

template <class Op>
__global__ __launch_bounds__(kBlock) void rows_block_kernel(
    const float* __restrict__ x, uint64_t rows, uint64_t n, uint64_t ld,
    float* __restrict__ out, int accum)
{
    __shared__ float lds[kWaves];
    for (uint64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float first = (threadIdx.x == 0 && accum) ? out[r] : Op::identity();
        const float v = row_lane_part<Op, kBlock>(x + r * ld, n, threadIdx.x, first);
        const float total = block_reduce<Op>(v, lds);
        if (threadIdx.x == 0)
            out[r] = total;
        __syncthreads(); // lds is rewritten by the next row
    }
}

// Grid cap for the row kernels: the kernels loop over the remaining rows,
// so any row count stays within the 2^32 work-item limit of a launch.
constexpr uint64_t kMaxRowGrid = 1u << 20;

__host__ inline unsigned cap_grid(uint64_t g)
{
    return (unsigned)(g < kMaxRowGrid ? (g ? g : 1) : kMaxRowGrid);
}

template <class Op>
hipError_t launch_rows_op(const float* x, size_t rows, size_t n, size_t ld,
                          float* out, int accum, const DeviceInfo& dev,
                          hipStream_t stream)
{
    if (n <= kThreadRowMax) {
        const unsigned grid = cap_grid((rows + kBlock - 1) / kBlock);
        const bool vec = (((uintptr_t)x & 15u) == 0) && (ld % 4 == 0);
        if (vec)
            rows_thread_kernel<Op, true><<<grid, kBlock, 0, stream>>>(
                x, rows, (uint32_t)n, ld, out, accum);
        else
            rows_thread_kernel<Op, false><<<grid, kBlock, 0, stream>>>(
                x, rows, (uint32_t)n, ld, out, accum);
    } else if (n <= kPairRowMax) {
        // Contiguous row ranges, a multiple of 8 rows each, for at most
        // kRowsWgPerCu workgroups per CU.  (Measured on MI355X for 65536
        // rows of 1000 from HBM: 39.9 us at 16 per CU, 40.5 at 4, 41.5 at
        // 8; one workgroup per 8 rows took 41.0 us.)
        const uint64_t steps = (rows + 2 * kWaves - 1) / (2 * kWaves);
        const uint64_t cap = (uint64_t)dev.cus * kRowsWgPerCu;
        const uint64_t grid = steps < cap ? steps : cap;
        const uint64_t per = (steps + grid - 1) / grid * (2 * kWaves);
        rows_wave2_kernel<Op><<<(unsigned)((rows + per - 1) / per), kBlock, 0, stream>>>(
            x, rows, n, ld, out, accum, per);
    } else if (n <= kWaveRowMax || rows >= (size_t)dev.cus * kRowsWavePerCu) {
        const unsigned grid = cap_grid((rows + kWaves - 1) / kWaves);
        rows_wave_kernel<Op><<<grid, kBlock, 0, stream>>>(x, rows, n, ld, out,
                                                          accum);
    } else {
        rows_block_kernel<Op><<<cap_grid(rows), kBlock, 0, stream>>>(
            x, rows, n, ld, out, accum);
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_rows(OpKind op, const float* x, size_t rows, size_t n,
                       size_t ld, float* out, int accum, const DeviceInfo& dev,
                       hipStream_t stream)
{
    switch (op) {
    case OpKind::Sum: return launch_rows_op<OpSum>(x, rows, n, ld, out, accum, dev, stream);
    case OpKind::Max: return launch_rows_op<OpMax>(x, rows, n, ld, out, accum, dev, stream);
    case OpKind::Min: return launch_rows_op<OpMin>(x, rows, n, ld, out, accum, dev, stream);
    }
    return hipErrorInvalidValue;
}

} // namespace red
