// reduce1d.hip -- 1-D fp32 vector -> scalar (sum / max / min, accum).
//
// One workgroup per compute unit streams the vector's 32 KiB sweeps with
// non-temporal 16-byte (dwordx4) loads: under 256 MiB, 512-thread
// workgroups with four loads in flight per thread take the sweeps in
// grid-stride order over the whole vector; from 256 MiB, 256-thread
// workgroups with eight take them region by region, one contiguous region
// per XCD (stream_shape, device.hpp).  Each thread folds its loads into a
// per-thread multi-wide accumulator, which collapses along a fixed tree;
// the wave reduces with DPP and the workgroup through LDS.
//
// The cross-workgroup step takes one of three forms:
//  * deterministic (default): every workgroup stores its partial; a second,
//    one-workgroup kernel combines the partials in index order (folding the
//    old destination first under accum) and writes the scalar.  (Measured
//    on MI355X for 64 MiB: 13.1 us per call, against 15-16 us for a single
//    kernel whose last-arriving workgroup finishes behind atomic counters.)
//  * fused: sum, max and min of the same vector from one read of it; each
//    result is bit-identical to the single-operation call's;
//  * atomic: every workgroup folds its partial into the destination with
//    one device-scope atomic, the structure of the block reduce in the
//    imxueqiu.com blog post on a Triton vector-sum kernel (warp reduce,
//    shared-memory combine, one atomic per block).
//
// The operation is the reduction of the TVM TIRx page "reduction ->
// sm100_packed" (introduction; "How inputs change the algorithm", accum),
// applied to a whole vector in HBM rather than to one thread's registers.
#include "device.hpp"
#include "internal.hpp"

namespace red {
namespace {

// The workgroup's share of x: region by region on kBlock threads (long
// vectors), else in grid-stride order over the whole vector on kWideBlock
// threads (stream_shape decides).
template <bool REGIONAL>
constexpr int kStreamThreads = REGIONAL ? kBlock : kWideBlock;

template <bool REGIONAL, class AccT>
__device__ __forceinline__ void stream_share(const float* __restrict__ x, uint64_t n,
                                             AccT& acc)
{
    if constexpr (REGIONAL)
        stream_regions(x, n, acc);
    else
        stream_chunk<kWideBlock, kWideUnroll>(x, n, blockIdx.x, gridDim.x, acc);
}

template <class Op, bool REGIONAL>
__device__ __forceinline__ float thread_part(const float* __restrict__ x,
                                             uint64_t n)
{
    Acc<Op> acc(Op::identity());
    stream_share<REGIONAL>(x, n, acc);
    return acc.collapse();
}

// Sum, max and min of one stream at once.  Each part is the accumulator the
// single-operation kernels use, fed the same elements in the same order, so
// each result equals the corresponding single-operation result bit for bit.
struct AccSumMaxMin {
    Acc<OpSum> sum;
    Acc<OpMax> max;
    Acc<OpMin> min;
    __device__ __forceinline__ AccSumMaxMin()
        : sum(OpSum::identity()), max(OpMax::identity()), min(OpMin::identity())
    {
    }
    __device__ __forceinline__ void fold2(const float4& a, const float4& b)
    {
        sum.fold2(a, b);
        max.fold2(a, b);
        min.fold2(a, b);
    }
    __device__ __forceinline__ void fold1(const float4& a)
    {
        sum.fold1(a);
        max.fold1(a);
        min.fold1(a);
    }
    __device__ __forceinline__ void fold_scalar(float v)
    {
        sum.fold_scalar(v);
        max.fold_scalar(v);
        min.fold_scalar(v);
    }
};

// The workgroup sum, max and min of (vs, vx, vn) behind one barrier: each
// is folded exactly as block_reduce folds it (DPP within the wave, then the
// waves in order), so the results equal three block_reduce calls bit for
// bit.  Only thread 0's results are meaningful.
template <int WAVES>
__device__ __forceinline__ void block_reduce_sum_max_min(float vs, float vx,
                                                         float vn,
                                                         float (*lds)[WAVES],
                                                         float* r)
{
    const float ws = wave_reduce<OpSum>(vs);
    const float wx = wave_reduce<OpMax>(vx);
    const float wn = wave_reduce<OpMin>(vn);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        lds[0][threadIdx.x / kWave] = ws;
        lds[1][threadIdx.x / kWave] = wx;
        lds[2][threadIdx.x / kWave] = wn;
    }
    __syncthreads();
    r[0] = lds[0][0];
    r[1] = lds[1][0];
    r[2] = lds[2][0];
#pragma unroll
    for (int k = 1; k < WAVES; ++k) {
        r[0] = OpSum::apply(r[0], lds[0][k]);
        r[1] = OpMax::apply(r[1], lds[1][k]);
        r[2] = OpMin::apply(r[2], lds[2][k]);
    }
}

// First pass: each workgroup writes its partial to partials[blockIdx.x].
// A grid of
// one workgroup (short vectors) is the whole call: it writes *out itself,
// with the old value folded first under accum, exactly as the finish
// kernel would, and no second kernel is launched.
template <class Op, bool REGIONAL>
__global__ __launch_bounds__(kStreamThreads<REGIONAL>) void reduce1d_stream_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ partials,
    float* __restrict__ out, int accum)
{
    constexpr int kW = kStreamThreads<REGIONAL> / kWave;
    __shared__ float lds[kW];
    const float r = red_dev::block_reduce<Op, kW>(thread_part<Op, REGIONAL>(x, n), lds);
    if (threadIdx.x == 0) {
        if (gridDim.x == 1)
            *out = accum ? Op::apply(*out, r) : r;
        else
            partials[blockIdx.x] = r;
    }
}

// A short vector in one workgroup (stream_short): the whole call, writing
// *out itself with the old value folded first under accum.
template <class Op>
__global__ __launch_bounds__(kShortBlock) void reduce1d_short_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ out, int accum)
{
    constexpr int kW = kShortBlock / kWave;
    __shared__ float lds[kW];
    Acc<Op> acc(Op::identity());
    stream_short(x, n, acc);
    const float r = red_dev::block_reduce<Op, kW>(acc.collapse(), lds);
    if (threadIdx.x == 0)
        *out = accum ? Op::apply(*out, r) : r;
}

// Second pass, one workgroup: combine the G partials in index order (each
// thread folds partials t, t + 256, ..., then the workgroup tree), with the
// old destination in the first slot under accum.  The old value and the
// partials are all requested before the first fold.  The kernel boundary
// makes the first pass's stores visible; no atomics are involved.
template <class Op>
__global__ __launch_bounds__(kBlock) void reduce1d_finish_kernel(
    const float* __restrict__ partials, unsigned G, float* __restrict__ out,
    int accum)
{
    __shared__ float lds[kWaves];
    const float o = *out; // read unconditionally, so it is requested first
    const float old = (threadIdx.x == 0 && accum) ? o : Op::identity();
    const float v = fold_strided<Op>(old, partials, G);
    const float total = block_reduce<Op>(v, lds);
    if (threadIdx.x == 0)
        *out = total;
}

// Fused first pass: partials[b], partials[G + b], partials[2G + b] receive
// workgroup b's sum, max and min.
template <bool REGIONAL>
__global__ __launch_bounds__(kStreamThreads<REGIONAL>) void reduce1d_summaxmin_stream_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ partials,
    float* __restrict__ out, int accum)
{
    constexpr int kW = kStreamThreads<REGIONAL> / kWave;
    __shared__ float lds[3][kW];
    AccSumMaxMin acc;
    stream_share<REGIONAL>(x, n, acc);
    float r[3];
    block_reduce_sum_max_min<kW>(acc.sum.collapse(), acc.max.collapse(),
                                 acc.min.collapse(), lds, r);
    if (threadIdx.x == 0) {
        if (gridDim.x == 1) { // the whole call, as for the single operations
            out[0] = accum ? OpSum::apply(out[0], r[0]) : r[0];
            out[1] = accum ? OpMax::apply(out[1], r[1]) : r[1];
            out[2] = accum ? OpMin::apply(out[2], r[2]) : r[2];
        } else {
            partials[blockIdx.x] = r[0];
            partials[gridDim.x + blockIdx.x] = r[1];
            partials[2 * gridDim.x + blockIdx.x] = r[2];
        }
    }
}

// Fused short vector in one workgroup: each result as the single-operation
// short kernel computes it.
__global__ __launch_bounds__(kShortBlock) void reduce1d_summaxmin_short_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ out, int accum)
{
    constexpr int kW = kShortBlock / kWave;
    __shared__ float lds[3][kW];
    AccSumMaxMin acc;
    stream_short(x, n, acc);
    float r[3];
    block_reduce_sum_max_min<kW>(acc.sum.collapse(), acc.max.collapse(),
                                 acc.min.collapse(), lds, r);
    if (threadIdx.x == 0) {
        out[0] = accum ? OpSum::apply(out[0], r[0]) : r[0];
        out[1] = accum ? OpMax::apply(out[1], r[1]) : r[1];
        out[2] = accum ? OpMin::apply(out[2], r[2]) : r[2];
    }
}

// Fused second pass: out[0] = sum, out[1] = max, out[2] = min, each folded
// exactly as the single-operation finish folds it.
__global__ __launch_bounds__(kBlock) void reduce1d_summaxmin_finish_kernel(
    const float* __restrict__ partials, unsigned G, float* __restrict__ out,
    int accum)
{
    __shared__ float lds[3][kWaves];
    const bool first = threadIdx.x == 0 && accum;
    const float os = out[0], ox = out[1], on = out[2]; // requested first
    float ps[kFinishBatch], px[kFinishBatch], pn[kFinishBatch];
    load_strided(partials, G, ps);
    load_strided(partials + G, G, px);
    load_strided(partials + 2 * G, G, pn);
    __builtin_amdgcn_sched_barrier(0); // every load above is issued before any fold
    const float vs = fold_loaded<OpSum>(first ? os : OpSum::identity(), ps, partials, G);
    const float vx = fold_loaded<OpMax>(first ? ox : OpMax::identity(), px, partials + G, G);
    const float vn = fold_loaded<OpMin>(first ? on : OpMin::identity(), pn, partials + 2 * G, G);
    float t[3];
    block_reduce_sum_max_min<kWaves>(vs, vx, vn, lds, t);
    if (threadIdx.x == 0) {
        out[0] = t[0];
        out[1] = t[1];
        out[2] = t[2];
    }
}

// Folding a workgroup's max / min into *out with device-scope atomics.
//
// Integer atomics order fp32 bit patterns like the floats themselves: for
// a non-negative r (sign bit clear) a signed-integer max (max) or min
// (min) of the two patterns is the float max / min, whatever the sign of
// the stored value; for a negative r the unsigned-integer min (max) or max
// (min) is.  So each workgroup needs one atomic, with no retry, provided
// the stored value is a number or a NaN that loses every comparison: a
// NaN with the sign bit set for max, clear for min.  The identity written
// when accum is off is such a NaN; an old value that is a NaN of the
// other sign (possible only under accum) is replaced by compare-and-swap
// first.  A NaN partial (every element of the workgroup's share NaN) is
// skipped, as maxNum / minNum ignore NaN operands.  Before its atomic a
// workgroup reads the stored value and skips the atomic when it would not
// change it.  +0 and -0 compare as the integers they are (max keeps +0,
// min keeps -0), an allowed choice for equal zeros.
template <class Op>
constexpr unsigned kLosingNaN = __is_same(Op, OpMax) ? 0xffc00000u : 0x7fc00000u;

template <class Op>
__device__ void atomic_fold_extreme(float* out, float r)
{
    if (__builtin_isnan(r))
        return;
    unsigned* p = reinterpret_cast<unsigned*>(out);
    unsigned cur = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // An old NaN of the winning sign: swap it for r (retrying while some
    // other workgroup changes the value first).
    while (__builtin_isnan(__uint_as_float(cur)) && (cur & 0x80000000u) != (kLosingNaN<Op> & 0x80000000u)) {
        if (__hip_atomic_compare_exchange_strong(p, &cur, __float_as_uint(r), __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
    if (__float_as_uint(Op::apply(__uint_as_float(cur), r)) == cur)
        return; // r would not change the stored value
    const unsigned bits = __float_as_uint(r);
    const bool neg = (bits & 0x80000000u) != 0;
    if constexpr (__is_same(Op, OpMax)) {
        if (!neg)
            __hip_atomic_fetch_max(reinterpret_cast<int*>(out), (int)bits, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_fetch_min(p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        if (!neg)
            __hip_atomic_fetch_min(reinterpret_cast<int*>(out), (int)bits, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_fetch_max(p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class Op, bool REGIONAL>
__global__ __launch_bounds__(kStreamThreads<REGIONAL>) void reduce1d_atomic_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ out)
{
    constexpr int kW = kStreamThreads<REGIONAL> / kWave;
    __shared__ float lds[kW];
    const float r = red_dev::block_reduce<Op, kW>(thread_part<Op, REGIONAL>(x, n), lds);
    if (threadIdx.x == 0) {
        if constexpr (__is_same(Op, OpSum))
            unsafeAtomicAdd(out, r); // hardware global_atomic_add_f32
        else
            atomic_fold_extreme<Op>(out, r);
    }
}

// The single-pass variant on a short vector: one workgroup (stream_short)
// and its one atomic.
template <class Op>
__global__ __launch_bounds__(kShortBlock) void reduce1d_atomic_short_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ out)
{
    constexpr int kW = kShortBlock / kWave;
    __shared__ float lds[kW];
    Acc<Op> acc(Op::identity());
    stream_short(x, n, acc);
    const float r = red_dev::block_reduce<Op, kW>(acc.collapse(), lds);
    if (threadIdx.x == 0) {
        if constexpr (__is_same(Op, OpSum))
            unsafeAtomicAdd(out, r);
        else
            atomic_fold_extreme<Op>(out, r);
    }
}

__global__ void fill_u32_kernel(unsigned* __restrict__ p, uint64_t count,
                                unsigned value)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        p[i] = value;
}

template <class Op>
hipError_t launch_det(const float* x, size_t n, float* out, int accum,
                      StreamShape sh, const Workspace& ws, hipStream_t stream)
{
    if (sh.one_shot) {
        reduce1d_short_kernel<Op><<<1, kShortBlock, 0, stream>>>(x, n, out, accum);
        return hipGetLastError();
    }
    float* partials = static_cast<float*>(ws.partials);
    const unsigned grid = sh.grid;
    if (sh.regional)
        reduce1d_stream_kernel<Op, true><<<grid, kBlock, 0, stream>>>(x, n, partials, out, accum);
    else
        reduce1d_stream_kernel<Op, false><<<grid, kWideBlock, 0, stream>>>(x, n, partials, out,
                                                                          accum);
    if (grid > 1)
        reduce1d_finish_kernel<Op><<<1, kBlock, 0, stream>>>(partials, grid, out, accum);
    return hipGetLastError();
}

template <class Op>
hipError_t launch_atomic(const float* x, size_t n, float* out, int accum,
                         StreamShape sh, hipStream_t stream)
{
    if (!accum) {
        // -0.0 for the sum; for max / min the NaN that loses every
        // integer comparison of atomic_fold_extreme.
        const unsigned ident = __is_same(Op, OpSum) ? 0x80000000u : kLosingNaN<Op>;
        fill_u32_kernel<<<1, 64, 0, stream>>>(
            reinterpret_cast<unsigned*>(out), 1, ident);
    }
    if (sh.one_shot)
        reduce1d_atomic_short_kernel<Op><<<1, kShortBlock, 0, stream>>>(x, n, out);
    else if (sh.regional)
        reduce1d_atomic_kernel<Op, true><<<sh.grid, kBlock, 0, stream>>>(x, n, out);
    else
        reduce1d_atomic_kernel<Op, false><<<sh.grid, kWideBlock, 0, stream>>>(x, n, out);
    return hipGetLastError();
}

} // namespace

// Launch shape of the deterministic 1-D kernels for x[0, n).
StreamShape reduce1d_shape(const float* x, size_t n, const DeviceInfo& dev)
{
    return stream_shape(x, n, dev.cus);
}

hipError_t launch_reduce1d_summaxmin(const float* x, size_t n, float* out,
                                     int accum, const DeviceInfo& dev,
                                     const Workspace& ws, hipStream_t stream)
{
    const StreamShape sh = reduce1d_shape(x, n, dev);
    const unsigned grid = sh.grid;
    if (sh.one_shot) {
        reduce1d_summaxmin_short_kernel<<<1, kShortBlock, 0, stream>>>(x, n, out, accum);
        return hipGetLastError();
    }
    if ((size_t)grid * 3 * sizeof(float) > ws.partial_bytes)
        return hipErrorInvalidValue;
    float* partials = static_cast<float*>(ws.partials);
    if (sh.regional)
        reduce1d_summaxmin_stream_kernel<true><<<grid, kBlock, 0, stream>>>(x, n, partials, out,
                                                                           accum);
    else
        reduce1d_summaxmin_stream_kernel<false><<<grid, kWideBlock, 0, stream>>>(x, n, partials,
                                                                                out, accum);
    if (grid > 1)
        reduce1d_summaxmin_finish_kernel<<<1, kBlock, 0, stream>>>(partials, grid, out, accum);
    return hipGetLastError();
}

unsigned reduce1d_grid(const float* x, size_t n, const DeviceInfo& dev)
{
    return reduce1d_shape(x, n, dev).grid;
}

hipError_t launch_reduce1d(OpKind op, const float* x, size_t n, float* out,
                           int accum, const DeviceInfo& dev,
                           const Workspace& ws, hipStream_t stream)
{
    const StreamShape sh = reduce1d_shape(x, n, dev);
    if ((size_t)sh.grid * sizeof(float) > ws.partial_bytes)
        return hipErrorInvalidValue;
    switch (op) {
    case OpKind::Sum: return launch_det<OpSum>(x, n, out, accum, sh, ws, stream);
    case OpKind::Max: return launch_det<OpMax>(x, n, out, accum, sh, ws, stream);
    case OpKind::Min: return launch_det<OpMin>(x, n, out, accum, sh, ws, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce1d_atomic(OpKind op, const float* x, size_t n,
                                  float* out, int accum, const DeviceInfo& dev,
                                  hipStream_t stream)
{
    // The stream kernels' launch shape: one workgroup per CU at most, so
    // at most one same-address atomic per CU (they serialize, ~9 ns each).
    // (Measured on MI355X, 64 MiB, median per call, one 256-thread
    // workgroup per CU against two: sum with accum 16.7 -> 13.9 us, without
    // 20.8 -> 18.2 us; max without accum 20.3 -> 18.1 us.)
    const StreamShape sh = stream_shape(x, n, dev.cus);
    switch (op) {
    case OpKind::Sum: return launch_atomic<OpSum>(x, n, out, accum, sh, stream);
    case OpKind::Max: return launch_atomic<OpMax>(x, n, out, accum, sh, stream);
    case OpKind::Min: return launch_atomic<OpMin>(x, n, out, accum, sh, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fill_u32(unsigned* p, size_t count, unsigned value,
                           hipStream_t stream)
{
    if (count == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((count + kBlock - 1) / kBlock);
    fill_u32_kernel<<<blocks, kBlock, 0, stream>>>(p, count, value);
    return hipGetLastError();
}

} // namespace red
