// reduce1d.hip -- 1-D fp32 vector -> scalar (sum / max / min, accum).
//
// One kernel per call.  Each thread streams its share of the vector in
// grid-stride order with 16-byte (dwordx4) loads, eight loads in flight,
// into a per-thread multi-wide accumulator; the accumulator collapses along
// a fixed tree, the wave reduces with DPP, the workgroup through LDS.
//
// The cross-workgroup step takes one of two forms:
//  * deterministic (default): every workgroup stores its partial, then
//    takes a ticket with a device-scope atomic; the workgroup that draws the
//    last ticket combines all partials in index order (folding the old
//    destination first under accum), writes the scalar and returns the
//    ticket counter to zero.  No second kernel launch.
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

constexpr int kUnroll = 8; // float4 loads in flight per thread

// Elements before the first 16-byte boundary of x (x is 4-byte aligned).
__host__ __device__ inline uint32_t head_count(const float* x, uint64_t n)
{
    const uint32_t mis = (uint32_t)(((uintptr_t)x >> 2) & 3u);
    const uint64_t h = (4u - mis) & 3u;
    return (uint32_t)(h < n ? h : n);
}

// Per-thread part: grid-stride stream + scalar head / tail, then the
// thread's collapse.  Returns the thread's value.
template <class Op>
__device__ __forceinline__ float thread_part(const float* __restrict__ x,
                                             uint64_t n, float first)
{
    const uint32_t head = head_count(x, n);
    const uint64_t nvec = (n - head) / 4;
    const uint64_t T = (uint64_t)gridDim.x * kBlock;
    const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const float4* __restrict__ xv = reinterpret_cast<const float4*>(x + head);

    Acc<Op> acc(first);
    uint64_t i = t;
    for (; i + (kUnroll - 1) * T < nvec; i += kUnroll * T) {
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = xv[i + u * T];
#pragma unroll
        for (int u = 0; u < kUnroll; u += 2)
            acc.fold2(v[u], v[u + 1]);
    }
    for (; i < nvec; i += T)
        acc.fold1(xv[i]);
    if (t == 0) {
        for (uint32_t k = 0; k < head; ++k)
            acc.fold_scalar(x[k]);
        for (uint64_t k = head + 4 * nvec; k < n; ++k)
            acc.fold_scalar(x[k]);
    }
    return acc.collapse();
}

template <class Op>
__global__ __launch_bounds__(kBlock) void reduce1d_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ out,
    int accum, float* __restrict__ partials, unsigned* __restrict__ ticket)
{
    __shared__ float lds[kWaves];
    __shared__ int s_last;

    const float r = block_reduce<Op>(thread_part<Op>(x, n, Op::identity()), lds);

    // Publish this workgroup's partial; the release half of the ticket RMW
    // orders the store before the ticket.
    if (threadIdx.x == 0) {
        partials[blockIdx.x] = r;
        const unsigned prev = __hip_atomic_fetch_add(
            ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last)
        return;

    // Last workgroup: every partial is visible after the acquire.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    float v = Op::identity();
    if (threadIdx.x == 0 && accum)
        v = *out; // the old destination takes the first slot
    for (unsigned k = threadIdx.x; k < gridDim.x; k += kBlock)
        v = Op::apply(v, partials[k]);
    const float total = block_reduce<Op>(v, lds);
    if (threadIdx.x == 0) {
        *out = total;
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Fold r into *out with maxNum / minNum semantics by compare-and-swap.
// Ends when the CAS succeeds or the stored value already is the result.
template <class Op>
__device__ void atomic_fold_cas(float* out, float r)
{
    unsigned* p = reinterpret_cast<unsigned*>(out);
    unsigned cur = __hip_atomic_load(p, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const unsigned want = __float_as_uint(Op::apply(__uint_as_float(cur), r));
        if (want == cur)
            return;
        if (__hip_atomic_compare_exchange_strong(
                p, &cur, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
}

template <class Op>
__global__ __launch_bounds__(kBlock) void reduce1d_atomic_kernel(
    const float* __restrict__ x, uint64_t n, float* __restrict__ out)
{
    __shared__ float lds[kWaves];
    const float r = block_reduce<Op>(thread_part<Op>(x, n, Op::identity()), lds);
    if (threadIdx.x == 0) {
        if constexpr (__is_same(Op, OpSum))
            unsafeAtomicAdd(out, r); // hardware global_atomic_add_f32
        else
            atomic_fold_cas<Op>(out, r);
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
                      unsigned grid, const Workspace& ws, hipStream_t stream)
{
    reduce1d_kernel<Op><<<grid, kBlock, 0, stream>>>(
        x, n, out, accum, static_cast<float*>(ws.partials), ws.tickets);
    return hipGetLastError();
}

template <class Op>
hipError_t launch_atomic(const float* x, size_t n, float* out, int accum,
                         unsigned grid, hipStream_t stream)
{
    if (!accum) {
        const unsigned ident = __builtin_bit_cast(
            unsigned, __is_same(Op, OpSum) ? -0.0f : __builtin_nanf(""));
        fill_u32_kernel<<<1, 64, 0, stream>>>(
            reinterpret_cast<unsigned*>(out), 1, ident);
    }
    reduce1d_atomic_kernel<Op><<<grid, kBlock, 0, stream>>>(x, n, out);
    return hipGetLastError();
}

} // namespace

unsigned reduce1d_grid(const float* x, size_t n, const DeviceInfo& dev)
{
    const uint64_t nvec = (n - head_count(x, n)) / 4;
    const uint64_t per_wg = (uint64_t)kBlock * kUnroll; // vectors per sweep
    uint64_t g = (nvec + per_wg - 1) / per_wg;
    const uint64_t cap = (uint64_t)dev.cus * kWgPerCu;
    if (g > cap)
        g = cap;
    if (g < 1)
        g = 1;
    return (unsigned)g;
}

hipError_t launch_reduce1d(OpKind op, const float* x, size_t n, float* out,
                           int accum, const DeviceInfo& dev,
                           const Workspace& ws, hipStream_t stream)
{
    const unsigned grid = reduce1d_grid(x, n, dev);
    if ((size_t)grid * sizeof(float) > ws.partial_bytes || ws.n_tickets < 1)
        return hipErrorInvalidValue;
    switch (op) {
    case OpKind::Sum: return launch_det<OpSum>(x, n, out, accum, grid, ws, stream);
    case OpKind::Max: return launch_det<OpMax>(x, n, out, accum, grid, ws, stream);
    case OpKind::Min: return launch_det<OpMin>(x, n, out, accum, grid, ws, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce1d_atomic(OpKind op, const float* x, size_t n,
                                  float* out, int accum, const DeviceInfo& dev,
                                  hipStream_t stream)
{
    const unsigned grid = reduce1d_grid(x, n, dev);
    switch (op) {
    case OpKind::Sum: return launch_atomic<OpSum>(x, n, out, accum, grid, stream);
    case OpKind::Max: return launch_atomic<OpMax>(x, n, out, accum, grid, stream);
    case OpKind::Min: return launch_atomic<OpMin>(x, n, out, accum, grid, stream);
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
