// device.hpp -- device-side building blocks shared by the libreduce kernels
// (gfx950 / CDNA4, wave64).
//
//  * operator traits for sum / max / min with their identities, and the
//    wave64 DPP reduction (from include/reduce_device.hpp);
//  * per-thread multi-wide accumulators (8 slots for sum, 4 for max / min)
//    and their fixed collapse trees, for streaming loops;
//  * the workgroup reduction over a 256-thread library workgroup;
//  * non-temporal 16-byte streaming loads.
//
// Everything here is deterministic: the combination order depends only on
// lane, wave and workgroup indices, never on timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "reduce_device.hpp"

namespace red {

constexpr int kBlock = 256;            // threads per workgroup
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kWaves = kBlock / kWave; // wavefronts per workgroup

// Operators and the wave reduction come from the public device header, so
// the library's kernels and kernels written against include/ share them.
using red_dev::OpMax;
using red_dev::OpMin;
using red_dev::OpSum;
using red_dev::wave_reduce;

// ---------------------------------------------------------------------------
// Per-thread accumulators.
//
// sum: eight fp32 slots.  A pair of float4 loads (8 elements) adds one
// element into each slot.  The collapse follows the tree of the TVM TIRx
// page "reduction -> sm100_packed" (section "Algorithm"): slots (0,1) take
// slots (2,3), slots (4,5) take slots (6,7), slots (0,1) take slots (4,5),
// and the result is slot 0 + slot 1.
//
// max / min: four slots, each folding two new elements per step with one
// three-input max3 / min3 (same page, "Algorithm", max / min).  The result
// does not depend on how elements are assigned to slots.
// ---------------------------------------------------------------------------
template <class Op>
struct Acc;

template <>
struct Acc<OpSum> {
    float s[8];
    __device__ __forceinline__ explicit Acc(float first)
    {
        s[0] = first;
#pragma unroll
        for (int k = 1; k < 8; ++k)
            s[k] = -0.0f;
    }
    __device__ __forceinline__ void fold2(const float4& a, const float4& b)
    {
        s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
        s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
    }
    __device__ __forceinline__ void fold1(const float4& a)
    {
        s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
    }
    __device__ __forceinline__ void fold_scalar(float v) { s[0] += v; }
    __device__ __forceinline__ float collapse() const
    {
        const float s02 = s[0] + s[2], s13 = s[1] + s[3];
        const float s46 = s[4] + s[6], s57 = s[5] + s[7];
        return (s02 + s46) + (s13 + s57);
    }
};

template <class Op>
struct AccMinMax {
    float m[4];
    __device__ __forceinline__ explicit AccMinMax(float first)
    {
        m[0] = first;
        m[1] = m[2] = m[3] = Op::identity();
    }
    __device__ __forceinline__ void fold2(const float4& a, const float4& b)
    {
        m[0] = Op::apply3(m[0], a.x, a.y);
        m[1] = Op::apply3(m[1], a.z, a.w);
        m[2] = Op::apply3(m[2], b.x, b.y);
        m[3] = Op::apply3(m[3], b.z, b.w);
    }
    __device__ __forceinline__ void fold1(const float4& a)
    {
        m[0] = Op::apply3(m[0], a.x, a.y);
        m[1] = Op::apply3(m[1], a.z, a.w);
    }
    __device__ __forceinline__ void fold_scalar(float v) { m[0] = Op::apply(m[0], v); }
    __device__ __forceinline__ float collapse() const
    {
        return Op::apply(Op::apply3(m[0], m[1], m[2]), m[3]);
    }
};

template <>
struct Acc<OpMax> : AccMinMax<OpMax> {
    using AccMinMax<OpMax>::AccMinMax;
};
template <>
struct Acc<OpMin> : AccMinMax<OpMin> {
    using AccMinMax<OpMin>::AccMinMax;
};

// A float4 of identities, for masked-off loads.
template <class Op>
__device__ __forceinline__ float4 identity4()
{
    const float e = Op::identity();
    return make_float4(e, e, e, e);
}

// ---------------------------------------------------------------------------
// Streaming loads.  Every input element is read exactly once, so the loads
// carry the non-temporal hint: the lines are not kept in L2 / Infinity
// Cache at the expense of data that is reused.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float4* p)
{
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 load_stream(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Streaming one contiguous vector.
//
// The vector's whole 16-byte vectors are cut into sweeps of kSweep vectors
// (kStreamUnroll loads in flight per thread, kBlock threads).  `chunks`
// workgroups share the vector in grid-stride order: workgroup `chunk` takes
// sweeps chunk, chunk + chunks, chunk + 2 chunks, ..., so at any moment the
// workgroups read neighbouring 32 KiB pieces of one window of the vector.
// The partial last sweep goes to the workgroup whose turn it is; the scalars
// before the first 16-byte boundary and after the last whole vector go to
// thread 0 of chunk 0.  (Measured on MI355X at two workgroups per CU, event
// per call: 64 MiB 12.8 us against 13.4 us when each workgroup streamed one
// contiguous chunk, 4 GiB 605 against 617 us.  At eight workgroups per CU
// the grid-stride walk was far slower, ~5 TB/s.)
// ---------------------------------------------------------------------------
#ifndef RED_STREAM_UNROLL
#define RED_STREAM_UNROLL 8
#endif
constexpr int kStreamUnroll = RED_STREAM_UNROLL;                 // loads in flight per thread
constexpr uint64_t kSweep = (uint64_t)kBlock * kStreamUnroll;    // vectors per workgroup sweep

// Elements before the first 16-byte boundary of x (x is 4-byte aligned).
__host__ __device__ inline uint32_t head_count(const float* x, uint64_t n)
{
    const uint32_t mis = (uint32_t)(((uintptr_t)x >> 2) & 3u);
    const uint64_t h = (4u - mis) & 3u;
    return (uint32_t)(h < n ? h : n);
}

// Whole sweeps of the vector x[0, n).
__host__ __device__ inline uint64_t sweep_count(const float* x, uint64_t n)
{
    return ((n - head_count(x, n)) / 4 + kSweep - 1) / kSweep;
}

// TH threads per workgroup with U loads in flight each cover one sweep
// (TH * U == kSweep): 256 threads with 8 loads (the default) or 512 with 4.
template <int TH = kBlock, int U = kStreamUnroll, class AccT>
__device__ __forceinline__ void stream_chunk(const float* __restrict__ x,
                                             uint64_t n, uint64_t chunk,
                                             uint64_t chunks, AccT& acc)
{
    static_assert((uint64_t)TH * U == kSweep && U % 2 == 0, "one sweep per step, loads in pairs");
    const uint32_t head = head_count(x, n);
    const uint64_t nvec = (n - head) / 4;
    const float4* __restrict__ xv = reinterpret_cast<const float4*>(x + head);
    const uint64_t step = chunks * kSweep;

    uint64_t i = chunk * kSweep + threadIdx.x;
    for (; i + (uint64_t)(U - 1) * TH < nvec; i += step) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_stream(xv + i + (uint64_t)u * TH);
        // All loads of the sweep are issued before the first fold (left to
        // itself the scheduler interleaves max3 / min3 folds with the loads
        // and waits for the first load before issuing the rest).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; u += 2)
            acc.fold2(v[u], v[u + 1]);
    }
    // The partial last sweep, if it is this workgroup's turn (otherwise i is
    // already past the end).
    for (; i < nvec; i += TH)
        acc.fold1(load_stream(xv + i));
    if (chunk == 0 && threadIdx.x == 0) {
        for (uint32_t k = 0; k < head; ++k)
            acc.fold_scalar(x[k]);
        for (uint64_t k = head + 4 * nvec; k < n; ++k)
            acc.fold_scalar(x[k]);
    }
}

// ---------------------------------------------------------------------------
// Streaming one long vector region by region.
//
// MI355X dispatches the workgroups of a grid to its kXcds XCDs round-robin
// by linear index, each XCD with its own L2.  Here the vector's sweeps are
// cut into kXcds contiguous regions of equal length (the last one shorter),
// workgroup b serves region b mod kXcds, and the gridDim.x / kXcds
// workgroups of one region take its sweeps in grid-stride order.  So each
// XCD streams one contiguous stretch of the vector.  The partial last
// sweep goes to the workgroup whose turn it is; the scalars before the
// first 16-byte boundary and after the last whole vector go to thread 0 of
// workgroup 0.  gridDim.x must be a multiple of kXcds.  (Measured on MI355X
// with a read-only sink, 4 GiB: one workgroup per CU, 8 loads in flight,
// regions 577 us = 7.44 TB/s; the same grid in plain grid-stride order 589
// us; two workgroups per CU in grid-stride order 600 us; 16, 32 or 256
// regions 582, 589, 598 us.  1 GiB 145.5 against 153.6 us, 256 MiB 38.7
// against 39.9 us.  Shorter vectors run the plain walk: see stream_shape.)
// ---------------------------------------------------------------------------
constexpr uint32_t kXcds = 8;

template <class AccT>
__device__ __forceinline__ void stream_regions(const float* __restrict__ x,
                                               uint64_t n, AccT& acc)
{
    const uint32_t head = head_count(x, n);
    const uint64_t nvec = (n - head) / 4;
    const float4* __restrict__ xv = reinterpret_cast<const float4*>(x + head);
    const uint64_t per = gridDim.x / kXcds;   // workgroups per region
    const uint64_t region = blockIdx.x % kXcds;
    const uint64_t sweeps = (nvec + kSweep - 1) / kSweep;
    const uint64_t full = nvec / kSweep;      // sweeps of kSweep whole vectors
    const uint64_t len = (sweeps + kXcds - 1) / kXcds;
    const uint64_t first = region * len + blockIdx.x / kXcds;
    const uint64_t end = (region + 1) * len < sweeps ? (region + 1) * len : sweeps;
    const uint64_t stop = end < full ? end : full;

    uint64_t s = first;
    for (; s < stop; s += per) {
        const uint64_t i = s * kSweep + threadIdx.x;
        float4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = load_stream(xv + i + (uint64_t)u * kBlock);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; u += 2)
            acc.fold2(v[u], v[u + 1]);
    }
    // The partial last sweep (index `full`, present when nvec is not a
    // multiple of kSweep), if it lies in this region and is this
    // workgroup's turn.
    if (s == full && full < end)
        for (uint64_t i = full * kSweep + threadIdx.x; i < nvec; i += kBlock)
            acc.fold1(load_stream(xv + i));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        for (uint32_t k = 0; k < head; ++k)
            acc.fold_scalar(x[k]);
        for (uint64_t k = head + 4 * nvec; k < n; ++k)
            acc.fold_scalar(x[k]);
    }
}

// ---------------------------------------------------------------------------
// Short vectors in one workgroup, every load in flight at once.
//
// Up to kShortVecs whole 16-byte vectors (128 KiB): thread t loads vectors
// t, t + kShortBlock, ..., t + (kShortUnroll - 1) kShortBlock, all requested
// before the first fold (indices past the end load the last vector again and
// are not folded, which keeps the loads unconditional), then folds its valid
// ones in pairs in that order.  The scalars before the first 16-byte
// boundary and after the last whole vector go to thread 0.  One CU streams
// 128 KiB within the launch latency of a one-kernel call, so such a vector
// costs no more than a 32 KiB one and needs no second kernel.  (Measured on
// MI355X, one workgroup of 1024 threads against the two-kernel call, event
// per call, cold copies: 64 KiB 4.44 against 6.26 us, 128 KiB 4.40 against
// 6.28 us; 256 KiB took 6.5 us and 512 KiB 10.8 us in one workgroup, so
// longer vectors keep the grid.)
// ---------------------------------------------------------------------------
constexpr int kShortBlock = 1024;
constexpr int kShortUnroll = 8;
constexpr uint64_t kShortVecs = (uint64_t)kShortBlock * kShortUnroll;

template <class AccT>
__device__ __forceinline__ void stream_short(const float* __restrict__ x, uint64_t n,
                                             AccT& acc)
{
    const uint32_t head = head_count(x, n);
    const uint32_t nvec = (uint32_t)((n - head) / 4); // at most kShortVecs
    const float4* __restrict__ xv = reinterpret_cast<const float4*>(x + head);
    if (nvec > 0) {
        float4 v[kShortUnroll];
#pragma unroll
        for (int u = 0; u < kShortUnroll; ++u) {
            const uint32_t i = threadIdx.x + (uint32_t)u * kShortBlock;
            v[u] = load_stream(xv + (i < nvec ? i : nvec - 1));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kShortUnroll; u += 2) {
            const uint32_t i = threadIdx.x + (uint32_t)u * kShortBlock;
            if (i + kShortBlock < nvec)
                acc.fold2(v[u], v[u + 1]);
            else if (i < nvec)
                acc.fold1(v[u]);
        }
    }
    if (threadIdx.x == 0) {
        for (uint32_t k = 0; k < head; ++k)
            acc.fold_scalar(x[k]);
        for (uint64_t k = head + 4 * (uint64_t)nvec; k < n; ++k)
            acc.fold_scalar(x[k]);
    }
}

// Launch shape of a kernel that streams one vector, one workgroup per CU
// at most: vectors of at most kShortVecs whole 16-byte vectors run one
// workgroup of kShortBlock threads (stream_short); vectors of at least
// kRegionalMinBytes on a device whose CU count
// is a multiple of kXcds run workgroups of kBlock threads with
// kStreamUnroll loads in flight, region by region (stream_regions);
// shorter ones run workgroups of kWideBlock threads with kWideUnroll loads
// in flight, at most one per sweep, in plain grid-stride order
// (stream_chunk<kWideBlock, kWideUnroll>).  Both keep 32 KiB in flight per
// CU.  (Measured on MI355X with a read-only sink, µs per read, plain order
// on 512-thread workgroups / plain order on two 256-thread workgroups per
// CU / regions: 32 MiB 6.5 / 6.6 / 7.0, 64 MiB 11.0 / 11.2 / 11.4, 128 MiB
// 20.2 / 20.8 / 21.0, 256 MiB 39.1 / 40.3 / 38.5, 1 GiB 151 / 155 / 146,
// 4 GiB 596 / 604 / 580.)
#ifndef RED_REGIONAL_MIN_BYTES
#define RED_REGIONAL_MIN_BYTES (256ull << 20)
#endif
constexpr uint64_t kRegionalMinBytes = RED_REGIONAL_MIN_BYTES;
constexpr int kWideBlock = 512;  // threads per workgroup of the plain 1-D stream
constexpr int kWideUnroll = 4;   // its loads in flight per thread
static_assert((uint64_t)kWideBlock * kWideUnroll == kSweep, "one sweep per step");

struct StreamShape {
    unsigned grid = 1;
    bool regional = false;
    bool one_shot = false; // one workgroup of kShortBlock threads (stream_short)
    unsigned threads() const
    {
        return one_shot ? (unsigned)kShortBlock : regional ? (unsigned)kBlock : (unsigned)kWideBlock;
    }
};

inline StreamShape stream_shape(const float* x, uint64_t n, int cus)
{
    StreamShape sh;
    if ((n - head_count(x, n)) / 4 <= kShortVecs) {
        sh.one_shot = true;
        return sh;
    }
    const uint64_t sweeps = sweep_count(x, n);
    if (n * sizeof(float) >= kRegionalMinBytes && cus % (int)kXcds == 0 &&
        sweeps >= (uint64_t)cus) {
        sh.grid = (unsigned)cus;
        sh.regional = true;
        return sh;
    }
    const uint64_t g = sweeps < (uint64_t)cus ? sweeps : (uint64_t)cus;
    sh.grid = (unsigned)(g < 1 ? 1 : g);
    return sh;
}

// Folding, in index order, the values v[t], v[t + kBlock], v[t + 2 kBlock],
// ... (t = threadIdx.x, indices below count >= 1) into a starting value,
// with every load of the first kFinishBatch rounds issued before the first
// fold, so the fold waits for one memory round trip rather than one per
// round.  Lanes past the end load v[0] and fold the identity instead, which
// keeps the loads unconditional (a conditional load would be sunk next to
// its fold).  The result is the plain sequential fold, bit for bit.
constexpr int kFinishBatch = 4;

__device__ __forceinline__ void load_strided(const float* __restrict__ v,
                                             uint64_t count,
                                             float (&p)[kFinishBatch])
{
#pragma unroll
    for (int b = 0; b < kFinishBatch; ++b) {
        const uint64_t k = threadIdx.x + (uint64_t)b * kBlock;
        p[b] = v[k < count ? k : 0];
    }
}

template <class Op>
__device__ __forceinline__ float fold_loaded(float first,
                                             const float (&p)[kFinishBatch],
                                             const float* __restrict__ v,
                                             uint64_t count)
{
    float r = first;
#pragma unroll
    for (int b = 0; b < kFinishBatch; ++b) {
        const uint64_t k = threadIdx.x + (uint64_t)b * kBlock;
        r = Op::apply(r, k < count ? p[b] : Op::identity());
    }
    for (uint64_t k = threadIdx.x + (uint64_t)kFinishBatch * kBlock; k < count; k += kBlock)
        r = Op::apply(r, v[k]);
    return r;
}

template <class Op>
__device__ __forceinline__ float fold_strided(float first,
                                              const float* __restrict__ v,
                                              uint64_t count)
{
    float p[kFinishBatch];
    load_strided(v, count, p);
    // Keep the instruction scheduler from moving any use (and its wait)
    // above the last load.
    __builtin_amdgcn_sched_barrier(0);
    return fold_loaded<Op>(first, p, v, count);
}

// Workgroup reduction over the kWaves waves of a library workgroup: every
// wave reduces with DPP, lane 0 of wave w writes lds[w], and after the
// barrier every thread folds lds[0..kWaves) in wave order.  `lds` must not
// be reused before another barrier.
template <class Op>
__device__ __forceinline__ float block_reduce(float v, float* lds)
{
    return red_dev::block_reduce<Op, kWaves>(v, lds);
}

} // namespace red
