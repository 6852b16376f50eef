// device.hpp -- device-side building blocks shared by the libreduce kernels
// (gfx950 / CDNA4, wave64).
//
//  * operator traits for sum / max / min with their identities;
//  * per-thread multi-wide accumulators (8 slots for sum, 4 for max / min)
//    and their fixed collapse trees;
//  * a wave64 reduction built from DPP row shifts and row broadcasts;
//  * a workgroup reduction that combines the per-wave results through LDS
//    in wave order.
//
// Everything here is deterministic: the combination order depends only on
// lane, wave and workgroup indices, never on timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace red {

constexpr int kBlock = 256;            // threads per workgroup
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kWaves = kBlock / kWave; // wavefronts per workgroup

// ---------------------------------------------------------------------------
// Operators.  The identity of IEEE addition is -0.0 (x + -0.0 == x for every
// x, +0 included).  Under maxNum / minNum a quiet NaN is the identity:
// fmaxf(NaN, x) == x, and the result stays NaN only if every operand is NaN.
// ---------------------------------------------------------------------------
struct OpSum {
    static __device__ __forceinline__ float identity() { return -0.0f; }
    static __device__ __forceinline__ float apply(float a, float b) { return a + b; }
};

struct OpMax {
    static __device__ __forceinline__ float identity() { return __builtin_nanf(""); }
    static __device__ __forceinline__ float apply(float a, float b) { return fmaxf(a, b); }
    // Lowered to v_max3_f32.
    static __device__ __forceinline__ float apply3(float a, float b, float c)
    {
        return fmaxf(fmaxf(a, b), c);
    }
};

struct OpMin {
    static __device__ __forceinline__ float identity() { return __builtin_nanf(""); }
    static __device__ __forceinline__ float apply(float a, float b) { return fminf(a, b); }
    // Lowered to v_min3_f32.
    static __device__ __forceinline__ float apply3(float a, float b, float c)
    {
        return fminf(fminf(a, b), c);
    }
};

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
// Wave64 reduction with DPP.
//
// GFX9 DPP controls used: row_shr:k (0x110 + k) reads lane i-k of the same
// 16-lane row; row_bcast:15 (0x142) feeds lane 15 of each row to the next
// row; row_bcast:31 (0x143) feeds lane 31 to rows 2 and 3.  A lane whose
// source is outside the row, or whose row is masked off, receives `old`,
// which is set to the operator's identity (bound_ctrl off).
//
// After the four row shifts, lane 15 of each row holds that row's total;
// the two broadcasts fold row 0 into row 1, row 2 into row 3, then rows
// 0..1 into rows 2..3, leaving the wave total in lane 63.  Must be called
// with all 64 lanes active.
// ---------------------------------------------------------------------------
template <class Op, int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_fold(float v)
{
    const int t = __builtin_amdgcn_update_dpp(__float_as_int(Op::identity()),
                                              __float_as_int(v), CTRL,
                                              ROW_MASK, 0xf, false);
    return Op::apply(v, __int_as_float(t));
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float v)
{
    v = dpp_fold<Op, 0x111, 0xf>(v); // row_shr:1
    v = dpp_fold<Op, 0x112, 0xf>(v); // row_shr:2
    v = dpp_fold<Op, 0x114, 0xf>(v); // row_shr:4
    v = dpp_fold<Op, 0x118, 0xf>(v); // row_shr:8
    v = dpp_fold<Op, 0x142, 0xa>(v); // row_bcast:15 -> rows 1, 3
    v = dpp_fold<Op, 0x143, 0xc>(v); // row_bcast:31 -> rows 2, 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---------------------------------------------------------------------------
// Workgroup reduction: every wave reduces with DPP, lane 0 of wave w writes
// lds[w], and after the barrier every thread folds lds[0..kWaves) in wave
// order.  Returns the same value in every thread.  `lds` must not be reused
// before another barrier.
// ---------------------------------------------------------------------------
template <class Op>
__device__ __forceinline__ float block_reduce(float v, float* lds)
{
    const float w = wave_reduce<Op>(v);
    if ((threadIdx.x & (kWave - 1)) == 0)
        lds[threadIdx.x / kWave] = w;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k)
        r = Op::apply(r, lds[k]);
    return r;
}

} // namespace red
