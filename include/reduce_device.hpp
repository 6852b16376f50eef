// reduce_device.hpp -- device-side reductions for use inside HIP kernels on
// AMD Instinct MI355X (gfx950, wave64).  Header-only; include it from a
// .hip translation unit.
//
// Three scopes:
//
//   thread     thread_sum / thread_max / thread_min over a register array
//              float src[N] (N known at compile time) into one value, with
//              accum.  This is the thread-scope primitive of the TVM TIRx
//              docs page "reduction -> sm100_packed" (introduction; "What it
//              accepts": thread scope, a local 1-D fp32 source, a one-element
//              local destination) and its algorithm ("Algorithm"): sum keeps
//              eight slots that take the first eight elements, folds every
//              further chunk of eight slot by slot, adds leftovers into slot
//              i mod 8 and collapses (0,1)+=(2,3), (4,5)+=(6,7), (0,1)+=(4,5),
//              result = slot 0 + slot 1; max / min keep four slots folded with
//              three-input max3 / min3.  accum adds the old destination into
//              the first slot before anything else ("How inputs change the
//              algorithm").  Any N >= 1 is accepted (the page's fast path
//              needs N >= 8; shorter arrays fill unused slots with the
//              identity).  The sum is bit-for-bit the page's order in IEEE
//              single precision (no flush of subnormals).
//
//   wave       wave_sum / wave_max / wave_min: all 64 lanes of a wave
//              contribute one value each; every lane receives the result.
//              DPP row shifts and row broadcasts, fixed order.  Call with all
//              64 lanes active.
//
//   workgroup  block_sum / block_max / block_min<WAVES>: a workgroup of
//              WAVES wave64s (blockDim.x == 64 * WAVES); every thread
//              receives the result.  `lds` points to WAVES floats of
//              __shared__ memory that must not be touched again before the
//              next barrier.  Call from every thread of the workgroup.
//
// max / min follow IEEE-754-2008 maxNum / minNum: a quiet NaN operand is
// ignored and the result is NaN only if every operand is; a quiet NaN is
// therefore their identity.  The identity of the sum is -0.0.  Every result
// depends only on the inputs and their positions, never on timing.
#pragma once

#include <hip/hip_runtime.h>

namespace red_dev {

// ---------------------------------------------------------------------------
// Operators
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
// Thread scope
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ float thread_sum(const float (&src)[N],
                                            float old = 0.0f, bool accum = false)
{
    static_assert(N >= 1, "thread_sum needs at least one element");
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        s[k] = (k < N) ? src[k < N ? k : 0] : -0.0f;
    if (accum)
        s[0] = s[0] + old;
    constexpr int kEnd = (N >= 8) ? (N / 8) * 8 : 8; // first leftover element
#pragma unroll
    for (int c = 8; c + 8 <= N; c += 8)
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s[k] = s[k] + src[c + k];
#pragma unroll
    for (int i = kEnd; i < N; ++i)
        s[i - kEnd] = s[i - kEnd] + src[i];
    s[0] = s[0] + s[2];
    s[1] = s[1] + s[3];
    s[4] = s[4] + s[6];
    s[5] = s[5] + s[7];
    s[0] = s[0] + s[4];
    s[1] = s[1] + s[5];
    return s[0] + s[1];
}

template <class Op, int N>
__device__ __forceinline__ float thread_extreme(const float (&src)[N], float old,
                                                bool accum)
{
    static_assert(N >= 1, "thread reductions need at least one element");
    float m[4] = {accum ? old : Op::identity(), Op::identity(), Op::identity(),
                  Op::identity()};
    constexpr int kFull = (N / 8) * 8;
#pragma unroll
    for (int c = 0; c < kFull; c += 8)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m[k] = Op::apply3(m[k], src[c + 2 * k], src[c + 2 * k + 1]);
#pragma unroll
    for (int i = kFull; i < N; ++i)
        m[0] = Op::apply(m[0], src[i]);
    return Op::apply(Op::apply3(m[0], m[1], m[2]), m[3]);
}

template <int N>
__device__ __forceinline__ float thread_max(const float (&src)[N],
                                            float old = 0.0f, bool accum = false)
{
    return thread_extreme<OpMax, N>(src, old, accum);
}

template <int N>
__device__ __forceinline__ float thread_min(const float (&src)[N],
                                            float old = 0.0f, bool accum = false)
{
    return thread_extreme<OpMin, N>(src, old, accum);
}

// ---------------------------------------------------------------------------
// Wave scope.
//
// GFX9 DPP controls used: row_shr:k (0x110 + k) reads lane i-k of the same
// 16-lane row; row_bcast:15 (0x142) feeds lane 15 of each row to the next
// row; row_bcast:31 (0x143) feeds lane 31 to rows 2 and 3.  A lane whose
// source is outside the row, or whose row is masked off, receives `old`,
// which is set to the operator's identity (bound_ctrl off).
//
// After the four row shifts, lane 15 of each row holds that row's total;
// the two broadcasts fold row 0 into row 1, row 2 into row 3, then rows
// 0..1 into rows 2..3, leaving the wave total in lane 63, which readlane
// hands to every lane.
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

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<OpSum>(v); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce<OpMax>(v); }
__device__ __forceinline__ float wave_min(float v) { return wave_reduce<OpMin>(v); }

// ---------------------------------------------------------------------------
// Workgroup scope: every wave reduces with DPP, lane 0 of wave w writes
// lds[w], and after the barrier every thread folds lds[0..WAVES) in wave
// order.
// ---------------------------------------------------------------------------
template <class Op, int WAVES>
__device__ __forceinline__ float block_reduce(float v, float* lds)
{
    static_assert(WAVES >= 1 && WAVES <= 16, "1 to 16 wave64s per workgroup");
    const float w = wave_reduce<Op>(v);
    if ((threadIdx.x & 63) == 0)
        lds[threadIdx.x / 64] = w;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int k = 1; k < WAVES; ++k)
        r = Op::apply(r, lds[k]);
    return r;
}

template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float* lds)
{
    return block_reduce<OpSum, WAVES>(v, lds);
}
template <int WAVES>
__device__ __forceinline__ float block_max(float v, float* lds)
{
    return block_reduce<OpMax, WAVES>(v, lds);
}
template <int WAVES>
__device__ __forceinline__ float block_min(float v, float* lds)
{
    return block_reduce<OpMin, WAVES>(v, lds);
}

} // namespace red_dev
