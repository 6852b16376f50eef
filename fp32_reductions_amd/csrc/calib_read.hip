// calib_read.hip -- measurement only: the read-only streaming ceiling that
// the benchmark reports beside the reductions.  Not part of the C ABI in
// include/reduce.h and not used by any entry point; it builds into its own
// library (libreduce_calib.so).
//
// The kernel is the 1-D stream kernel with the reduction replaced by a
// trivial sink: the same launch shape (stream_shape) and the same sweeps of
// eight non-temporal 16-byte loads per thread (stream_chunk or
// stream_regions), but each element's bits are XORed into one word per
// thread instead of being added, and a thread stores its word only when it
// equals a value the caller passes (so the loads cannot be removed, and in
// practice nothing is stored).  Its time for a vector is therefore what
// reading the vector costs on this device with that launch, launch
// included.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace red {
namespace {

struct AccXor {
    uint32_t w = 0;
    __device__ __forceinline__ void fold1(const float4& a)
    {
        w ^= __float_as_uint(a.x) ^ __float_as_uint(a.y) ^ __float_as_uint(a.z) ^
             __float_as_uint(a.w);
    }
    __device__ __forceinline__ void fold2(const float4& a, const float4& b)
    {
        fold1(a);
        fold1(b);
    }
    __device__ __forceinline__ void fold_scalar(float v) { w ^= __float_as_uint(v); }
};

template <bool REGIONAL>
__global__ __launch_bounds__(REGIONAL ? kBlock : kWideBlock) void read_sink_kernel(const float* __restrict__ x,
                                                           uint64_t n,
                                                           uint32_t* __restrict__ sink,
                                                           uint32_t match)
{
    AccXor acc;
    if constexpr (REGIONAL)
        stream_regions(x, n, acc);
    else
        stream_chunk<kWideBlock, kWideUnroll>(x, n, blockIdx.x, gridDim.x, acc);
    if (acc.w == match)
        sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.w;
}

} // namespace
} // namespace red

// The stream kernel's grid for x[0, n).
extern "C" int calib_read_grid(const float* x, size_t n, int cus)
{
    return (int)red::stream_shape(x, n, cus).grid;
}

// Streams x[0, n) once on `stream`.  sink must hold grid * 512 words, grid
// as returned by calib_read_grid.  Returns a hipError_t value.

extern "C" int calib_read_f32(const float* x, size_t n, unsigned* sink,
                              unsigned match, int cus, void* stream)
{
    if (n == 0)
        return 0;
    const red::StreamShape sh = red::stream_shape(x, n, cus);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (sh.regional)
        red::read_sink_kernel<true><<<sh.grid, red::kBlock, 0, s>>>(x, n, sink, match);
    else
        red::read_sink_kernel<false><<<sh.grid, red::kWideBlock, 0, s>>>(x, n, sink, match);
    return (int)hipGetLastError();
}
