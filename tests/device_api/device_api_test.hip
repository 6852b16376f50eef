// device_api_test.hip -- test kernels for include/reduce_device.hpp.
// Test support only: each kernel calls one device-side reduction and stores
// its result so the tests can compare it with the CPU oracle.
#include <hip/hip_runtime.h>

#include "reduce_device.hpp"

namespace {

// One thread per row of an N-column row-major matrix: thread scope.
template <int N>
__global__ void thread_kernel(const float* __restrict__ x, int rows,
                              float* __restrict__ out, int op, int accum,
                              const float* __restrict__ old)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows)
        return;
    float v[N];
#pragma unroll
    for (int k = 0; k < N; ++k)
        v[k] = x[(size_t)r * N + k];
    const float o = accum ? old[r] : 0.0f;
    float res;
    if (op == 0)
        res = red_dev::thread_sum<N>(v, o, accum != 0);
    else if (op == 1)
        res = red_dev::thread_max<N>(v, o, accum != 0);
    else
        res = red_dev::thread_min<N>(v, o, accum != 0);
    out[r] = res;
}

template <int N>
hipError_t launch_thread(const float* x, int rows, float* out, int op, int accum,
                         const float* old)
{
    thread_kernel<N><<<(rows + 255) / 256, 256>>>(x, rows, out, op, accum, old);
    return hipGetLastError();
}

// One wave per workgroup: every lane stores the wave's result.
__global__ void wave_kernel(const float* __restrict__ x, float* __restrict__ out, int op)
{
    const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
    const float v = x[i];
    out[i] = op == 0 ? red_dev::wave_sum(v) : op == 1 ? red_dev::wave_max(v)
                                                     : red_dev::wave_min(v);
}

// WAVES wave64s per workgroup: every thread stores the workgroup's result.
template <int WAVES>
__global__ void block_kernel(const float* __restrict__ x, float* __restrict__ out, int op)
{
    __shared__ float lds[WAVES];
    const size_t i = (size_t)blockIdx.x * (64 * WAVES) + threadIdx.x;
    const float v = x[i];
    float r;
    if (op == 0)
        r = red_dev::block_sum<WAVES>(v, lds);
    else if (op == 1)
        r = red_dev::block_max<WAVES>(v, lds);
    else
        r = red_dev::block_min<WAVES>(v, lds);
    out[i] = r;
}

} // namespace

extern "C" {

// x: rows * n floats; out: rows floats; op 0 sum, 1 max, 2 min.
// Returns a hipError_t value (0 on success); n must be one of the sizes below.
int devtest_thread(const float* x, int n, int rows, float* out, int op, int accum,
                   const float* old)
{
    switch (n) {
    case 1: return launch_thread<1>(x, rows, out, op, accum, old);
    case 3: return launch_thread<3>(x, rows, out, op, accum, old);
    case 5: return launch_thread<5>(x, rows, out, op, accum, old);
    case 8: return launch_thread<8>(x, rows, out, op, accum, old);
    case 9: return launch_thread<9>(x, rows, out, op, accum, old);
    case 16: return launch_thread<16>(x, rows, out, op, accum, old);
    case 17: return launch_thread<17>(x, rows, out, op, accum, old);
    case 32: return launch_thread<32>(x, rows, out, op, accum, old);
    case 33: return launch_thread<33>(x, rows, out, op, accum, old);
    case 64: return launch_thread<64>(x, rows, out, op, accum, old);
    default: return (int)hipErrorInvalidValue;
    }
}

// x and out: nwaves * 64 floats.
int devtest_wave(const float* x, int nwaves, float* out, int op)
{
    wave_kernel<<<nwaves, 64>>>(x, out, op);
    return (int)hipGetLastError();
}

// x and out: nblocks * 64 * waves floats; waves one of 1, 4, 16.
int devtest_block(const float* x, int nblocks, int waves, float* out, int op)
{
    switch (waves) {
    case 1: block_kernel<1><<<nblocks, 64>>>(x, out, op); break;
    case 4: block_kernel<4><<<nblocks, 256>>>(x, out, op); break;
    case 16: block_kernel<16><<<nblocks, 1024>>>(x, out, op); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

} // extern "C"
