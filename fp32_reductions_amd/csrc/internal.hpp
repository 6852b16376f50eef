// internal.hpp -- host-side interface between the C ABI (api.hip) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace red {

enum class OpKind { Sum, Max, Min };

// Per-(device, stream) scratch owned by the library: the partial results
// the first pass of a reduction hands to its second pass.  Calls on one
// stream are ordered, so they can share it.
struct Workspace {
    void* partials = nullptr;
    size_t partial_bytes = 0;
};

// Launch geometry chosen by the host from the device.
struct DeviceInfo {
    int cus = 0;                   // compute units
};

// Workgroups per compute unit that the split-row kernel aims at, and that
// the column product plans for (measured on MI355X: fewer, longer-lived
// workgroups stream HBM faster than a full-occupancy grid).  The 1-D
// kernels take their launch shape from stream_shape (device.hpp).
#ifndef RED_STREAM_WG_PER_CU
#define RED_STREAM_WG_PER_CU 2
#endif
#ifndef RED_COLPROD_WG_PER_CU
#define RED_COLPROD_WG_PER_CU 1
#endif
constexpr int kStreamWgPerCu = RED_STREAM_WG_PER_CU;
constexpr int kColprodWgPerCu = RED_COLPROD_WG_PER_CU;
// Row count from which the row kernels use one wave per row whatever n is.
constexpr int kRowsWavePerCu = 8;

// ---- 1-D vector -> scalar (reduce1d.hip) ----------------------------------
// Deterministic form: per-workgroup partials, then a one-workgroup finish.
hipError_t launch_reduce1d(OpKind op, const float* x, size_t n, float* out,
                           int accum, const DeviceInfo& dev,
                           const Workspace& ws, hipStream_t stream);
// Fused: out[0..3) = sum, max, min of x from one read of x.
hipError_t launch_reduce1d_summaxmin(const float* x, size_t n, float* out,
                                     int accum, const DeviceInfo& dev,
                                     const Workspace& ws, hipStream_t stream);
// Single-pass form: one device-scope atomic per workgroup.
hipError_t launch_reduce1d_atomic(OpKind op, const float* x, size_t n,
                                  float* out, int accum, const DeviceInfo& dev,
                                  hipStream_t stream);
// Number of workgroups launch_reduce1d uses for n elements at address x.
unsigned reduce1d_grid(const float* x, size_t n, const DeviceInfo& dev);
// Set `count` 32-bit words to `value` on `stream` with a kernel.
hipError_t launch_fill_u32(unsigned* p, size_t count, unsigned value,
                           hipStream_t stream);

// ---- segmented rows (rows.hip) --------------------------------------------
// Chunks per row of the split row kernel for this problem: 0 when another
// row kernel runs, 1 when it needs no partials, K > 1 when it writes
// rows * K partials to the workspace.
uint32_t rows_chunks(const float* x, size_t rows, size_t n, const DeviceInfo& dev);
hipError_t launch_rows(OpKind op, const float* x, size_t rows, size_t n,
                       size_t ld, float* out, int accum, const DeviceInfo& dev,
                       const Workspace& ws, hipStream_t stream);

// ---- column product (colprod.hip) -----------------------------------------
// U16 carries int16 and uint16 (same bits); uint32 runs as I32 (same bits).
enum class ColType { F32, F16, BF16, I32, U16 };
size_t colprod_elem_size(ColType t);
// Row splits the colprod kernel uses, and the workspace it needs.
struct ColprodPlan {
    unsigned col_blocks = 0;  // 256-byte column blocks
    unsigned group_rows = 16; // row groups per column block (1, 4 or 16)
    unsigned splits = 1;      // workgroups along the rows (S)
    size_t partial_bytes = 0; // S * C * 4 when S > 1
    unsigned narrow_w = 0;    // units per row when the narrow-row kernel runs, else 0
    bool narrow_vec = false;  // its unit: a 16-byte vector (true) or one element
    unsigned wide_vpl = 0;    // vectors per lane of the wide-strip kernel, 0 when it does not run
    unsigned full_strips = 0; // its workgroups that own whole strips
    unsigned wide_grid = 0;   // its grid (full strips, then the remaining blocks)
    unsigned finish_blocks = 0;     // second-pass workgroups (S > 1)
    unsigned finish_cols_log2 = 0;  // log2 of the columns per second-pass workgroup
};
ColprodPlan colprod_plan(ColType t, const void* src, size_t R, size_t C, size_t ld,
                         const DeviceInfo& dev, const Workspace& ws);
hipError_t launch_colprod(ColType t, const void* src, size_t R, size_t C,
                          size_t ld, void* dst, const ColprodPlan& plan,
                          const Workspace& ws, hipStream_t stream);
// Column sum / max / min of an fp32 tile (plan from colprod_plan(F32, ...)).
hipError_t launch_cols(OpKind op, const float* src, size_t R, size_t C,
                       size_t ld, float* dst, int accum, const ColprodPlan& plan,
                       const Workspace& ws, hipStream_t stream);

} // namespace red
