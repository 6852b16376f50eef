// internal.hpp -- host-side interface between the C ABI (api.hip) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace red {

enum class OpKind { Sum, Max, Min };

// Per-(device, stream) scratch owned by the library.  Tickets must be zero
// whenever no kernel of this library is running on the stream: every kernel
// that takes a ticket puts it back to zero before it exits.
struct Workspace {
    void* partials = nullptr;      // per-workgroup partial results
    size_t partial_bytes = 0;
    unsigned* tickets = nullptr;   // arrival counters
    size_t n_tickets = 0;
};

// Launch geometry chosen by the host from the device.
struct DeviceInfo {
    int cus = 0;                   // compute units
};

// Workgroups launched per compute unit for the streaming kernels.
constexpr int kWgPerCu = 8;

// ---- 1-D vector -> scalar (reduce1d.hip) ----------------------------------
// Deterministic form: partials + last-arriving-workgroup finish.
hipError_t launch_reduce1d(OpKind op, const float* x, size_t n, float* out,
                           int accum, const DeviceInfo& dev,
                           const Workspace& ws, hipStream_t stream);
// Single-pass form: one device-scope atomic per workgroup.
hipError_t launch_reduce1d_atomic(OpKind op, const float* x, size_t n,
                                  float* out, int accum, const DeviceInfo& dev,
                                  hipStream_t stream);
// Number of workgroups launch_reduce1d uses for n elements at address x.
unsigned reduce1d_grid(const float* x, size_t n, const DeviceInfo& dev);
// Zero `count` 32-bit words on `stream` with a kernel (no memset node).
hipError_t launch_fill_u32(unsigned* p, size_t count, unsigned value,
                           hipStream_t stream);

// ---- segmented rows (rows.hip) --------------------------------------------
hipError_t launch_rows(OpKind op, const float* x, size_t rows, size_t n,
                       size_t ld, float* out, int accum, const DeviceInfo& dev,
                       hipStream_t stream);

// ---- column product (colprod.hip) -----------------------------------------
enum class ColType { F32, F16, BF16, I32 };
size_t colprod_elem_size(ColType t);
// Row splits the colprod kernel uses, and the workspace it needs.
struct ColprodPlan {
    unsigned col_blocks = 0;  // workgroups across the columns
    unsigned splits = 1;      // workgroups along the rows (S)
    size_t rows_per_split = 0;
    size_t partial_bytes = 0; // S * C * 4 when S > 1
};
ColprodPlan colprod_plan(ColType t, size_t R, size_t C, const DeviceInfo& dev,
                         const Workspace& ws);
hipError_t launch_colprod(ColType t, const void* src, size_t R, size_t C,
                          size_t ld, void* dst, const ColprodPlan& plan,
                          const Workspace& ws, hipStream_t stream);

} // namespace red
