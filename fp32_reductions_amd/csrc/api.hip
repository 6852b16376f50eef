// api.hip -- the extern "C" entry points declared in include/reduce.h.
//
// Every entry point validates its arguments before touching the HIP
// runtime, returns early (RED_OK, nothing enqueued) for empty input, looks
// up the device's compute-unit count and, where the kernel needs one, the
// calling stream's workspace, then enqueues the kernel and returns.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <memory>
#include <mutex>
#include <tuple>

#include "internal.hpp"
#include "reduce.h"

namespace {

using red::ColType;
using red::DeviceInfo;
using red::OpKind;
using red::Workspace;

// Fixed workspace per (device, stream) for partial results.  The kernels
// size their grids so that they never need more than this.
constexpr size_t kPartialBytes = size_t(16) << 20;

// One workspace and the lock a call holds while it enqueues the kernels
// that use it: the first pass writes the partials and the second reads
// them, so two calls on one stream from different host threads must not
// interleave their launches.  `released` is set (under `mu`) when
// red_release_workspace has taken the slot out of the map.
struct Slot {
    Workspace ws;
    std::mutex mu;
    bool released = false;
};

// A workspace belongs to a (device, stream).  hipStreamPerThread is one
// handle for a different stream in every host thread, so for it the key is
// the calling thread instead.
enum KeyKind { kStreamKey = 0, kThreadKey = 1 };
using SlotKey = std::tuple<int, int, uintptr_t>;

// Devices whose compute-unit count is cached (a fixed table, so that a
// lookup never allocates host memory); devices past it are queried on
// every call.
constexpr int kMaxDevices = 64;

std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices]; // cus == 0: not looked up yet
std::map<SlotKey, std::shared_ptr<Slot>> g_ws;
std::atomic<uint64_t> g_next_thread{1};

// A number for the calling host thread, never reused within the process.
uint64_t thread_token()
{
    thread_local uint64_t token = g_next_thread.fetch_add(1);
    return token;
}

SlotKey slot_key(int dev, hipStream_t stream)
{
    if (stream == hipStreamPerThread)
        return SlotKey(dev, kThreadKey, (uintptr_t)thread_token());
    return SlotKey(dev, kStreamKey, (uintptr_t)stream);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// (count - 1) * stride + width elements of `elem` bytes fit in size_t.
bool extent_ok(size_t count, size_t stride, size_t width, size_t elem)
{
    size_t span;
    if (__builtin_mul_overflow(count - 1, stride, &span))
        return false;
    if (__builtin_add_overflow(span, width, &span))
        return false;
    return !__builtin_mul_overflow(span, elem, &span);
}

int device_info(int dev, DeviceInfo* info)
{
    const bool cached = dev < kMaxDevices;
    if (cached) {
        std::lock_guard<std::mutex> lock(g_mu);
        if (g_dev[dev].cus > 0) {
            *info = g_dev[dev];
            return RED_OK;
        }
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess || cus <= 0)
        return RED_ERR_HIP;
    info->cus = cus;
    if (cached) {
        std::lock_guard<std::mutex> lock(g_mu);
        g_dev[dev] = *info;
    }
    return RED_OK;
}

// The current device and the figures the launch plans use.  Test hook:
// RED_TEST_CUS (a count from 1 to 65536), when set, replaces the compute-
// unit count in every plan, so that tests run the planning of other device
// sizes (a partitioned GPU, a smaller or larger part) on this one.
int current_device(int* dev, DeviceInfo* info)
{
    if (hipGetDevice(dev) != hipSuccess || *dev < 0)
        return RED_ERR_HIP;
    const int st = device_info(*dev, info);
    if (st != RED_OK)
        return st;
    const char* t = std::getenv("RED_TEST_CUS");
    if (t && *t) {
        const long v = std::strtol(t, nullptr, 10);
        if (v >= 1 && v <= 65536)
            info->cus = (int)v;
    }
    return RED_OK;
}

// The slot of (dev, stream), created on first use.
int find_slot(int dev, hipStream_t stream, std::shared_ptr<Slot>* out)
{
    std::lock_guard<std::mutex> lock(g_mu);
    const SlotKey key = slot_key(dev, stream);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
        *out = it->second;
        return RED_OK;
    }
    // Failure injection for tests of the RED_ERR_NOMEM path.
    const char* fail = std::getenv("RED_TEST_FAIL_ALLOC");
    if (fail && fail[0] == '1')
        return RED_ERR_NOMEM;
    void* base = nullptr;
    if (hipMalloc(&base, kPartialBytes) != hipSuccess) {
        (void)hipGetLastError(); // clear the sticky allocation error
        return RED_ERR_NOMEM;
    }
    auto slot = std::make_shared<Slot>();
    slot->ws.partials = base;
    slot->ws.partial_bytes = kPartialBytes;
    g_ws.emplace(key, slot);
    *out = slot;
    return RED_OK;
}

// The workspace of (dev, stream), held for the caller until it goes out of
// scope: `lock` keeps other host threads from enqueueing on the same
// workspace in between this call's launches.
struct HeldWorkspace {
    std::shared_ptr<Slot> slot;
    std::unique_lock<std::mutex> lock;
};

int stream_workspace(int dev, hipStream_t stream, Workspace* ws, HeldWorkspace* held)
{
    for (;;) {
        std::shared_ptr<Slot> slot;
        const int st = find_slot(dev, stream, &slot);
        if (st != RED_OK)
            return st;
        std::unique_lock<std::mutex> lock(slot->mu);
        if (slot->released)
            continue; // released after the lookup: look again
        *ws = slot->ws;
        held->slot = std::move(slot);
        held->lock = std::move(lock);
        return RED_OK;
    }
}

int hip_status(hipError_t e) { return e == hipSuccess ? RED_OK : RED_ERR_HIP; }

// ---- static scratch of the allocation-free fused call ---------------------
//
// red_sum_max_min_f32_noalloc keeps its per-workgroup partials (3 floats
// per workgroup of the first pass) in this file-scope device array instead
// of a hipMalloc'd workspace.  Each GPU the library runs on holds its own
// copy until the process ends, and every call on that GPU shares it.  In
// host code `scratch` only names the symbol: its device address on a
// device comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the first call there and kept in g_scratch.
constexpr size_t kScratchBytes = 16384;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices]; // device address of each device's `scratch`

// The device address of `scratch` on the current device `dev`.
int scratch_address(int dev, float** out)
{
    if (dev >= kMaxDevices)
        return RED_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return RED_ERR_HIP;
        }
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return RED_OK;
}

// Bytes of scratch a call may use: kScratchBytes, or less when the test
// hook RED_TEST_SCRATCH_LIMIT (bytes) asks for less, so that tests can
// reach the rejection path on a device whose grids always fit.
size_t scratch_limit()
{
    const char* s = std::getenv("RED_TEST_SCRATCH_LIMIT");
    if (s && *s) {
        const unsigned long long v = std::strtoull(s, nullptr, 10);
        if (v < kScratchBytes)
            return (size_t)v;
    }
    return kScratchBytes;
}

// Called right before a call's launches: drops an error an earlier,
// unrelated HIP call left on this thread, so that the status returned after
// the launches (hipGetLastError) reports this call's own launches.  A
// sticky error (a fault of an earlier kernel) is reported again by the
// launches themselves.
void clear_stale_error() { (void)hipGetLastError(); }

int check_1d(const float* x, size_t n, const float* out)
{
    if (!x || !out)
        return RED_ERR_INVALID;
    if (n > SIZE_MAX / sizeof(float))
        return RED_ERR_INVALID;
    if (!aligned(x, sizeof(float)) || !aligned(out, sizeof(float)))
        return RED_ERR_ALIGN;
    return RED_OK;
}

int reduce1d(OpKind op, const float* x, size_t n, float* out, int accum,
             red_stream_t stream)
{
    if (n == 0)
        return RED_OK;
    int st = check_1d(x, n, out);
    if (st != RED_OK)
        return st;
    int dev;
    DeviceInfo info;
    if ((st = current_device(&dev, &info)) != RED_OK)
        return st;
    Workspace ws;
    HeldWorkspace held;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = stream_workspace(dev, s, &ws, &held)) != RED_OK)
        return st;
    clear_stale_error();
    return hip_status(red::launch_reduce1d(op, x, n, out, accum, info, ws, s));
}

int reduce1d_summaxmin(const float* x, size_t n, float* out, int accum,
                       red_stream_t stream)
{
    if (n == 0)
        return RED_OK;
    int st = check_1d(x, n, out);
    if (st != RED_OK)
        return st;
    int dev;
    DeviceInfo info;
    if ((st = current_device(&dev, &info)) != RED_OK)
        return st;
    Workspace ws;
    HeldWorkspace held;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = stream_workspace(dev, s, &ws, &held)) != RED_OK)
        return st;
    clear_stale_error();
    return hip_status(red::launch_reduce1d_summaxmin(x, n, out, accum, info, ws, s));
}

int reduce1d_summaxmin_noalloc(const float* x, size_t n, float* out, int accum,
                               red_stream_t stream)
{
    if (n == 0)
        return RED_OK;
    int st = check_1d(x, n, out);
    if (st != RED_OK)
        return st;
    int dev;
    DeviceInfo info;
    if ((st = current_device(&dev, &info)) != RED_OK)
        return st;
    Workspace ws;
    ws.partial_bytes = scratch_limit();
    if ((size_t)red::reduce1d_grid(x, n, info) * 3 * sizeof(float) > ws.partial_bytes)
        return RED_ERR_SCRATCH;
    float* p;
    if ((st = scratch_address(dev, &p)) != RED_OK)
        return st;
    ws.partials = p;
    clear_stale_error();
    return hip_status(red::launch_reduce1d_summaxmin(x, n, out, accum, info, ws,
                                                     static_cast<hipStream_t>(stream)));
}

int reduce1d_atomic(OpKind op, const float* x, size_t n, float* out, int accum,
                    red_stream_t stream)
{
    if (n == 0)
        return RED_OK;
    int st = check_1d(x, n, out);
    if (st != RED_OK)
        return st;
    int dev;
    DeviceInfo info;
    if ((st = current_device(&dev, &info)) != RED_OK)
        return st;
    clear_stale_error();
    return hip_status(red::launch_reduce1d_atomic(
        op, x, n, out, accum, info, static_cast<hipStream_t>(stream)));
}

int reduce_rows(OpKind op, const float* x, size_t rows, size_t n, size_t ld,
                float* out, int accum, red_stream_t stream)
{
    if (rows == 0 || n == 0)
        return RED_OK;
    if (!x || !out || ld < n || !extent_ok(rows, ld, n, sizeof(float)) ||
        rows > SIZE_MAX / sizeof(float))
        return RED_ERR_INVALID;
    if (!aligned(x, sizeof(float)) || !aligned(out, sizeof(float)))
        return RED_ERR_ALIGN;
    int dev;
    DeviceInfo info;
    int st = current_device(&dev, &info);
    if (st != RED_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Workspace ws;
    HeldWorkspace held;
    if (red::rows_chunks(x, rows, n, info) > 1 &&
        (st = stream_workspace(dev, s, &ws, &held)) != RED_OK)
        return st;
    clear_stale_error();
    return hip_status(red::launch_rows(op, x, rows, n, ld, out, accum, info, ws, s));
}

// Column reductions share validation: ld >= C, extents, grid limit,
// alignment to the element size.
int check_cols(ColType t, const void* src, size_t R, size_t C, size_t ld,
               const void* dst)
{
    const size_t es = red::colprod_elem_size(t);
    if (!src || !dst || ld < C || !extent_ok(R, ld, C, es) ||
        C > SIZE_MAX / sizeof(float))
        return RED_ERR_INVALID;
    // A launch holds at most 2^32 - 1 work-items per grid dimension.  Each
    // column workgroup covers at least one block of 16 lanes x (16 / es)
    // columns on 256 threads; the 512-thread layout runs only when the
    // blocks are too few to give every compute unit a workgroup of 4 row
    // groups (fewer than 4 per CU).  So fewer than 2^24 blocks keep every
    // grid under the limit.
    const size_t cols_per_wg = 16 * (16 / es);
    if ((C + cols_per_wg - 1) / cols_per_wg >= (size_t(1) << 24))
        return RED_ERR_INVALID;
    if (!aligned(src, es) || !aligned(dst, es))
        return RED_ERR_ALIGN;
    return RED_OK;
}

int cols(OpKind op, const float* src, size_t R, size_t C, size_t ld, float* dst,
         int accum, red_stream_t stream)
{
    if (R == 0 || C == 0)
        return RED_OK;
    int st = check_cols(ColType::F32, src, R, C, ld, dst);
    if (st != RED_OK)
        return st;
    int dev;
    DeviceInfo info;
    if ((st = current_device(&dev, &info)) != RED_OK)
        return st;
    Workspace ws;
    HeldWorkspace held;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = stream_workspace(dev, s, &ws, &held)) != RED_OK)
        return st;
    const red::ColprodPlan plan = red::colprod_plan(ColType::F32, src, R, C, ld, info, ws);
    clear_stale_error();
    return hip_status(red::launch_cols(op, src, R, C, ld, dst, accum, plan, ws, s));
}

int colprod(ColType t, const void* src, size_t R, size_t C, size_t ld,
            void* dst, red_stream_t stream)
{
    if (R == 0 || C == 0)
        return RED_OK;
    int st = check_cols(t, src, R, C, ld, dst);
    if (st != RED_OK)
        return st;
    int dev;
    DeviceInfo info;
    if ((st = current_device(&dev, &info)) != RED_OK)
        return st;
    Workspace ws;
    HeldWorkspace held;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = stream_workspace(dev, s, &ws, &held)) != RED_OK)
        return st;
    const red::ColprodPlan plan = red::colprod_plan(t, src, R, C, ld, info, ws);
    clear_stale_error();
    return hip_status(red::launch_colprod(t, src, R, C, ld, dst, plan, ws, s));
}

} // namespace

extern "C" {

int red_sum_f32(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d(OpKind::Sum, x, n, out, accum, stream);
}
int red_max_f32(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d(OpKind::Max, x, n, out, accum, stream);
}
int red_min_f32(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d(OpKind::Min, x, n, out, accum, stream);
}

int red_sum_max_min_f32(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d_summaxmin(x, n, out, accum, stream);
}

int red_sum_max_min_f32_noalloc(const float* x, size_t n, float* out, int accum,
                                red_stream_t stream)
{
    return reduce1d_summaxmin_noalloc(x, n, out, accum, stream);
}

int red_sum_f32_atomic(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d_atomic(OpKind::Sum, x, n, out, accum, stream);
}
int red_max_f32_atomic(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d_atomic(OpKind::Max, x, n, out, accum, stream);
}
int red_min_f32_atomic(const float* x, size_t n, float* out, int accum, red_stream_t stream)
{
    return reduce1d_atomic(OpKind::Min, x, n, out, accum, stream);
}

int red_sum_rows_f32(const float* x, size_t rows, size_t n, size_t ld, float* out,
                     int accum, red_stream_t stream)
{
    return reduce_rows(OpKind::Sum, x, rows, n, ld, out, accum, stream);
}
int red_max_rows_f32(const float* x, size_t rows, size_t n, size_t ld, float* out,
                     int accum, red_stream_t stream)
{
    return reduce_rows(OpKind::Max, x, rows, n, ld, out, accum, stream);
}
int red_min_rows_f32(const float* x, size_t rows, size_t n, size_t ld, float* out,
                     int accum, red_stream_t stream)
{
    return reduce_rows(OpKind::Min, x, rows, n, ld, out, accum, stream);
}

int red_sum_cols_f32(const float* src, size_t R, size_t C, size_t ld, float* dst,
                     int accum, red_stream_t stream)
{
    return cols(OpKind::Sum, src, R, C, ld, dst, accum, stream);
}
int red_max_cols_f32(const float* src, size_t R, size_t C, size_t ld, float* dst,
                     int accum, red_stream_t stream)
{
    return cols(OpKind::Max, src, R, C, ld, dst, accum, stream);
}
int red_min_cols_f32(const float* src, size_t R, size_t C, size_t ld, float* dst,
                     int accum, red_stream_t stream)
{
    return cols(OpKind::Min, src, R, C, ld, dst, accum, stream);
}

int red_colprod_f32(const float* src, size_t R, size_t C, size_t ld, float* dst,
                    red_stream_t stream)
{
    return colprod(ColType::F32, src, R, C, ld, dst, stream);
}
int red_colprod_f16(const uint16_t* src, size_t R, size_t C, size_t ld, uint16_t* dst,
                    red_stream_t stream)
{
    return colprod(ColType::F16, src, R, C, ld, dst, stream);
}
int red_colprod_bf16(const uint16_t* src, size_t R, size_t C, size_t ld, uint16_t* dst,
                     red_stream_t stream)
{
    return colprod(ColType::BF16, src, R, C, ld, dst, stream);
}
int red_colprod_i32(const int32_t* src, size_t R, size_t C, size_t ld, int32_t* dst,
                    red_stream_t stream)
{
    return colprod(ColType::I32, src, R, C, ld, dst, stream);
}

int red_colprod_i16(const int16_t* src, size_t R, size_t C, size_t ld, int16_t* dst,
                    red_stream_t stream)
{
    return colprod(ColType::U16, src, R, C, ld, dst, stream);
}
int red_colprod_u16(const uint16_t* src, size_t R, size_t C, size_t ld, uint16_t* dst,
                    red_stream_t stream)
{
    return colprod(ColType::U16, src, R, C, ld, dst, stream);
}
int red_colprod_u32(const uint32_t* src, size_t R, size_t C, size_t ld, uint32_t* dst,
                    red_stream_t stream)
{
    return colprod(ColType::I32, src, R, C, ld, dst, stream);
}

int red_release_workspace(red_stream_t stream)
{
    int dev;
    if (hipGetDevice(&dev) != hipSuccess)
        return RED_ERR_HIP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::shared_ptr<Slot> slot;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_ws.find(slot_key(dev, s));
        if (it == g_ws.end())
            return RED_OK;
        slot = it->second;
        g_ws.erase(it);
    }
    {
        // Waits for a call that is enqueueing on this workspace; a call
        // that looked the slot up before the erase finds it released and
        // takes a new one.
        std::lock_guard<std::mutex> lock(slot->mu);
        slot->released = true;
    }
    // Work already enqueued on the stream may still read the partials.
    const hipError_t e = hipStreamSynchronize(s);
    const hipError_t f = hipFree(slot->ws.partials);
    return (e == hipSuccess && f == hipSuccess) ? RED_OK : RED_ERR_HIP;
}

const char* red_status_str(int status)
{
    switch (status) {
    case RED_OK: return "ok";
    case RED_ERR_INVALID: return "invalid argument";
    case RED_ERR_ALIGN: return "pointer not aligned to its element size";
    case RED_ERR_NOMEM: return "workspace allocation failed";
    case RED_ERR_HIP: return "HIP runtime error";
    case RED_ERR_SCRATCH: return "the call needs more scratch than the static buffer holds";
    default: return "unknown status";
    }
}

int red_abi_version(void) { return RED_ABI_VERSION; }

} // extern "C"
