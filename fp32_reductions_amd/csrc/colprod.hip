// colprod.hip -- column product of a row-major tile (TCOLPROD), and the
// column sum / max / min built on the same layout.
//
// PTO ISA "TCOLPROD", "Math Interpretation": dst[0,j] is the product of
// src[i,j] over the R valid rows, for each of the C valid columns;
// "Constraints": row-major source, destination of the same element type
// (half, float, bfloat16, int16, uint16, int32, uint32 among the listed
// ones).
//
// Layout of the work:
//  * each lane owns V consecutive columns, V = 16 bytes / sizeof(T) (4 for
//    f32 / i32, 8 for f16 / bf16), so one 16-byte load per row feeds all of
//    them; 16 lanes cover 256 contiguous bytes of a row and a wave reads
//    four rows per load;
//  * a workgroup covers one block of 16*V columns and its share of the
//    rows: 512 threads (32 row groups of 16 lanes, 4 rows in flight per
//    lane) when the rows are not split or not 16-byte aligned, else 256
//    threads (16 row groups, 8 rows in flight); its row groups take
//    interleaved rows and combine their partial products in LDS in
//    row-group order.  Short, wide tiles, whose blocks alone would give
//    thousands of short-lived workgroups, put 4 or 16 adjacent blocks in a
//    workgroup instead, with 4 or 1 row groups each; with more blocks
//    still, a wide-strip kernel gives each lane 2 to 8 vectors of a row and
//    fewer rows in flight;
//  * when the grid needs more workgroups than there are column blocks, S
//    workgroups (blockIdx.y) share each block's rows in interleaved chunks
//    of 128 rows (grid-stride along the rows); each stores its partial row
//    in the workspace, and a second kernel combines the S partial rows of
//    each column in a fixed order (strided runs per thread, then a pairwise
//    tree in LDS), narrows once to T and writes dst;
//  * rows narrower than 256 bytes would leave most of those lanes idle: a
//    narrow-row kernel reads whole rows instead, 256 / W rows of W units
//    per step (16-byte vectors when the tile is aligned and C * sizeof(T) is
//    a multiple of 16, else elements), each workgroup walking sweeps of
//    several steps grid-stride;
//  * tile loads are non-temporal: each element is read once.
//
// Column sum / max / min of an fp32 tile reduce each column by the TVM
// page's operators ("reduction -> sm100_packed"), the 2-D case its fast
// path leaves to a generic fallback ("How inputs change the algorithm"),
// with the same identities and maxNum / minNum rules as the 1-D calls.
//
// Arithmetic: f32, f16 and bf16 multiply in fp32 (16-bit values widen
// exactly); i32 / u32 and i16 / u16 in uint32 (wrapping modulo 2^32; the
// 16-bit types keep the low 16 bits of the final product).  f16 / bf16
// round once, to nearest even, when the final product is stored.
#include "device.hpp"
#include "internal.hpp"

namespace red {
namespace {

#ifndef RED_COLPROD_UNROLL
#define RED_COLPROD_UNROLL 8
#endif
constexpr int kRowsInFlight = RED_COLPROD_UNROLL; // 16-byte loads in flight per lane
constexpr int kLanesPerRow = 16;                  // lanes sharing one row of a column block
// Narrow rows read in elements: bytes each lane keeps in flight (16 loads
// of 4-byte elements, 32 of 2-byte ones).  Measured on MI355X with
// 256 MiB fp32 tiles of 1 to 63 columns: 16 loads per lane at 2 workgroups
// per CU (32 KiB in flight per CU) streamed at 5.8-6.1 TB/s; 8 loads gave
// 4.5-4.8 TB/s, and 64 KiB per CU (32 loads, or 8 workgroups per CU) less.
#ifndef RED_COLPROD_ELEM_BYTES_IN_FLIGHT
#define RED_COLPROD_ELEM_BYTES_IN_FLIGHT 64
#endif
template <class T>
constexpr int kElemRowsInFlight = RED_COLPROD_ELEM_BYTES_IN_FLIGHT / (int)sizeof(T);

struct TraitsF32 {
    using T = float;
    using A = float;
    static constexpr int V = 4;
    static __device__ __forceinline__ A one() { return 1.0f; }
    static __device__ __forceinline__ A widen(T v) { return v; }
    static __device__ __forceinline__ T narrow(A a) { return a; }
    static __device__ __forceinline__ void unpack(const uint4& u, A* a)
    {
        a[0] = __uint_as_float(u.x); a[1] = __uint_as_float(u.y);
        a[2] = __uint_as_float(u.z); a[3] = __uint_as_float(u.w);
    }
    static __device__ __forceinline__ uint4 pack(const A* a)
    {
        return make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]),
                          __float_as_uint(a[2]), __float_as_uint(a[3]));
    }
};

struct TraitsI32 {
    using T = int32_t;
    using A = uint32_t;
    static constexpr int V = 4;
    static __device__ __forceinline__ A one() { return 1u; }
    static __device__ __forceinline__ A widen(T v) { return (uint32_t)v; }
    static __device__ __forceinline__ T narrow(A a) { return (int32_t)a; }
    static __device__ __forceinline__ void unpack(const uint4& u, A* a)
    {
        a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
    }
    static __device__ __forceinline__ uint4 pack(const A* a)
    {
        return make_uint4(a[0], a[1], a[2], a[3]);
    }
};

// IEEE binary16 stored as its 16-bit pattern.
struct TraitsF16 {
    using T = uint16_t;
    using A = float;
    static constexpr int V = 8;
    static __device__ __forceinline__ A one() { return 1.0f; }
    static __device__ __forceinline__ A widen(T v)
    {
        return (float)__builtin_bit_cast(_Float16, v);
    }
    static __device__ __forceinline__ T narrow(A a)
    {
        return __builtin_bit_cast(uint16_t, (_Float16)a); // round to nearest even
    }
    static __device__ __forceinline__ void unpack(const uint4& u, A* a)
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[2 * k] = widen((uint16_t)(w[k] & 0xffffu));
            a[2 * k + 1] = widen((uint16_t)(w[k] >> 16));
        }
    }
    static __device__ __forceinline__ uint4 pack(const A* a)
    {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)narrow(a[2 * k]) | ((uint32_t)narrow(a[2 * k + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};

// bfloat16 stored as its 16-bit pattern: the upper half of a binary32.
struct TraitsBF16 {
    using T = uint16_t;
    using A = float;
    static constexpr int V = 8;
    static __device__ __forceinline__ A one() { return 1.0f; }
    static __device__ __forceinline__ A widen(T v)
    {
        return __uint_as_float((uint32_t)v << 16);
    }
    static __device__ __forceinline__ T narrow(A a)
    {
        const uint32_t u = __float_as_uint(a);
        if ((u & 0x7fffffffu) > 0x7f800000u)
            return (uint16_t)((u >> 16) | 0x0040u); // NaN stays a quiet NaN
        return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
    static __device__ __forceinline__ void unpack(const uint4& u, A* a)
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[2 * k] = __uint_as_float(w[k] << 16);
            a[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ uint4 pack(const A* a)
    {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)narrow(a[2 * k]) | ((uint32_t)narrow(a[2 * k + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};

// int16 / uint16 stored as their 16-bit patterns.  Products are taken in
// uint32 and truncated once at the end: reduction modulo 2^16 commutes with
// multiplication, so the low 16 bits are those of the exact product for the
// signed and the unsigned reading alike.
struct TraitsU16 {
    using T = uint16_t;
    using A = uint32_t;
    static constexpr int V = 8;
    static __device__ __forceinline__ A one() { return 1u; }
    static __device__ __forceinline__ A widen(T v) { return (uint32_t)v; }
    static __device__ __forceinline__ T narrow(A a) { return (uint16_t)(a & 0xffffu); }
    static __device__ __forceinline__ void unpack(const uint4& u, A* a)
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[2 * k] = w[k] & 0xffffu;
            a[2 * k + 1] = w[k] >> 16;
        }
    }
    static __device__ __forceinline__ uint4 pack(const A* a)
    {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)narrow(a[2 * k]) | ((uint32_t)narrow(a[2 * k + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};

// Product, the TCOLPROD operator, over the accumulator type A.
template <class A>
struct OpMul {
    static __device__ __forceinline__ A identity() { return A(1); }
    static __device__ __forceinline__ A apply(A a, A b) { return a * b; }
};

// VEC: src is 16-byte aligned and ld * sizeof(T) is a multiple of 16, so
// every lane's V columns of every row form one aligned 16-byte vector.
// Op combines accumulators (OpMul for TCOLPROD; OpSum / OpMax / OpMin for
// the column sum / max / min).  Under accum (never for products) the old
// dst[j] is folded in first.
//
// A column block is kCols = 16 * V columns (256 bytes of each row).  A
// workgroup's THREADS threads form THREADS / 16 row groups of 16 lanes, GPB
// row groups per column block, so that it owns THREADS / 16 / GPB adjacent
// column blocks: row group gr of a block reads rows gr, gr + GPB,
// gr + 2 GPB, ... of each of its chunks of GPB * RIF rows, each lane one
// 16-byte vector per row, with RIF = kRowsInFlight * 256 / THREADS rows in
// flight (32 KiB in flight per workgroup whatever its size).  The GPB
// partial products of a block are combined in LDS in row-group order
// (GPB = 1 stores straight from the lanes).  One block per workgroup (512
// threads, GPB = 32, 4 rows in flight; a wave reading 256 bytes of four
// rows) serves tiles of many rows; GPB = 4 and 1 (256 threads) give short,
// wide tiles fewer and longer-lived workgroups, a wave reading 1 KiB of a
// row.  Every layout walks the rows in chunks of 128.  (Measured on MI355X
// for a 4096 x 16384 fp32 tile read from HBM: 40.6 us per call with 256
// workgroups of one block and no second pass, against 44.1 us for
// workgroups of 256 columns whose waves each read 1 KiB of a row, split
// four ways over the rows and finished by a second kernel.  One block per
// workgroup as 512 threads with 4 rows in flight against 256 threads with
// 8, interleaved on one box: fp32 42.4 -> 41.3 us, int32 42.1 -> 41.3, bf16
// 2048 x 32768 21.6 -> 21.2, fp16 21.6 -> 21.4; 1024 threads with 2 rows in
// flight 42.3 / 42.3 / 22.1 / 22.3; 256 threads with 4 rows 44.5.)
// The work of workgroup `wg` along the columns and `s` of S along the rows.
// The rows are walked in chunks of GPB * RIF (each row group's rows in
// flight at once); with S > 1 workgroup s takes chunks s, s + S, s + 2S, ...
// (grid-stride along the rows).
template <class Tr, class Op, bool VEC, int GPB, int THREADS = kBlock>
__device__ __forceinline__ void colred_blocks(
    const typename Tr::T* __restrict__ src, uint64_t R, uint64_t C,
    uint64_t ld, typename Tr::T* __restrict__ dst,
    typename Tr::A* __restrict__ partials, int accum,
    uint64_t wg, uint64_t s, uint32_t S)
{
    using T = typename Tr::T;
    using A = typename Tr::A;
    constexpr int V = Tr::V;
    constexpr int kCols = kLanesPerRow * V;          // columns per block
    constexpr int kGroups = THREADS / kLanesPerRow;  // row groups per workgroup
    constexpr int kBlocksPerWg = kGroups / GPB;
    constexpr int RIF = kRowsInFlight * kBlock / THREADS; // rows in flight per lane
    static_assert(kGroups % GPB == 0, "row groups split evenly over blocks");
    static_assert(RIF >= 1 && RIF * THREADS == kRowsInFlight * kBlock, "same bytes in flight");

    // Row g of the LDS combine holds row group g's partial products, column
    // c of the block at index (c mod V) * 16 + c / V for 16-byte vector
    // lanes and c for element lanes (lane q's k-th value at k * 16 + q
    // either way), each row padded by 16: one store instruction of a wave
    // (four row groups) then hits 64 distinct banks.
    constexpr int kLdsRow = kCols + kLanesPerRow;
    __shared__ A lds[GPB > 1 ? kGroups : 1][GPB > 1 ? kLdsRow : 1];

    const uint32_t g = threadIdx.x / kLanesPerRow;
    const uint32_t q = threadIdx.x % kLanesPerRow;
    const uint32_t gr = g % GPB;                      // row group within the block
    const uint64_t cb = wg * kBlocksPerWg + g / GPB;
    const uint64_t jb = cb * kCols; // first column of the block
    constexpr uint64_t kChunk = (uint64_t)GPB * RIF;
    const uint64_t step = (uint64_t)S * kChunk;
    const bool full = VEC && jb + kCols <= C;

    A acc[V];
#pragma unroll
    for (int k = 0; k < V; ++k)
        acc[k] = Op::identity();

    // The chunk that reaches past R (if it is this workgroup's) is the last
    // one: its remaining rows are read one at a time.
    uint64_t r = s * kChunk + gr;
    if (jb >= C) {
        // A block past the last column (the last workgroup's last blocks
        // when its kBlocksPerWg blocks do not divide the block count):
        // nothing to read; its row groups combine the identity.
    } else if (full) {
        // Lane q owns columns jb + qV .. jb + qV + V - 1: one 16-byte vector
        // per row.
        const T* __restrict__ col = src + jb + (uint64_t)q * V;
        for (; r + (uint64_t)GPB * (RIF - 1) < R; r += step) {
            uint4 v[RIF];
#pragma unroll
            for (int u = 0; u < RIF; ++u)
                v[u] = load_stream(reinterpret_cast<const uint4*>(
                    col + (r + (uint64_t)u * GPB) * ld));
#pragma unroll
            for (int u = 0; u < RIF; ++u) {
                A a[V];
                Tr::unpack(v[u], a);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    acc[k] = Op::apply(acc[k], a[k]);
            }
        }
        for (; r < R; r += GPB) {
            A a[V];
            Tr::unpack(load_stream(reinterpret_cast<const uint4*>(col + r * ld)), a);
#pragma unroll
            for (int k = 0; k < V; ++k)
                acc[k] = Op::apply(acc[k], a[k]);
        }
    } else {
        // Rows not 16-byte aligned, or the ragged last column block:
        // element loads, lane q owning columns jb + q + 16k, so that each
        // load instruction of a row group reads 16 consecutive elements.
        // RIF rows are requested before any is folded; columns
        // at or past C reload column jb (always valid) and are not folded.
        const T* __restrict__ blk = src + jb;
        uint32_t off[V];
        bool ok[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t c = q + (uint32_t)kLanesPerRow * k;
            ok[k] = jb + c < C;
            off[k] = ok[k] ? c : 0u;
        }
        for (; r + (uint64_t)GPB * (RIF - 1) < R; r += step) {
            T v[RIF][V];
#pragma unroll
            for (int u = 0; u < RIF; ++u)
#pragma unroll
                for (int k = 0; k < V; ++k)
                    v[u][k] = blk[(r + (uint64_t)u * GPB) * ld + off[k]];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < RIF; ++u)
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (ok[k])
                        acc[k] = Op::apply(acc[k], Tr::widen(v[u][k]));
        }
        for (; r < R; r += GPB) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (ok[k])
                    acc[k] = Op::apply(acc[k], Tr::widen(blk[r * ld + off[k]]));
        }
    }

    if constexpr (GPB == 1) {
        // One row group per block: each lane holds its columns' results.
        if (jb < C) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint64_t j = jb + (full ? (uint64_t)q * V + k
                                              : (uint64_t)q + (uint64_t)kLanesPerRow * k);
                if (j < C) {
                    if (S == 1)
                        dst[j] = Tr::narrow(accum ? Op::apply(Tr::widen(dst[j]), acc[k]) : acc[k]);
                    else
                        partials[s * C + j] = acc[k];
                }
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k)
            lds[g][k * kLanesPerRow + q] = acc[k];
        // Combine each block's row groups' partial rows in row-group order.
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < (uint32_t)(kBlocksPerWg * kCols); i += THREADS) {
            const uint32_t b = i / kCols;
            const uint32_t e = i % kCols; // LDS index: value e / 16 of lane e % 16
            A p = lds[b * GPB][e];
#pragma unroll
            for (int w = 1; w < GPB; ++w)
                p = Op::apply(p, lds[b * GPB + w][e]);
            // Block b's own layout decides the column of index e: with several
            // blocks per workgroup, the thread combining it need not be one of
            // the block's readers, and a ragged last block is read in elements
            // while its neighbours are read in vectors.
            const uint64_t jb_b = (wg * kBlocksPerWg + b) * kCols;
            const bool full_b = VEC && jb_b + kCols <= C;
            const uint32_t c = full_b ? (e % kLanesPerRow) * V + e / kLanesPerRow : e;
            const uint64_t j = jb_b + c;
            if (j < C) {
                if (S == 1)
                    dst[j] = Tr::narrow(accum ? Op::apply(Tr::widen(dst[j]), p) : p);
                else
                    partials[s * C + j] = p;
            }
        }
    }
}

// Workgroups are dispatched round-robin over the 8 XCDs (by linear index),
// each XCD with its own L2.  When rows do not start on 128-byte lines,
// neighbouring column blocks share a line in every row, and blocks on
// different XCDs each fetch it.  With `xcd_contiguous` the workgroups are
// taken in slice-major order (all column workgroups of row share s, then
// s + 1, ...) and XCD x gets one contiguous run of that order, so an XCD
// holds whole row shares with adjacent column blocks.  (Measured on MI355X:
// a 4096 x 16383 fp32 tile 59.6 -> 49.7 us, 2048 x 32767 bf16 32.1 -> 28.5
// us; no gain for tiles of 128-byte aligned rows, which keep the plain
// order.)
__device__ __forceinline__ void column_workgroup(int xcd_contiguous, uint64_t& wg, uint64_t& s)
{
    if (!xcd_contiguous) {
        wg = blockIdx.x;
        s = blockIdx.y;
        return;
    }
    constexpr uint32_t kXcds = 8;
    const uint32_t nx = gridDim.x;
    const uint32_t n = nx * gridDim.y;
    const uint32_t lin = blockIdx.x + blockIdx.y * nx;
    const uint32_t q = n / kXcds, rem = n % kXcds;
    const uint32_t x = lin % kXcds, i = lin / kXcds;
    const uint32_t f = x * q + (x < rem ? x : rem) + i; // slice-major position
    wg = f % nx;
    s = f / nx;
}

template <class Tr, class Op, bool VEC, int GPB, int THREADS>
__global__ __launch_bounds__(THREADS) void colred_kernel(
    const typename Tr::T* __restrict__ src, uint64_t R, uint64_t C,
    uint64_t ld, typename Tr::T* __restrict__ dst,
    typename Tr::A* __restrict__ partials, int accum, int xcd_contiguous)
{
    uint64_t wg, s;
    column_workgroup(xcd_contiguous, wg, s);
    colred_blocks<Tr, Op, VEC, GPB, THREADS>(src, R, C, ld, dst, partials, accum, wg, s,
                                             gridDim.y);
}

// Short, wide tiles with so many column blocks that a workgroup can own a
// strip of 16 * VPL whole blocks and the grid still has one workgroup per
// CU (16-byte aligned rows; never split along the rows).  A wave reads VPL
// KiB contiguous of a row: lane l owns the vectors l, l + 64, ..., of its
// wave's span, and RU = kRowsInFlight / VPL rows are requested before any
// is folded, so a lane keeps its loads in flight on one or two rows rather
// than on eight rows that lie megabytes apart.  Workgroups past the full
// strips take the remaining blocks (the ragged last block included) as
// the one-row-group-per-block layout does.  (Measured on MI355X, fp32
// column product of 256 MiB: 16 x 4 Mi 58.0 -> 44.8 us with VPL = 8,
// 64 x 1 Mi 56.1 -> 41.1 us with VPL = 4, bit-identical results.)
template <class Tr, class Op, int VPL>
__global__ __launch_bounds__(kBlock) void colred_wide_kernel(
    const typename Tr::T* __restrict__ src, uint64_t R, uint64_t C,
    uint64_t ld, typename Tr::T* __restrict__ dst, int accum, uint32_t full_strips)
{
    using T = typename Tr::T;
    using A = typename Tr::A;
    constexpr int V = Tr::V;
    constexpr int RU = kRowsInFlight / VPL;
    static_assert(RU * VPL == kRowsInFlight, "VPL divides the loads in flight");

    if (blockIdx.x >= full_strips) {
        colred_blocks<Tr, Op, true, 1>(src, R, C, ld, dst, nullptr, accum,
                                       (uint64_t)full_strips * VPL + (blockIdx.x - full_strips),
                                       0, 1);
        return;
    }
    const uint32_t w = threadIdx.x / kWave;
    const uint32_t l = threadIdx.x % kWave;
    // First column of the lane's vector m = 0; vector m starts 64 V later.
    const uint64_t col0 = (((uint64_t)blockIdx.x * kWaves + w) * VPL * kWave + l) * V;
    const T* __restrict__ col = src + col0;

    A acc[VPL][V];
#pragma unroll
    for (int m = 0; m < VPL; ++m)
#pragma unroll
        for (int k = 0; k < V; ++k)
            acc[m][k] = Op::identity();

    auto fold = [&](int m, const uint4& u) {
        A a[V];
        Tr::unpack(u, a);
#pragma unroll
        for (int k = 0; k < V; ++k)
            acc[m][k] = Op::apply(acc[m][k], a[k]);
    };
    uint64_t r = 0;
    for (; r + RU <= R; r += RU) {
        uint4 v[RU][VPL];
#pragma unroll
        for (int u = 0; u < RU; ++u)
#pragma unroll
            for (int m = 0; m < VPL; ++m)
                v[u][m] = load_stream(reinterpret_cast<const uint4*>(
                    col + (r + u) * ld + (uint64_t)m * kWave * V));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < RU; ++u)
#pragma unroll
            for (int m = 0; m < VPL; ++m)
                fold(m, v[u][m]);
    }
    for (; r < R; ++r)
#pragma unroll
        for (int m = 0; m < VPL; ++m)
            fold(m, load_stream(reinterpret_cast<const uint4*>(
                col + r * ld + (uint64_t)m * kWave * V)));

    // One row of results per C elements read: with a 16-byte aligned dst
    // each lane stores (and, under accum, first reads) whole vectors.
    if (((uintptr_t)dst & 15u) == 0) {
#pragma unroll
        for (int m = 0; m < VPL; ++m) {
            uint4* p = reinterpret_cast<uint4*>(dst + col0 + (uint64_t)m * kWave * V);
            A o[V];
            if (accum) {
                Tr::unpack(*p, o);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    o[k] = Op::apply(o[k], acc[m][k]);
            } else {
#pragma unroll
                for (int k = 0; k < V; ++k)
                    o[k] = acc[m][k];
            }
            *p = Tr::pack(o);
        }
    } else {
#pragma unroll
        for (int m = 0; m < VPL; ++m)
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint64_t j = col0 + (uint64_t)m * kWave * V + k;
                dst[j] = Tr::narrow(accum ? Op::apply(Tr::widen(dst[j]), acc[m][k]) : acc[m][k]);
            }
    }
}

// Narrow rows (a row narrower than 256 bytes): the column-block layout
// above would leave most lanes idle, so a workgroup reads whole rows
// instead.  The unit a thread reads per row is one aligned 16-byte vector
// of V elements when VEC (tile 16-byte aligned, ld * sizeof(T) and
// C * sizeof(T) multiples of 16), else one element; a row is W units.
// Thread t owns unit cu = t % W of row offset ro = t / W; RB = 256 / W rows
// form one step, read as RB * W consecutive units (threads past RB * W and
// units of padding columns stay idle).  Steps are taken NF at a time as
// sweeps of NF * RB rows (NF = 8 vector rows, or 64 bytes of element rows
// per lane), and workgroup s walks sweeps s, s + S, s + 2S, ... (grid-
// stride, as the 1-D stream).  Each thread folds its rows in
// increasing order; the RB row offsets are then combined in LDS by a fixed
// pairwise tree, and the threads of row offset 0 store the workgroup's
// partial row (or dst when S == 1).
template <class Tr, class Op, bool VEC>
__global__ __launch_bounds__(kBlock) void colred_narrow_kernel(
    const typename Tr::T* __restrict__ src, uint64_t R, uint64_t C,
    uint64_t ld, uint32_t W, typename Tr::T* __restrict__ dst,
    typename Tr::A* __restrict__ partials, int accum)
{
    using T = typename Tr::T;
    using A = typename Tr::A;
    constexpr int U = VEC ? Tr::V : 1; // elements per unit
    constexpr int NF = VEC ? kRowsInFlight : kElemRowsInFlight<T>; // rows in flight

    __shared__ A lds[kBlock][U];

    const uint32_t RB = kBlock / W;
    const uint32_t t = threadIdx.x;
    const uint32_t ro = t / W;
    const uint32_t cu = t - ro * W;
    const bool live = ro < RB && (uint64_t)cu * U < C;
    const uint32_t S = gridDim.x;
    const uint64_t s = blockIdx.x;

    A acc[U];
#pragma unroll
    for (int k = 0; k < U; ++k)
        acc[k] = Op::identity();

    auto fold_row = [&](const T* p) {
        if constexpr (VEC) {
            A a[U];
            Tr::unpack(load_stream(reinterpret_cast<const uint4*>(p)), a);
#pragma unroll
            for (int k = 0; k < U; ++k)
                acc[k] = Op::apply(acc[k], a[k]);
        } else {
            acc[0] = Op::apply(acc[0], Tr::widen(__builtin_nontemporal_load(p)));
        }
    };

    if (live) {
        const T* __restrict__ col = src + (uint64_t)cu * U;
        const uint64_t sweep = (uint64_t)NF * RB;
        uint64_t r = s * sweep + ro;
        for (; r + (uint64_t)(NF - 1) * RB < R; r += (uint64_t)S * sweep) {
            if constexpr (VEC) {
                uint4 v[NF];
#pragma unroll
                for (int u = 0; u < NF; ++u)
                    v[u] = load_stream(reinterpret_cast<const uint4*>(
                        col + (r + (uint64_t)u * RB) * ld));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < NF; ++u) {
                    A a[U];
                    Tr::unpack(v[u], a);
#pragma unroll
                    for (int k = 0; k < U; ++k)
                        acc[k] = Op::apply(acc[k], a[k]);
                }
            } else {
                T v[NF];
#pragma unroll
                for (int u = 0; u < NF; ++u)
                    v[u] = __builtin_nontemporal_load(col + (r + (uint64_t)u * RB) * ld);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < NF; ++u)
                    acc[0] = Op::apply(acc[0], Tr::widen(v[u]));
            }
        }
        // The sweep that reaches past R (if it is this workgroup's) is the
        // last one: its remaining rows are read one step at a time.
        for (; r < R; r += RB)
            fold_row(col + r * ld);
    }
#pragma unroll
    for (int k = 0; k < U; ++k)
        lds[t][k] = acc[k];

    uint32_t half = 1;
    while (half * 2 < RB)
        half *= 2;
    for (; half >= 1; half /= 2) {
        __syncthreads();
        if (ro < half && ro + half < RB) {
#pragma unroll
            for (int k = 0; k < U; ++k)
                lds[t][k] = Op::apply(lds[t][k], lds[t + half * W][k]);
        }
    }
    __syncthreads();

    if (ro == 0 && live) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint64_t j = (uint64_t)cu * U + k;
            const A p = lds[t][k];
            if (S == 1)
                dst[j] = Tr::narrow(accum ? Op::apply(Tr::widen(dst[j]), p) : p);
            else
                partials[s * C + j] = p;
        }
    }
}

// Second pass (S > 1).  Workgroup b takes FC consecutive columns (FC a power
// of two chosen by the host so that each thread has few slices to read);
// its threads form H = 256 / FC slice groups.  Thread (h, c) folds slices
// h, h + H, h + 2H, ... of its column in increasing order with eight loads
// in flight, the H values of a column are combined in LDS by a fixed
// pairwise tree, and the result is folded after the old dst[j] under accum
// and narrowed once to T.
template <class Tr, class Op>
__global__ __launch_bounds__(kBlock) void colred_finish_kernel(
    const typename Tr::A* __restrict__ partials, uint32_t S, uint64_t C,
    uint32_t fc_log2, typename Tr::T* __restrict__ dst, int accum)
{
    using A = typename Tr::A;
    constexpr int kBatch = 8;
    __shared__ A lds[kBlock];

    const uint32_t FC = 1u << fc_log2;
    const uint32_t H = kBlock >> fc_log2;
    const uint32_t c = threadIdx.x & (FC - 1);
    const uint32_t h = threadIdx.x >> fc_log2;
    const uint64_t j = (uint64_t)blockIdx.x * FC + c;

    A p = Op::identity();
    if (j < C) {
        for (uint32_t k = h; k < S; k += kBatch * H) {
            A v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const uint32_t sl = k + u * H;
                v[u] = partials[(uint64_t)(sl < S ? sl : k) * C + j];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (k + u * H < S)
                    p = Op::apply(p, v[u]);
        }
    }
    lds[threadIdx.x] = p;
    for (uint32_t half = H / 2; half >= 1; half /= 2) {
        __syncthreads();
        if (h < half)
            lds[threadIdx.x] = Op::apply(lds[threadIdx.x], lds[threadIdx.x + half * FC]);
    }
    __syncthreads();
    if (h == 0 && j < C) {
        const A q = lds[threadIdx.x];
        dst[j] = Tr::narrow(accum ? Op::apply(Tr::widen(dst[j]), q) : q);
    }
}

template <class Tr, class Op>
hipError_t launch_typed(const void* src, size_t R, size_t C, size_t ld,
                        void* dst, int accum, const ColprodPlan& plan,
                        const Workspace& ws, hipStream_t stream)
{
    using T = typename Tr::T;
    using A = typename Tr::A;
    const bool vec = (((uintptr_t)src & 15u) == 0) && ((ld * sizeof(T)) % 16 == 0);
    const T* s = static_cast<const T*>(src);
    T* d = static_cast<T*>(dst);
    A* part = static_cast<A*>(ws.partials);
    if (plan.narrow_w) {
        if (plan.narrow_vec)
            colred_narrow_kernel<Tr, Op, true><<<plan.splits, kBlock, 0, stream>>>(
                s, R, C, ld, plan.narrow_w, d, part, accum);
        else
            colred_narrow_kernel<Tr, Op, false><<<plan.splits, kBlock, 0, stream>>>(
                s, R, C, ld, plan.narrow_w, d, part, accum);
    } else if (plan.wide_vpl) {
        auto go = [&](auto kern) {
            kern<<<plan.wide_grid, kBlock, 0, stream>>>(s, R, C, ld, d, accum, plan.full_strips);
        };
        if (plan.wide_vpl == 8)
            go(colred_wide_kernel<Tr, Op, 8>);
        else if (plan.wide_vpl == 4)
            go(colred_wide_kernel<Tr, Op, 4>);
        else
            go(colred_wide_kernel<Tr, Op, 2>);
    } else {
        // group_rows is counted in row groups of a 256-thread workgroup: 1
        // or 4 run as such.  16 (one block per workgroup) runs as one block
        // of 32 row groups on 512 threads, with the same 128-row chunks,
        // when the workgroup walks its block's whole column (S = 1) or the
        // rows are not 16-byte aligned (element loads); aligned rows shared
        // by several workgroups keep 256 threads.  (Measured on MI355X,
        // interleaved A/B, 256 threads -> 512: 4096 x 16384 fp32 41.5 ->
        // 41.2 us, 4096 x 16383 fp32 50.6 -> 42.0, one element past
        // alignment 51.0 -> 49.2, 2048 x 32767 bf16 27.7 -> 23.0; with the
        // rows shared, 8192 x 8192 44.1 -> 43.2 and 16384 x 4096 45.6 ->
        // 44.7 but 65536 x 1024 41.8 -> 43.8 and 257 blocks split 6 ways
        // 44.0 -> 44.6.)
        const bool wide_wg = plan.splits == 1 || !vec;
        const unsigned per_wg = kBlock / kLanesPerRow / plan.group_rows;
        const dim3 grid((plan.col_blocks + per_wg - 1) / per_wg, plan.splits);
        const int xcd = (((uintptr_t)src & 127u) != 0) || ((ld * sizeof(T)) % 128 != 0);
        auto go = [&](auto kern, unsigned threads) {
            kern<<<grid, threads, 0, stream>>>(s, R, C, ld, d, part, accum, xcd);
        };
        if (plan.group_rows == 1)
            vec ? go(colred_kernel<Tr, Op, true, 1, kBlock>, kBlock)
                : go(colred_kernel<Tr, Op, false, 1, kBlock>, kBlock);
        else if (plan.group_rows == 4)
            vec ? go(colred_kernel<Tr, Op, true, 4, kBlock>, kBlock)
                : go(colred_kernel<Tr, Op, false, 4, kBlock>, kBlock);
        else if (!wide_wg)
            go(colred_kernel<Tr, Op, true, 16, kBlock>, kBlock);
        else
            vec ? go(colred_kernel<Tr, Op, true, 32, 2 * kBlock>, 2 * kBlock)
                : go(colred_kernel<Tr, Op, false, 32, 2 * kBlock>, 2 * kBlock);
    }
    if (plan.splits > 1)
        colred_finish_kernel<Tr, Op><<<plan.finish_blocks, kBlock, 0, stream>>>(
            part, plan.splits, C, plan.finish_cols_log2, d, accum);
    return hipGetLastError();
}

} // namespace

size_t colprod_elem_size(ColType t)
{
    return (t == ColType::F16 || t == ColType::BF16 || t == ColType::U16) ? 2 : 4;
}

constexpr uint64_t kMaxSplits = 65535; // gridDim.y limit
// Workgroups per compute unit for the narrow-row kernel (grid-stride).
#ifndef RED_COLPROD_NARROW_WG_PER_CU
#define RED_COLPROD_NARROW_WG_PER_CU 2
#endif
constexpr uint64_t kNarrowWgPerCu = RED_COLPROD_NARROW_WG_PER_CU;
#ifndef RED_COLPROD_NARROW_ELEM_WG_PER_CU
#define RED_COLPROD_NARROW_ELEM_WG_PER_CU 2
#endif
constexpr uint64_t kNarrowElemWgPerCu = RED_COLPROD_NARROW_ELEM_WG_PER_CU;
// Row groups per column block, from the fewest the planner may choose
// (1, 4 or 16).
#ifndef RED_COLPROD_MIN_GROUP_ROWS
#define RED_COLPROD_MIN_GROUP_ROWS 1
#endif
constexpr uint64_t kMinGroupRows = RED_COLPROD_MIN_GROUP_ROWS;
// Most vectors per lane of the wide-strip kernel (8, 4 or 2; a divisor of
// the rows in flight).
#ifndef RED_COLPROD_MAX_WIDE_VPL
#define RED_COLPROD_MAX_WIDE_VPL 8
#endif
constexpr uint64_t kMaxWideVpl = RED_COLPROD_MAX_WIDE_VPL;
// Row shares for tiles whose workgroups overrun a multiple of the CU count
// by at most a quarter of it.
#ifndef RED_COLPROD_OVER_SPLITS
#define RED_COLPROD_OVER_SPLITS 6
#endif
constexpr uint64_t kOverSplits = RED_COLPROD_OVER_SPLITS;
// Second pass: at most this many slices per thread when the column count
// allows it.
constexpr uint64_t kFinishSlicesPerThread = 8;

ColprodPlan colprod_plan(ColType t, const void* src, size_t R, size_t C, size_t ld,
                         const DeviceInfo& dev, const Workspace& ws)
{
    ColprodPlan p;
    const uint64_t es = colprod_elem_size(t);
    const bool vec = (((uintptr_t)src & 15u) == 0) && ((ld * es) % 16 == 0);
    uint64_t S = 1;
    if (ld * es < (uint64_t)kLanesPerRow * 16) {
        // Narrow rows: one workgroup spans whole rows, in 16-byte vectors
        // when the tile allows, else in elements; the grid-stride walk
        // covers every sweep whatever S is.
        p.narrow_vec = vec && (C * es) % 16 == 0;
        p.narrow_w = (unsigned)(p.narrow_vec ? ld * es / 16 : ld);
        p.col_blocks = 1;
        const uint64_t rows_per_step = kBlock / p.narrow_w;
        const uint64_t sweep = rows_per_step *
            (p.narrow_vec ? kRowsInFlight : RED_COLPROD_ELEM_BYTES_IN_FLIGHT / es);
        const uint64_t sweeps = (R + sweep - 1) / sweep;
        S = (uint64_t)dev.cus * (p.narrow_vec ? kNarrowWgPerCu : kNarrowElemWgPerCu);
        if (S > sweeps)
            S = sweeps;
        while (S > 1 && S * C * 4 > ws.partial_bytes)
            S = (S + 1) / 2;
        if (S < 1)
            S = 1;
    } else {
        const uint64_t cols = (uint64_t)kLanesPerRow * (16 / es);
        p.col_blocks = (unsigned)((C + cols - 1) / cols);
        const uint64_t target = (uint64_t)dev.cus * kColprodWgPerCu;
        // Fewest row groups per block that still give the grid `target`
        // workgroups; tiles with fewer blocks than that keep 16 and split
        // their rows instead.
        const uint64_t groups = kBlock / kLanesPerRow;
        p.group_rows = (unsigned)groups;
        for (uint64_t g = kMinGroupRows; g < groups; g *= 4) {
            if ((p.col_blocks * g + groups - 1) / groups >= target) {
                p.group_rows = (unsigned)g;
                break;
            }
        }
        // Row shares per block.  Each workgroup streams until its share is
        // done, so the time goes as the rounds of workgroups the CUs run
        // divided by the workgroups: of floor(target / wgs) and the ceiling,
        // take the one with less of it (a grid a little over the CU count
        // leaves its extra workgroups a second round of their own).  On a
        // tie, aligned rows take fewer workgroups and unaligned rows (element
        // loads, which gain from more loads in flight) more.  (Measured on
        // MI355X, 256 MiB fp32 tiles of 62 column blocks: 5 shares, 310
        // workgroups, 52.8 us; 4 shares, 248 workgroups, 43.1 us.  4096 x
        // 16000 of stride 16001: 2 shares 50.4 us, 1 share 53.5 us.)
        const uint64_t wgs = (p.col_blocks * p.group_rows + groups - 1) / groups;
        const bool lines = (((uintptr_t)src & 127u) == 0) && ((ld * es) % 128 == 0);
        const uint64_t chunk_rows = (uint64_t)p.group_rows * kRowsInFlight;
        if (wgs > target && lines && p.group_rows > 1 && wgs % target != 0 &&
            (wgs % target) * 4 <= target &&
            (R + chunk_rows - 1) / chunk_rows >= kOverSplits) {
            // A last round of workgroups at most a quarter full runs alone
            // for as long as a full round: kOverSplits row shares, each of
            // at least one chunk (32 KiB per workgroup), turn it into a
            // short tail at the price of the second pass.  Rows off
            // 128-byte lines keep one share (they read lines shared by
            // neighbouring blocks, and their shorter workgroups were
            // slower), and tiles of one row group per block have the
            // wide-strip kernel.  (Measured on MI355X, fp32 tiles, one
            // share -> six: 256 MiB of 257 blocks 55.1 -> 44.2 us, 520
            // blocks 54.3 -> 46.6, 1100 blocks of 4 row groups 55.8 -> 47.7;
            // 64 MiB of 257 blocks 16.0 -> 15.0, 272 blocks 17.4 -> 15.0.
            // With fewer than six chunks per block the second pass and the
            // shorter workgroups cost more than the tail: 64 MiB of 776
            // blocks, 3 chunks, one share 14.3 us, three 15.7 us.  Fuller last rounds gained at 256 MiB
            // and lost at 64 MiB: 384 blocks 49.3 -> 46.8 but 14.0 -> 15.0.)
            S = kOverSplits;
        } else if (wgs < target) {
            const uint64_t lo = target / wgs;
            const uint64_t hi = (target + wgs - 1) / wgs;
            S = lo;
            if (hi != lo) {
                const uint64_t rounds_lo = (wgs * lo + target - 1) / target;
                const uint64_t rounds_hi = (wgs * hi + target - 1) / target;
                // rounds_hi / (wgs hi) against rounds_lo / (wgs lo)
                const uint64_t cost_hi = rounds_hi * lo, cost_lo = rounds_lo * hi;
                if (cost_hi < cost_lo || (cost_hi == cost_lo && !vec))
                    S = hi;
            }
        }
        // At least one chunk of rows per workgroup.
        const uint64_t chunk = (uint64_t)p.group_rows * kRowsInFlight;
        const uint64_t chunks = (R + chunk - 1) / chunk;
        if (S > chunks)
            S = chunks;
        if (S > kMaxSplits)
            S = kMaxSplits;
        // The workspace bounds S * C partial values.
        while (S > 1 && S * C * 4 > ws.partial_bytes)
            S = (S + 1) / 2;
        if (S < 1)
            S = 1;
        // Wide strips: the most vectors per lane that still give every CU a
        // workgroup of whole blocks.
        if (vec && p.group_rows == 1 && S == 1) {
            const uint64_t full_blocks = C / cols;
            for (uint64_t vpl = kMaxWideVpl; vpl >= 2; vpl /= 2) {
                const uint64_t strips = full_blocks / (groups * vpl);
                if (strips >= target) {
                    const uint64_t tail = p.col_blocks - strips * groups * vpl;
                    p.wide_vpl = (unsigned)vpl;
                    p.full_strips = (unsigned)strips;
                    p.wide_grid = (unsigned)(strips + (tail + groups - 1) / groups);
                    break;
                }
            }
        }
    }
    p.splits = (unsigned)S;
    p.partial_bytes = S > 1 ? S * C * 4 : 0;
    if (S > 1) {
        // Columns per second-pass workgroup: a power of two, no wider than
        // needed to cover C, and narrow enough that each thread reads at
        // most kFinishSlicesPerThread slices when it can.
        uint32_t lg = 8; // 256 columns
        while (lg > 0 && (((uint64_t)1 << lg) * S > kBlock * kFinishSlicesPerThread ||
                          ((uint64_t)1 << lg) >= 2 * C))
            --lg;
        p.finish_cols_log2 = lg;
        p.finish_blocks = (unsigned)((C + ((uint64_t)1 << lg) - 1) >> lg);
    }
    return p;
}

hipError_t launch_colprod(ColType t, const void* src, size_t R, size_t C,
                          size_t ld, void* dst, const ColprodPlan& plan,
                          const Workspace& ws, hipStream_t stream)
{
    switch (t) {
    case ColType::F32: return launch_typed<TraitsF32, OpMul<float>>(src, R, C, ld, dst, 0, plan, ws, stream);
    case ColType::I32: return launch_typed<TraitsI32, OpMul<uint32_t>>(src, R, C, ld, dst, 0, plan, ws, stream);
    case ColType::F16: return launch_typed<TraitsF16, OpMul<float>>(src, R, C, ld, dst, 0, plan, ws, stream);
    case ColType::BF16: return launch_typed<TraitsBF16, OpMul<float>>(src, R, C, ld, dst, 0, plan, ws, stream);
    case ColType::U16: return launch_typed<TraitsU16, OpMul<uint32_t>>(src, R, C, ld, dst, 0, plan, ws, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cols(OpKind op, const float* src, size_t R, size_t C,
                       size_t ld, float* dst, int accum, const ColprodPlan& plan,
                       const Workspace& ws, hipStream_t stream)
{
    switch (op) {
    case OpKind::Sum: return launch_typed<TraitsF32, OpSum>(src, R, C, ld, dst, accum, plan, ws, stream);
    case OpKind::Max: return launch_typed<TraitsF32, OpMax>(src, R, C, ld, dst, accum, plan, ws, stream);
    case OpKind::Min: return launch_typed<TraitsF32, OpMin>(src, R, C, ld, dst, accum, plan, ws, stream);
    }
    return hipErrorInvalidValue;
}

} // namespace red
