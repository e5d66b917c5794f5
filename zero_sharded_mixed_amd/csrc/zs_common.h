// zs_common.h — definitions shared by the shard-pipeline kernels and their host entry points.
//
// Index spaces the kernels walk (see include/zero_shard.h for the layout):
//   * shard columns x in [0, shard_numel): rank r's flat fp32 shard.  Bucket b owns
//     [O_b, O_b + L_b); column x of the shard is column x - O_b of every rank row of b.
//     Parameter i owns [off_i, end_i), end_i = off_i + s_i.  end_i never decreases with i.
//   * unpack chunks u in [0, total_chunks): parameter i owns chunks [ucb_i, ucend_i),
//     ucend_i - ucb_i = ceil(numel_i / 8); chunk u covers its elements 8*(u - ucb_i) + 0..7.
// Both spaces are cut into tiles; tile_first[j] is the first parameter whose range ends after
// the tile's first column (or chunk), so the parameter owning any point of tile j is found by
// a binary search over [tile_first[j], tile_first[j+1]] — usually a range of one or two.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_shard.h"
#include "zs_grid.h"

namespace zs {

constexpr int kBlock = 256;                  // threads per block in every hot kernel
constexpr int kChunk = 8;                    // elements per thread chunk (16 bytes of 16-bit data)
constexpr int kTileShift = 11;               // shard tile = 2048 columns = one chunk per thread
constexpr int64_t kTileCols = int64_t(1) << kTileShift;
constexpr int kUTileShift = 8;               // unpack tile = 256 chunks = one chunk per thread
constexpr int64_t kUTileChunks = int64_t(1) << kUTileShift;
constexpr int32_t kMaxNd = 65535;
constexpr int64_t kMaxNumel = int64_t(1) << 48;

// Read-only view of a plan's device tables, passed to kernels by value.
struct DevPlan {
    int64_t n;            // parameters
    int64_t nd;           // ranks
    int64_t rank;
    int64_t shard_numel;  // sum of L_b
    int64_t n_tiles;      // ceil(shard_numel / kTileCols)
    int64_t n_utiles;     // ceil(total_chunks / kUTileChunks)
    const int64_t* numel;
    const int64_t* s;
    const int64_t* off;
    const int64_t* end;
    const double* inv_s;     // 1.0 / s_i (0 when s_i == 0)
    const int32_t* bucket;
    const int64_t* ucb;
    const int64_t* ucend;
    const int64_t* b_base;   // O_b
    const int64_t* b_stride; // L_b
    const int64_t* b_row;    // S_b
    const int32_t* tile_first;   // [n_tiles + 1]
    const int32_t* utile_first;  // [n_utiles + 1]
};

// Address-space helpers.  Plan tables are never written by the hot kernels: reading them
// through the constant address space lets a block-uniform index become a scalar load.  Data
// pointers taken from the caller's pointer tables are generic; casting them to the global
// address space gives global (not flat) loads and stores.
#define ZS_CONST __attribute__((address_space(4)))
#define ZS_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
    return ((const ZS_CONST T*)p)[i];
}
__device__ __forceinline__ float2 ld_const_f2(const float2* p, int64_t i) {
    const uint64_t u = ld_const(reinterpret_cast<const uint64_t*>(p), i);
    return make_float2(__uint_as_float(uint32_t(u)), __uint_as_float(uint32_t(u >> 32)));
}
template <class T>
__device__ __forceinline__ const ZS_GLOBAL T* gptr(const T* p) {
    return (const ZS_GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ ZS_GLOBAL T* gptr(T* p) {
    return (ZS_GLOBAL T*)p;
}

// First index i in [lo, hi] with key[i] > x, given key non-decreasing and key[hi] > x
// (or hi == n).  Returns hi when none before it qualifies.
__device__ __forceinline__ int64_t first_greater(const int64_t* __restrict__ key, int64_t lo, int64_t hi, int64_t x) {
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (key[mid] > x) hi = mid; else lo = mid + 1;
    }
    return lo;
}

// Parameter whose shard range could hold column x: the first i with end_i > x (n if none).
// The caller checks off_i <= x (otherwise x lies in a row gap).
__device__ __forceinline__ int64_t param_of_column(const DevPlan& P, int64_t x) {
    int64_t j = x >> kTileShift;
    return first_greater(P.end, ld_const(P.tile_first, j), ld_const(P.tile_first, j + 1), x);
}

// Parameter owning unpack chunk u (first i with ucend_i > u).
__device__ __forceinline__ int64_t param_of_chunk(const DevPlan& P, int64_t u) {
    int64_t j = u >> kUTileShift;
    return first_greater(P.ucend, ld_const(P.utile_first, j), ld_const(P.utile_first, j + 1), u);
}

// 16-byte global loads and stores (native vector types: the HIP vector classes cannot be
// copied across address spaces).
typedef uint32_t zs_u32x4 __attribute__((ext_vector_type(4)));
typedef float zs_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const void* p) {
    const zs_u32x4 w = *gptr(reinterpret_cast<const zs_u32x4*>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}
// The same at base + byte_off with base uniform across the wavefront: the address is one
// scalar base and a 32-bit per-lane offset, so a thread holding loads of many rows in flight
// spends one register on their addresses rather than two per row.
// NT: a nontemporal load, for streams whose every load instruction covers whole cache lines.
template <bool NT = false>
__device__ __forceinline__ uint4 load16_off(const uint16_t* base, uint32_t byte_off) {
    const ZS_GLOBAL zs_u32x4* p = (const ZS_GLOBAL zs_u32x4*)((const ZS_GLOBAL char*)base + byte_off);
    zs_u32x4 w;
    if constexpr (NT) w = __builtin_nontemporal_load(p);
    else w = *p;
    return make_uint4(w.x, w.y, w.z, w.w);
}
// The 16-byte stores are nontemporal (the nt bit): every kernel writes each output once and no
// later work of the same kernel reads it.  Measured on MI355X against ordinary stores, in one
// process: unpack 5-8% faster, pack 0.4-3%, Adam 3%, the fused reduce + Adam 2-4%, the reduce
// 1%.  (Nontemporal loads are the opposite: a load instruction that covers only parts of the
// cache lines it touches -- the unpack's second granule, Adam's two half-lines per thread --
// then fetches those lines again, and the kernels ran 1-17% slower.)
__device__ __forceinline__ void store16(void* p, const uint4& v) {
    zs_u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, gptr(reinterpret_cast<zs_u32x4*>(p)));
}
__device__ __forceinline__ float4 load4f(const float* p) {
    const zs_f32x4 w = *gptr(reinterpret_cast<const zs_f32x4*>(p));
    return make_float4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ void store4f(float* p, const float4& v) {
    zs_f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, gptr(reinterpret_cast<zs_f32x4*>(p)));
}
__device__ __forceinline__ float4 load4f_nt(const float* p) {
    const zs_f32x4 w = __builtin_nontemporal_load(gptr(reinterpret_cast<const zs_f32x4*>(p)));
    return make_float4(w.x, w.y, w.z, w.w);
}

// Sixteen bytes from any 2-byte aligned address: one global_load_dwordx4, the memory system
// handling the misalignment (measured on MI355X: unaligned 16-byte loads of a streaming copy
// run at the aligned rate and return the bytes at the exact address).
typedef zs_u32x4 zs_u32x4_a2 __attribute__((aligned(2)));
__device__ __forceinline__ uint4 load16_any(const uint16_t* p) {
    const zs_u32x4_a2 w = *(const ZS_GLOBAL zs_u32x4_a2*)p;
    return make_uint4(w.x, w.y, w.z, w.w);
}

__device__ __forceinline__ void store16_any(uint16_t* p, const uint4& v) {
    zs_u32x4_a2 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (ZS_GLOBAL zs_u32x4_a2*)p);
}

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

__device__ __forceinline__ uint16_t elem_of(const uint4& v, int t) {
    const uint32_t w = t < 2 ? v.x : t < 4 ? v.y : t < 6 ? v.z : v.w;
    return uint16_t((t & 1) ? (w >> 16) : (w & 0xffffu));
}

__device__ __forceinline__ uint4 pack8(const uint16_t (&h)[8]) {
    return make_uint4(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16),
                      uint32_t(h[4]) | (uint32_t(h[5]) << 16), uint32_t(h[6]) | (uint32_t(h[7]) << 16));
}

// Exact 16-bit -> fp32 conversions.  DT is a zero_dtype.
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t h) {
    if constexpr (DT == ZERO_BF16) {
        return __uint_as_float(h << 16);
    } else {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
    }
}

// Convert the eight 16-bit values of v and add them, in order, into acc (or set acc).
template <int DT, bool kFirst>
__device__ __forceinline__ void accumulate8(float (&acc)[8], const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float lo = to_f32<DT>(w[t] & 0xffffu);
        const float hi = to_f32<DT>(w[t] >> 16);
        if constexpr (kFirst) {
            acc[2 * t] = lo;
            acc[2 * t + 1] = hi;
        } else {
            acc[2 * t] = acc[2 * t] + lo;
            acc[2 * t + 1] = acc[2 * t + 1] + hi;
        }
    }
}

// fp32 -> 16-bit, round to nearest even (finite inputs; NaN becomes a quiet NaN).
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float f) {
    if constexpr (DT == ZERO_BF16) {
        const uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t(((u >> 16) & 0x8000u) | 0x7fc0u);
        return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    } else {
        // The empty asm pins f as a stored fp32 value: without it the compiler folds the
        // conversion into the producing fma (a mixed-precision fma rounding the exact result
        // straight to fp16), which differs from rounding the fp32 master when that value lies
        // on an fp16 tie.
        asm volatile("" : "+v"(f));
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
    }
}

__device__ __forceinline__ bool non_finite(float f) { return (__float_as_uint(f) & 0x7f800000u) == 0x7f800000u; }

// ------------------------------------------------------------------ the Nd-way reduce --
// Eight columns of the rank rows: acc = f32(row_0), then acc = acc + f32(row_k) for
// k = 1..nd-1 (one fp32 round-to-nearest-even addition each, in this order).  The columns are
// element `lane` of row k starting at rows_u + k * row_stride, rows_u uniform across the
// wavefront (the tile's first column) and lane the thread's offset in the tile.  Every form
// adds in the same order; they differ in how many row loads a thread keeps in flight, which
// sets its registers, and the kernels pick the form that measured fastest for them on MI355X:
//   kRowsLow   row 0, then groups of kAhead rows from row 1, then one row at a time: fewest
//              registers (the ZeRO-3 layer launch, which shares its registers with the pack
//              and the unpack, and the fused reduce + Adam on whole tiles);
//   kRowsGroup groups of kAhead rows from row 0, each group's loads then its adds, the last
//              partial group loaded whole (the reduce: every tile below Nd = 16, the tiles inside
//              one parameter from Nd = 16);
//   kRowsPipe  the same groups with the next group's loads issued before the current group's
//              adds, two groups in registers (the tiles that hold several parameters, in the
//              reduce from Nd = 16 and in the fused reduce + Adam).
// NT makes the row loads nontemporal (each wave's load covers 1 KB of whole lines).
enum RowForm { kRowsLow, kRowsGroup, kRowsPipe };
constexpr int kAhead = 8;
template <int DT>
__device__ __forceinline__ void reduce_group_adds(float (&acc)[8], const uint4 (&v)[kAhead], bool first) {
    if (first) accumulate8<DT, true>(acc, v[0]);
    else accumulate8<DT, false>(acc, v[0]);
#pragma unroll
    for (int u = 1; u < kAhead; ++u) accumulate8<DT, false>(acc, v[u]);
}
template <bool NT>
__device__ __forceinline__ void reduce_group_loads(uint4 (&v)[kAhead], const uint16_t* rows_u, uint32_t lane_bytes,
                                                   int64_t k, int64_t row_stride) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) v[u] = load16_off<NT>(rows_u + (k + u) * row_stride, lane_bytes);
}
template <int DT, int FORM, bool NT = false>
__device__ __forceinline__ void reduce_rows8(const uint16_t* rows_u, uint32_t lane, int64_t nd, int64_t row_stride,
                                             float (&acc)[8]) {
    const uint32_t lb = lane * 2u;
    const int64_t ng = nd / kAhead;  // full groups
    uint4 a[kAhead];
    if constexpr (FORM == kRowsLow) {
        accumulate8<DT, true>(acc, load16_off<NT>(rows_u, lb));
        int64_t k = 1;
        for (; k + kAhead <= nd; k += kAhead) {
            reduce_group_loads<NT>(a, rows_u, lb, k, row_stride);
            reduce_group_adds<DT>(acc, a, false);
        }
        for (; k < nd; ++k) accumulate8<DT, false>(acc, load16_off<NT>(rows_u + k * row_stride, lb));
        return;
    } else if constexpr (FORM == kRowsGroup) {
        for (int64_t g = 0; g < ng; ++g) {
            reduce_group_loads<NT>(a, rows_u, lb, g * kAhead, row_stride);
            reduce_group_adds<DT>(acc, a, g == 0);
        }
    } else {
        uint4 b[kAhead];
        if (ng > 0) {
            reduce_group_loads<NT>(a, rows_u, lb, 0, row_stride);
            for (int64_t g = 0;; g += 2) {  // a holds group g, b group g + 1
                if (g + 1 < ng) reduce_group_loads<NT>(b, rows_u, lb, (g + 1) * kAhead, row_stride);
                reduce_group_adds<DT>(acc, a, g == 0);
                if (g + 1 >= ng) break;
                if (g + 2 < ng) reduce_group_loads<NT>(a, rows_u, lb, (g + 2) * kAhead, row_stride);
                reduce_group_adds<DT>(acc, b, false);
                if (g + 2 >= ng) break;
            }
        }
    }
    const int rem = int(nd - ng * kAhead);
    if (rem == 0) return;
    const int64_t k0 = ng * kAhead;
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
        if (u < rem) a[u] = load16_off<NT>(rows_u + (k0 + u) * row_stride, lb);
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        if (u >= rem) break;
        if (u == 0 && k0 == 0) accumulate8<DT, true>(acc, a[0]);
        else accumulate8<DT, false>(acc, a[u]);
    }
}

// Bit t of the result is set when column x + t belongs to a live parameter (i is the first
// parameter with end > x).
__device__ __forceinline__ unsigned live_mask8(const DevPlan& P, const uint8_t* __restrict__ live, int64_t x,
                                               int64_t i) {
    if (i < P.n && P.off[i] <= x && x + kChunk <= P.end[i]) return live[i] ? 0xffu : 0u;
    unsigned m = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t xt = x + t;
        while (i < P.n && P.end[i] <= xt) ++i;
        if (i < P.n && P.off[i] <= xt && live[i]) m |= 1u << t;
    }
    return m;
}

// True if a masked value is inf or NaN.
__device__ __forceinline__ bool any_bad8(const float (&v)[8], unsigned mask) {
    bool bad = false;
#pragma unroll
    for (int t = 0; t < 8; ++t) bad |= ((mask >> t) & 1u) && non_finite(v[t]);
    return bad;
}

// OR 1 into *flag when `bad` holds on any active lane of the wavefront: a ballot across the
// lanes, then one atomic from the lowest lane that found a value (none when nothing was found),
// skipped when a device-scope load already sees the flag set -- in a step where most waves
// find an inf, atomics on the one address from every wave would otherwise queue up behind each
// other (a stale 0 from the load only costs the atomic).  Called once per thread after its
// loops, where the wavefront has reconverged.
__device__ __forceinline__ void flag_wave(bool bad, int32_t* flag) {
    const unsigned long long m = __ballot(bad);
    if (m != 0ull && __lane_id() == unsigned(__builtin_ctzll(m)) &&
        __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
        atomicOr(flag, 1);
}

}  // namespace zs

// Host side: the opaque plan.
struct zero_plan {
    int64_t n = 0, nd = 0, rank = 0, n_buckets = 0, shard_numel = 0, shard_elems = 0;
    int64_t numel_total = 0, padded_total = 0, bucket_elems = 0, total_chunks = 0;
    int32_t dtype = 0, device = 0;
    // host copies, one row per parameter / bucket
    int64_t* h_param = nullptr;   // n * kParamFields
    int64_t* h_bucket = nullptr;  // n_buckets * kBucketFields
    int64_t* h_bucket_chunks = nullptr;  // [n_buckets][2]: the bucket's unpack chunk range [u0, u1)
    // Shard tiles of every bucket, split by kind: [n_buckets][3] = offset into d_ptiles (in
    // entries), tiles that lie inside one parameter ("whole"), then tiles holding several
    // parameters, padding or the row gap ("mixed"); d_ptiles lists each bucket's whole tiles,
    // then its mixed ones, one entry = (tile index, first parameter whose range ends after the
    // tile's first column) as two int64.
    int64_t* h_ptile = nullptr;
    int64_t* d_ptiles = nullptr;
    // device tables
    void* d_mem = nullptr;        // one allocation holding every table below
    zs::DevPlan dev{};
    int32_t* d_bfirst = nullptr;
    int32_t* d_bcount = nullptr;
    float* d_adam_scal = nullptr; // [n][2] per-parameter step size and 1/sqrt(bias correction 2)
    float* d_adam_const = nullptr;// [8] fp32 hyperparameters formed on the device
};

namespace zs {
enum ParamField { PF_NUMEL, PF_PAD, PF_PADDED, PF_SHARD, PF_START, PF_END, PF_OFFSET, PF_BUCKET, PF_COL, kParamFields };
enum BucketField { BF_FIRST, BF_COUNT, BF_ROW, BF_STRIDE, BF_BASE, kBucketFields };

// Thread-local error text and status helpers (defined in plan.hip).
zero_status fail(zero_status st, const char* fmt, ...);
zero_status check_launch(const char* what);
zero_status check_device(const zero_plan* plan);
inline bool host_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
}  // namespace zs
