// pack.hip — rank-major bucket packing, unpacking after the all-gather, and the p32 shard
// initialisation.  All three are bit moves between the per-parameter flats and the
// [Nd][L_b] bucket blocks (or rank r's fp32 shard); no arithmetic on values.
//
// Pages: ColossalAI issue "[zero] improving compatibility of low level zero" — BWD (view each
// gradient of a full bucket as [world_size, -1], gather the rows per rank, flatten each rank's
// rows into one buffer) and INIT (pad, view as [world_size, -1], clone row r as p32);
// llm-engineer "ZeRO-3" — the ZeRO-1/2 all-gather restores the full updated parameters.
//
// Work decomposition.  Both the pack and the shard init are driven by their OUTPUT, one
// 16-byte chunk (8 elements of a 16-bit block, or 8 fp32 shard columns) per thread: every
// store is an aligned dwordx4 (rows start 16-byte aligned because L_b is a multiple of 8), and
// the parameter that owns a chunk is found through the shard tile map.  A chunk that lies
// inside one parameter reads its 8 source elements with at most two aligned 16-byte loads
// and a funnel shift (load8_realigned); chunks that straddle parameters, padding or a row gap
// fall back to per-element work.  The unpack is driven by its output too, in per-parameter
// chunk space.
#include <cmath>
#include <cstring>

#include "zs_common.h"

namespace zs {

// ------------------------------------------------------------------------------- pack --
#ifndef ZS_PACK_ROWS
#define ZS_PACK_ROWS 2
#endif
#ifndef ZS_UNPACK_UNROLL
#define ZS_UNPACK_UNROLL 2
#endif
constexpr int kPackRows = ZS_PACK_ROWS;          // rows per block iteration of the pack
constexpr int kUnpackUnroll = ZS_UNPACK_UNROLL;  // chunks per thread per iteration of the unpack

// The input check of the checked pack: true if one of the eight 16-bit values is inf or NaN
// or larger in magnitude than 2^126 / Nd (below it no fp32 sum of Nd values overflows).  For
// bf16 and fp16 alike, finite magnitudes order as their bit patterns with the sign cleared, and
// every inf or NaN pattern lies above every finite one, so the test is one unsigned compare
// per value against `limit`: the largest magnitude pattern whose value v has v * Nd <= 2^126
// exactly (check_limit_bits on the host).
__device__ __forceinline__ bool out_of_range8(const uint4& v, uint32_t limit) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    bool bad = false;
#pragma unroll
    for (int t = 0; t < 4; ++t) bad |= ((w[t] & 0x7fffu) > limit) | (((w[t] >> 16) & 0x7fffu) > limit);
    return bad;
}

// Generic per-thread pack of one 8-column chunk of row k (parameter boundaries, padding,
// row gaps, dead parameters, unaligned sources).  i is the first parameter with end > x.
template <bool CHECK>
__device__ __forceinline__ void pack_chunk_generic(const DevPlan& P, int64_t i, int64_t k, int64_t x,
                                                   const uint16_t* const* __restrict__ grads, uint16_t* dst,
                                                   uint32_t limit, bool& bad) {
    if (i < P.n && P.off[i] <= x && x + kChunk <= P.end[i]) {
        const uint16_t* g = grads[i];
        if (!g) return;  // no gradient this step: leave the slots alone
        const int64_t numel = P.numel[i];
        const int64_t e0 = k * P.s[i] + (x - P.off[i]);
        uint4 v;
        if (e0 + kChunk <= numel && aligned16(g)) {
            v = load8_realigned(g, e0);
        } else {
            const ZS_GLOBAL uint16_t* gg = gptr(g);
            uint16_t h[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) h[t] = (e0 + t < numel) ? gg[e0 + t] : uint16_t(0);
            v = pack8(h);
        }
        if constexpr (CHECK) bad |= out_of_range8(v, limit);
        store16(dst, v);
        return;
    }
    uint16_t h[8];
    unsigned keep = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t xt = x + t;
        while (i < P.n && P.end[i] <= xt) ++i;
        h[t] = 0;
        if (i < P.n && P.off[i] <= xt) {
            const uint16_t* g = grads[i];
            if (!g) continue;
            const int64_t e = k * P.s[i] + (xt - P.off[i]);
            if (e < P.numel[i]) h[t] = gptr(g)[e];
        }
        keep |= 1u << t;
    }
    if constexpr (CHECK) bad |= out_of_range8(pack8(h), limit);
    if (keep == 0xffu) {
        store16(dst, pack8(h));
    } else {
        ZS_GLOBAL uint16_t* d = gptr(dst);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            if (keep & (1u << t)) d[t] = h[t];
    }
}

// Tiles holding several parameters: the block stages the fields of every parameter that
// overlaps the tile in LDS once, and each thread finds its chunk's parameter there (a binary
// search in LDS instead of dependent global loads).  Tiles touching more than kStageMax
// parameters use the unstaged generic path.
#ifndef ZS_STAGE_MAX
#define ZS_STAGE_MAX 256
#endif
constexpr int kStageMax = ZS_STAGE_MAX;
struct PackMeta {
    int64_t off, end, s, numel;
    const uint16_t* g;
};

// First staged index t in [0, cnt] with sm[t].end > x.
__device__ __forceinline__ int staged_search(const PackMeta* sm, int cnt, int64_t x) {
    int lo = 0, hi = cnt;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sm[mid].end > x) hi = mid; else lo = mid + 1;
    }
    return lo;
}

template <bool CHECK>
__device__ __forceinline__ void pack_chunk_staged(const PackMeta* sm, int cnt, int t0, int64_t k, int64_t x,
                                                  uint16_t* dst, uint32_t limit, bool& bad) {
    if (t0 < cnt && sm[t0].off <= x && x + kChunk <= sm[t0].end) {
        const PackMeta& m = sm[t0];
        if (!m.g) return;  // no gradient this step
        const int64_t e0 = k * m.s + (x - m.off);
        uint4 v;
        if (e0 + kChunk <= m.numel && aligned16(m.g)) {
            v = load8_realigned(m.g, e0);
        } else {
            const ZS_GLOBAL uint16_t* gg = gptr(m.g);
            uint16_t h[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) h[t] = (e0 + t < m.numel) ? gg[e0 + t] : uint16_t(0);
            v = pack8(h);
        }
        if constexpr (CHECK) bad |= out_of_range8(v, limit);
        store16(dst, v);
        return;
    }
    uint16_t h[8];
    unsigned keep = 0;
    int i = t0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t xt = x + t;
        while (i < cnt && sm[i].end <= xt) ++i;
        h[t] = 0;
        if (i < cnt && sm[i].off <= xt) {
            const uint16_t* g = sm[i].g;
            if (!g) continue;
            const int64_t e = k * sm[i].s + (xt - sm[i].off);
            if (e < sm[i].numel) h[t] = gptr(g)[e];
        }
        keep |= 1u << t;
    }
    if constexpr (CHECK) bad |= out_of_range8(pack8(h), limit);
    if (keep == 0xffu) {
        store16(dst, pack8(h));
    } else {
        ZS_GLOBAL uint16_t* d = gptr(dst);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            if (keep & (1u << t)) d[t] = h[t];
    }
}

// Work item w = (tile, group of kPackRows rows) of the bucket, rows varying fastest (on MI355X
// this dispatch order streams faster than tile-fastest).  When the whole tile lies inside one
// parameter with a 16-byte aligned gradient (decided once per block from scalar loads), each
// thread issues the loads of its rows before any store.
// CHECK: also OR 1 into *flag when a gradient element is non-finite or above `limit`.
template <bool CHECK>
__global__ __launch_bounds__(kBlock) void pack_kernel(DevPlan P, int64_t b_base, int64_t b_stride, int64_t tile0,
                                                      int64_t n_tile, int64_t n_rg,
                                                      const uint16_t* const* __restrict__ grads,
                                                      uint16_t* __restrict__ packed, uint32_t limit,
                                                      int32_t* __restrict__ flag) {
    __shared__ PackMeta sm[kStageMax];
    const int64_t n_work = n_tile * n_rg;
    bool bad = false;
    for (int64_t w = blockIdx.x; w < n_work; w += gridDim.x) {
        int64_t jt;
        if (n_work <= int64_t(UINT32_MAX)) jt = int64_t(uint32_t(w) / uint32_t(n_rg));  // 32-bit divide
        else jt = w / n_rg;
        const int64_t k0 = (w - jt * n_rg) * kPackRows;
        const int64_t kend = k0 + kPackRows < P.nd ? k0 + kPackRows : P.nd;
        const int64_t j = tile0 + jt;
        const int64_t x0 = j << kTileShift;
        const int64_t x = x0 + int64_t(threadIdx.x) * kChunk;
        // The tile's parameter fields, read once per block (scalar loads; index clamped into
        // range): the dependent chain is tile map -> fields and pointer -> data.
        const int64_t iu = ld_const(P.tile_first, j);
        const int64_t ic = iu < P.n ? iu : P.n - 1;
        const int64_t off = ld_const(P.off, ic), end = ld_const(P.end, ic);
        const int64_t s = ld_const(P.s, ic), numel = ld_const(P.numel, ic);
        const uint16_t* g = ld_const(grads, ic);
        const bool whole = iu < P.n && off <= x0 && end >= x0 + kTileCols;
        if (whole && !g) continue;  // the whole tile belongs to a parameter without a gradient
        if (whole && aligned16(g)) {
            const int64_t c = x - off;
            const bool direct = ((s | off) & 7) == 0;  // every source chunk 16-byte aligned
            uint16_t* dst = packed + (x - b_base);
            uint4 v[kPackRows];
#pragma unroll
            for (int u = 0; u < kPackRows; ++u) {
                const int64_t k = k0 + u;
                if (k >= kend) break;
                const int64_t e0 = k * s + c;
                if (e0 + kChunk <= numel) {
                    v[u] = direct ? load16(g + e0) : load8_realigned(g, e0);
                } else {
                    const ZS_GLOBAL uint16_t* gg = gptr(g);
                    uint16_t h[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) h[t] = (e0 + t < numel) ? gg[e0 + t] : uint16_t(0);
                    v[u] = pack8(h);
                }
                if constexpr (CHECK) bad |= out_of_range8(v[u], limit);
            }
#pragma unroll
            for (int u = 0; u < kPackRows; ++u) {
                const int64_t k = k0 + u;
                if (k >= kend) break;
                store16(dst + k * b_stride, v[u]);
            }
            continue;
        }
        // parameters overlapping the tile: [iu, last], last = the tile map's next entry (clamped)
        const int64_t inext = ld_const(P.tile_first, j + 1);
        const int64_t last = inext < P.n ? inext : P.n - 1;
        const int64_t cnt = iu < P.n ? last - iu + 1 : 0;
        if (cnt <= kStageMax) {
            __syncthreads();  // the previous iteration's readers are done with the stage
            for (int64_t t = threadIdx.x; t < cnt; t += kBlock) {
                const int64_t pi = iu + t;
                sm[t] = PackMeta{P.off[pi], P.end[pi], P.s[pi], P.numel[pi], grads[pi]};
            }
            __syncthreads();
            if (x < b_base || x >= b_base + b_stride) continue;
            const int t0 = staged_search(sm, int(cnt), x);
            for (int64_t k = k0; k < kend; ++k)
                pack_chunk_staged<CHECK>(sm, int(cnt), t0, k, x, packed + k * b_stride + (x - b_base), limit, bad);
            continue;
        }
        if (x < b_base || x >= b_base + b_stride) continue;
        const int64_t i = param_of_column(P, x);
        for (int64_t k = k0; k < kend; ++k)
            pack_chunk_generic<CHECK>(P, i, k, x, grads, packed + k * b_stride + (x - b_base), limit, bad);
    }
    if constexpr (CHECK) flag_wave(bad, flag);
}

// ----------------------------------------------------------------------------- unpack --
// Elements 0..split-1 of a followed by elements 0..7-split of b.
__device__ __forceinline__ uint4 merge_split(const uint4& a, const uint4& b, int split) {
    uint16_t h[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = t < split ? elem_of(a, t) : elem_of(b, (t - split) & 7);
    return pack8(h);
}

// One chunk of parameter fields (numel, s, column of the slice in the rows, 1/s, chunk base).
// Element e0..e0+7 of the parameter: row k = e0 / s, column j0 = e0 mod s.  A chunk inside one
// row is one realigned load; a chunk crossing into the next row (s >= 8) is two realigned
// loads and a merge (a crossing chunk is never in the last row, so both loads stay inside
// the block); the tail of a parameter and rows shorter than 8 go element by element.
__device__ __forceinline__ void unpack_chunk(int64_t u, int64_t ucb, int64_t numel, int64_t s, int64_t col,
                                             double inv_s, int64_t b_stride, const uint16_t* __restrict__ gathered,
                                             uint16_t* out) {
    const int64_t e0 = (u - ucb) * kChunk;
    // row k = e0 / s and column j0 = e0 mod s; the double estimate is off by at most one
    int64_t k = int64_t(double(e0) * inv_s);
    int64_t j0 = e0 - k * s;
    if (j0 < 0) { --k; j0 += s; } else if (j0 >= s) { ++k; j0 -= s; }
    if (e0 + kChunk <= numel && aligned16(out)) {
        if (j0 + kChunk <= s) {
            store16(out + e0, load8_realigned(gathered, k * b_stride + col + j0));
            return;
        }
        if (s >= kChunk) {
            const uint4 a = load8_realigned(gathered, k * b_stride + col + j0);
            const uint4 b = load8_realigned(gathered, (k + 1) * b_stride + col);
            store16(out + e0, merge_split(a, b, int(s - j0)));
            return;
        }
    }
    const int cnt = int(numel - e0 < kChunk ? numel - e0 : kChunk);
    ZS_GLOBAL uint16_t* o = gptr(out);
    const ZS_GLOBAL uint16_t* gsrc = gptr(gathered);
    for (int t = 0; t < cnt; ++t) {
        o[e0 + t] = gsrc[k * b_stride + col + j0];
        if (++j0 == s) { j0 = 0; ++k; }
    }
}

// One block iteration covers kUnpackUnroll consecutive chunk tiles (256 chunks each); a
// thread takes one chunk of each.  Chunks of the bucket's parameters are [u0, u1).  A group
// inside one parameter reads that parameter's fields once (scalar loads); otherwise each thread
// finds its chunk's parameter in the chunk tile map.  The kernel uses no LDS: staging the
// parameter fields of mixed groups in LDS, as the pack does, made every block carry a 14 KB
// allocation and cost 4-7% on whole lists (most groups are whole), more than it saved.
__global__ __launch_bounds__(kBlock) void unpack_kernel(DevPlan P, int64_t b_base, int64_t b_stride, int64_t u0,
                                                        int64_t u1, const uint16_t* __restrict__ gathered,
                                                        uint16_t* const* __restrict__ outs) {
    const int64_t ut0 = u0 >> kUTileShift;
    const int64_t n_ut = ((u1 + kUTileChunks - 1) >> kUTileShift) - ut0;
    const int64_t n_groups = (n_ut + kUnpackUnroll - 1) / kUnpackUnroll;
    for (int64_t w = blockIdx.x; w < n_groups; w += gridDim.x) {
        const int64_t ut = ut0 + w * kUnpackUnroll;
        const int64_t ua = ut << kUTileShift;
        const int64_t ub = ua + kUnpackUnroll * kUTileChunks;
        // parameter fields read once per block (scalar loads; index clamped into range)
        const int64_t iu = ld_const(P.utile_first, ut);
        const int64_t ic = iu < P.n ? iu : P.n - 1;
        const int64_t ucb = ld_const(P.ucb, ic), ucend = ld_const(P.ucend, ic);
        const int64_t numel = ld_const(P.numel, ic), s = ld_const(P.s, ic);
        const int64_t col = ld_const(P.off, ic) - b_base;
        const double inv_s = ld_const(P.inv_s, ic);
        uint16_t* const out = ld_const(outs, ic);
        const bool whole = ua >= u0 && ub <= u1 && iu < P.n && ucb <= ua && ucend >= ub;
        if (whole) {
            if (!out) continue;  // every chunk of the group belongs to a skipped parameter
            // Rows at least as long as the group: find the group's first row once per block;
            // each thread's chunk is then in that row or the next.
            constexpr int64_t kSpanElems = kUnpackUnroll * kUTileChunks * kChunk;
            if (s >= kSpanElems && aligned16(out)) {
                const int64_t es = (ua - ucb) * kChunk;
                int64_t ks = int64_t(double(es) * inv_s);
                int64_t js = es - ks * s;
                if (js < 0) { --ks; js += s; } else if (js >= s) { ++ks; js -= s; }
#pragma unroll
                for (int t = 0; t < kUnpackUnroll; ++t) {
                    const int64_t d = (int64_t(t) * kUTileChunks + threadIdx.x) * kChunk;
                    const int64_t e0 = es + d;
                    int64_t j0 = js + d, k = ks;
                    if (j0 >= s) { j0 -= s; ++k; }
                    if (e0 + kChunk <= numel && j0 + kChunk <= s)
                        store16(out + e0, load8_realigned(gathered, k * b_stride + col + j0));
                    else
                        unpack_chunk(ua + t * kUTileChunks + threadIdx.x, ucb, numel, s, col, inv_s, b_stride,
                                     gathered, out);
                }
                continue;
            }
#pragma unroll
            for (int t = 0; t < kUnpackUnroll; ++t)
                unpack_chunk(ua + t * kUTileChunks + threadIdx.x, ucb, numel, s, col, inv_s, b_stride, gathered, out);
            continue;
        }
        // a group of several parameters: each thread finds its chunk's parameter
#pragma unroll
        for (int t = 0; t < kUnpackUnroll; ++t) {
            const int64_t u = ua + t * kUTileChunks + threadIdx.x;
            if (u < u0 || u >= u1) continue;
            const int64_t i = param_of_chunk(P, u);
            uint16_t* o = outs[i];
            if (o) unpack_chunk(u, P.ucb[i], P.numel[i], P.s[i], P.off[i] - b_base, P.inv_s[i], b_stride, gathered, o);
        }
    }
}

// ------------------------------------------------------------------------- shard init --
// p32[off_i + j] = row r of the zero-padded master i; gaps zero; NULL masters skipped.
template <int SRC>  // 0 = fp32 source, else a zero_dtype
__global__ __launch_bounds__(kBlock) void shard_init_kernel(DevPlan P, const void* const* __restrict__ masters,
                                                            float* __restrict__ p32) {
    for (int64_t j = blockIdx.x; j < P.n_tiles; j += gridDim.x) {
        const int64_t x = (j << kTileShift) + int64_t(threadIdx.x) * kChunk;
        if (x >= P.shard_numel) continue;
        int64_t i = param_of_column(P, x);
        float vals[8];
        unsigned keep = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t xt = x + t;
            while (i < P.n && P.end[i] <= xt) ++i;
            vals[t] = 0.0f;
            if (i < P.n && P.off[i] <= xt) {
                const void* src = masters[i];
                if (!src) continue;
                const int64_t e = P.rank * P.s[i] + (xt - P.off[i]);
                if (e < P.numel[i]) {
                    if constexpr (SRC == 0) vals[t] = gptr(static_cast<const float*>(src))[e];
                    else vals[t] = to_f32<SRC>(gptr(static_cast<const uint16_t*>(src))[e]);
                }
            }
            keep |= 1u << t;
        }
        float* dst = p32 + x;
        if (keep == 0xffu) {
            store4f(dst, make_float4(vals[0], vals[1], vals[2], vals[3]));
            store4f(dst + 4, make_float4(vals[4], vals[5], vals[6], vals[7]));
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                if (keep & (1u << t)) gptr(dst)[t] = vals[t];
        }
    }
}

}  // namespace zs

using namespace zs;

static const int64_t* bucket_row(const zero_plan* plan, int64_t b) { return plan->h_bucket + b * kBucketFields; }

// Value of a 16-bit pattern with the sign cleared (exact in double).
static double half_bits_value(int dtype, uint32_t b) {
    if (dtype == ZERO_BF16) {
        const uint32_t w = b << 16;
        float f;
        std::memcpy(&f, &w, sizeof f);
        return double(f);
    }
    const int e = int((b >> 10) & 31u), m = int(b & 1023u);
    return e == 0 ? std::ldexp(double(m), -24) : std::ldexp(double(1024 + m), e - 25);
}

// The checked pack's threshold: the largest finite magnitude pattern b with value(b) * nd <=
// 2^126, the product exact in double (at most 11 significant bits times nd < 2^31).  Values
// grow with b, so a binary search finds it; for fp16 it is the largest finite pattern.
static uint32_t check_limit_bits(int dtype, int64_t nd) {
    const double bound = std::ldexp(1.0, 126);
    uint32_t lo = 0, hi = dtype == ZERO_BF16 ? 0x7f7fu : 0x7bffu;  // largest finite magnitudes
    if (half_bits_value(dtype, hi) * double(nd) <= bound) return hi;
    while (lo + 1 < hi) {  // value(lo) * nd <= bound < value(hi) * nd
        const uint32_t mid = (lo + hi) / 2;
        if (half_bits_value(dtype, mid) * double(nd) <= bound) lo = mid; else hi = mid;
    }
    return lo;
}

static zero_status pack_common(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs, void* d_packed,
                               int32_t* d_flag, bool check, void* stream, const char* who) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "%s: bucket %lld out of range", who, (long long)b);
    const int64_t* br = bucket_row(plan, b);
    const int64_t base = br[BF_BASE], stride = br[BF_STRIDE];
    if (stride == 0) return ZERO_OK;  // empty rows: nothing to read or write, buffers may be NULL
    if (!d_grad_ptrs || !d_packed || (check && !d_flag)) return fail(ZERO_EINVAL, "%s: NULL pointer", who);
    if (!host_aligned16(d_packed)) return fail(ZERO_EINVAL, "%s: packed buffer not 16-byte aligned", who);
    const int64_t tile0 = base >> kTileShift;
    const int64_t n_tile = ((base + stride + kTileCols - 1) >> kTileShift) - tile0;
    const int64_t n_rg = (plan->nd + kPackRows - 1) / kPackRows;
    const int g = grid_for(n_tile * n_rg);
    hipStream_t s = (hipStream_t)stream;
    const uint16_t* const* grads = reinterpret_cast<const uint16_t* const*>(d_grad_ptrs);
    uint16_t* packed = static_cast<uint16_t*>(d_packed);
    const uint32_t limit = check ? check_limit_bits(plan->dtype, plan->nd) : 0u;
    if (!check)
        pack_kernel<false><<<g, kBlock, 0, s>>>(plan->dev, base, stride, tile0, n_tile, n_rg, grads, packed, limit,
                                                nullptr);
    else
        pack_kernel<true><<<g, kBlock, 0, s>>>(plan->dev, base, stride, tile0, n_tile, n_rg, grads, packed, limit,
                                               d_flag);
    return check_launch(who);
}

extern "C" zero_status zero_pack_bucket(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs, void* d_packed,
                                        void* stream) {
    return pack_common(plan, b, d_grad_ptrs, d_packed, nullptr, false, stream, "zero_pack_bucket");
}

extern "C" zero_status zero_pack_bucket_check(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs,
                                              void* d_packed, int32_t* d_flag, void* stream) {
    return pack_common(plan, b, d_grad_ptrs, d_packed, d_flag, true, stream, "zero_pack_bucket_check");
}

extern "C" zero_status zero_unpack(const zero_plan* plan, int64_t b, const void* d_gathered, void* const* d_param_ptrs,
                                   void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "zero_unpack: bucket %lld out of range", (long long)b);
    const int64_t* br = bucket_row(plan, b);
    const int64_t u0 = plan->h_bucket_chunks[2 * b], u1 = plan->h_bucket_chunks[2 * b + 1];
    if (u1 == u0) return ZERO_OK;  // only empty parameters: nothing to move, buffers may be NULL
    if (!d_gathered || !d_param_ptrs) return fail(ZERO_EINVAL, "zero_unpack: NULL pointer");
    if (!host_aligned16(d_gathered)) return fail(ZERO_EINVAL, "zero_unpack: gathered buffer not 16-byte aligned");
    const int64_t n_ut = ((u1 + kUTileChunks - 1) >> kUTileShift) - (u0 >> kUTileShift);
    unpack_kernel<<<grid_for((n_ut + kUnpackUnroll - 1) / kUnpackUnroll), kBlock, 0, (hipStream_t)stream>>>(
        plan->dev, br[BF_BASE], br[BF_STRIDE], u0, u1, static_cast<const uint16_t*>(d_gathered),
        reinterpret_cast<uint16_t* const*>(d_param_ptrs));
    return check_launch("zero_unpack");
}

extern "C" zero_status zero_shard_init(const zero_plan* plan, const void* const* d_src_ptrs, int32_t src_dtype,
                                       float* d_p32, void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (src_dtype != 0 && src_dtype != ZERO_BF16 && src_dtype != ZERO_FP16)
        return fail(ZERO_EINVAL, "zero_shard_init: bad src_dtype %d", src_dtype);
    if (plan->shard_numel == 0) return ZERO_OK;  // empty shard: buffers may be NULL
    if (!d_src_ptrs || !d_p32) return fail(ZERO_EINVAL, "zero_shard_init: NULL pointer");
    if (!host_aligned16(d_p32)) return fail(ZERO_EINVAL, "zero_shard_init: p32 not 16-byte aligned");
    const int g = grid_for(plan->dev.n_tiles);
    hipStream_t s = (hipStream_t)stream;
    switch (src_dtype) {
        case 0: shard_init_kernel<0><<<g, kBlock, 0, s>>>(plan->dev, d_src_ptrs, d_p32); break;
        case ZERO_BF16: shard_init_kernel<ZERO_BF16><<<g, kBlock, 0, s>>>(plan->dev, d_src_ptrs, d_p32); break;
        case ZERO_FP16: shard_init_kernel<ZERO_FP16><<<g, kBlock, 0, s>>>(plan->dev, d_src_ptrs, d_p32); break;
        default: return fail(ZERO_EINVAL, "zero_shard_init: bad src_dtype %d", src_dtype);
    }
    return check_launch("zero_shard_init");
}
