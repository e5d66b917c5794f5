// zs_pack.h — device code of the bucket pack and the unpack (see pack.hip): the bodies that
// a launch of their own (pack.hip) or the ZeRO-3 layer launch (z3.hip) runs over its blocks.
#pragma once

#include "zs_common.h"

namespace zs {

// ------------------------------------------------------------------------------- pack --
constexpr int kUnpackUnroll = 2;  // chunks per thread per iteration of the unpack


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

// Eight elements of one row of parameter m, starting at element e of its flat gradient:
// one unaligned 16-byte load when all eight are gradient elements, else element by element
// with +0 for the padding (e >= numel).
// Eight elements starting at element e of a 16-byte aligned buffer, from the two aligned
// granules that hold them (never a granule that holds none of the eight): the d = e mod 8
// element shift is a selection of 32-bit words by d/2 and a 2-byte funnel shift when d is odd.
__device__ __forceinline__ uint4 funnel8(const uint4& a, const uint4& b, int d) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const int h = d >> 1;
    const uint32_t sh = (d & 1) ? 2u : 0u;
    uint32_t lo[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) {  // lo[t] = w[h + t] (h in 0..3, h + t <= 7)
        const uint32_t c0 = w[t], c1 = w[t + 1 < 8 ? t + 1 : 7], c2 = w[t + 2 < 8 ? t + 2 : 7],
                       c3 = w[t + 3 < 8 ? t + 3 : 7];
        lo[t] = h == 0 ? c0 : h == 1 ? c1 : h == 2 ? c2 : c3;
    }
    return make_uint4(__builtin_amdgcn_alignbyte(lo[1], lo[0], sh), __builtin_amdgcn_alignbyte(lo[2], lo[1], sh),
                      __builtin_amdgcn_alignbyte(lo[3], lo[2], sh), __builtin_amdgcn_alignbyte(lo[4], lo[3], sh));
}
// A 16-byte nontemporal load (the address 16-byte aligned).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
    const zs_u32x4 w = __builtin_nontemporal_load(gptr(reinterpret_cast<const zs_u32x4*>(p)));
    return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ uint4 load8_two(const uint16_t* __restrict__ base, int64_t e) {
    const int64_t q = e >> 3;
    const int d = int(e & 7);
    const uint4 a = load16(base + 8 * q);
    if (d == 0) return a;
    return funnel8(a, load16(base + 8 * q + 8), d);
}
__device__ __forceinline__ uint4 row_chunk(const uint16_t* g, int64_t e, int64_t numel) {
    if (e + kChunk <= numel) return load16_any(g + e);
    const ZS_GLOBAL uint16_t* gg = gptr(g);
    uint16_t h[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = (e + t < numel) ? gg[e + t] : uint16_t(0);
    return pack8(h);
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
        const uint4 v = row_chunk(g, k * P.s[i] + (x - P.off[i]), P.numel[i]);
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

// Mixed tiles stage the parameters that overlap them in LDS (at most kStageMax; tiles touching
// more parameters go chunk by chunk through the generic path).
constexpr int kStageMax = 256;

// Work items of one bucket, in dispatch order:
//  * mixed tiles (several parameters, padding, the row gap): kMixRows rows of one tile per
//    block, tiles varying fastest, by runs (above); they come first, so that these heavier
//    blocks do not form the launch's tail;
//  * whole tiles (a tile inside one parameter): kWholeRows rows of one tile per block, tiles
//    varying fastest, so that consecutive blocks read and write consecutive 4 KB pieces of the
//    same rows.  Each block moves only kWholeRows * 4 KB behind a chain of dependent loads
//    (list entry -> parameter fields and gradient pointer -> data), so the chain is kept at that
//    length (the list entry carries the parameter) and the rows of a block share it.
// Measured on MI355X, with the nontemporal stores: tiles varying fastest are 8% faster than
// rows varying fastest on the 7.5B list (Nd = 64) and level elsewhere (with ordinary stores
// rows-fastest had been 2-20% ahead); one or four rows per block lose 3-14%; a fixed grid that
// prefetches the next item loses 10-40% against this one-block-per-item grid; 4 rows per mixed
// block are 1% slower than 8 on the ragged list, 16 rows up to 50% slower (the run's 16 loads in
// flight cost registers, hence occupancy).
// tiles: the bucket's n_whole whole tiles, then its n_mixed mixed tiles (plan tables).
constexpr int kMixRows = 8;       // rows per block of a mixed tile
static_assert(kMixRows >= 1 && kMixRows < 32, "a run's rows are a 32-bit mask");
constexpr int kWholeRows = 2;   // rows per block of a whole tile

// The fields a whole-tile work item needs: its rows, its columns' parameter and that
// parameter's gradient pointer (NULL = no gradient this step).
struct WholeItem {
    int64_t k0, x0, off, s, numel;
    const uint16_t* g;
};

__device__ __forceinline__ WholeItem whole_item(const DevPlan& P, const int64_t* __restrict__ tiles,
                                                const uint16_t* const* __restrict__ grads, int64_t w, int64_t n_wrg,
                                                int64_t n_whole) {
    // tiles vary fastest: consecutive blocks take consecutive whole tiles of one row group
    const int64_t rg = n_whole * n_wrg <= int64_t(UINT32_MAX) ? int64_t(uint32_t(w) / uint32_t(n_whole)) : w / n_whole;
    const int64_t jw = w - rg * n_whole;
    const int64_t j = ld_const(tiles, 2 * jw), i = ld_const(tiles, 2 * jw + 1);  // the tile, its parameter
    return WholeItem{rg * kWholeRows, j << kTileShift, ld_const(P.off, i), ld_const(P.s, i), ld_const(P.numel, i),
                     ld_const(grads, i)};
}

template <bool CHECK>
__device__ __forceinline__ void whole_loads(const DevPlan& P, const WholeItem& it, uint4 (&v)[kWholeRows],
                                            uint32_t limit, bool& bad) {
    const int64_t c = it.x0 + int64_t(threadIdx.x) * kChunk - it.off;
#pragma unroll
    for (int u = 0; u < kWholeRows; ++u) {
        if (it.k0 + u >= P.nd) break;
        // a row piece at a 16-byte boundary of the gradient: each wave's load covers whole
        // lines, so it is nontemporal (0.5-3.4% on the model lists; the misaligned rows, where
        // a load covers parts of its first and last lines, keep ordinary loads)
        const int64_t e = (it.k0 + u) * it.s + c;
        if (e + kChunk <= it.numel && aligned16(it.g + e)) {
            v[u] = load16_nt(it.g + e);
            if constexpr (CHECK) bad |= out_of_range8(v[u], limit);
            continue;
        }
        v[u] = row_chunk(it.g, (it.k0 + u) * it.s + c, it.numel);
        if constexpr (CHECK) bad |= out_of_range8(v[u], limit);
    }
}

__device__ __forceinline__ void whole_stores(const DevPlan& P, const WholeItem& it, const uint4 (&v)[kWholeRows],
                                             uint16_t* __restrict__ packed, int64_t b_base, int64_t b_stride) {
    uint16_t* dst = packed + (it.x0 + int64_t(threadIdx.x) * kChunk - b_base);
#pragma unroll
    for (int u = 0; u < kWholeRows; ++u) {
        if (it.k0 + u >= P.nd) break;
        store16(dst + (it.k0 + u) * b_stride, v[u]);
    }
}

// Mixed tiles, by runs.  Row k of a bucket is the concatenation of the parameters' row
// pieces, piece i being elements [k * s_i, (k + 1) * s_i) of gradient i.  A piece of s_i >= 8
// columns is cut into runs of 8 starting at the parameter's first column, the last run moved
// back to end exactly at the piece's end (it overlaps its predecessor, which writes the same
// values); each run of each row is then one 16-byte load from the gradient and one 16-byte
// store into the row, both at whatever alignment they have.  A mixed tile takes every run that
// intersects it: a run crossing into a whole tile rewrites that tile's values there, and a run
// crossing two mixed tiles is written by both, always with the same values.  Pieces shorter
// than 8 columns, runs that reach into the padding (their elements at or past numel_i are +0)
// and the row gap [S_b, L_b) (+0) go element by element.  A parameter without a gradient has
// no runs: its columns are not written.
struct MixMeta {
    int64_t off, s, numel;
    const uint16_t* g;
    int64_t mlo;    // the parameter's first run that intersects the tile
    int32_t run0;   // index of that run in the tile's list (exclusive scan of the run counts)
};

// The kMixRows rows of one run: every row's load is issued before the first store, so that a
// thread waits for memory once per run rather than once per row.
template <bool CHECK>
__device__ __forceinline__ void pack_run(const MixMeta& m, int64_t mnum, int64_t k0, int64_t k1,
                                         uint16_t* __restrict__ packed, int64_t b_base, int64_t b_stride,
                                         uint32_t limit, bool& bad) {
    const int64_t s = m.s;
    const int64_t j = (s >= kChunk && 8 * mnum + kChunk > s) ? s - kChunk : 8 * mnum;  // first element of the run
    const int len = int(s - j < kChunk ? s - j : kChunk);
    const uint16_t* __restrict__ src = m.g + j;
    const int64_t lim = m.numel - j;  // element e of the run exists iff k * s + e < lim
    uint16_t* __restrict__ dst = packed + (m.off + j - b_base);
    uint4 v[kMixRows];
    unsigned fast = 0;  // bit u: row k0 + u is one 16-byte load and store
#pragma unroll
    for (int u = 0; u < kMixRows; ++u) {
        const int64_t k = k0 + u;
        if (k < k1 && len == kChunk && k * s + kChunk <= lim) {
            v[u] = load16_any(src + k * s);
            fast |= 1u << u;
        }
    }
#pragma unroll
    for (int u = 0; u < kMixRows; ++u) {
        if (fast & (1u << u)) {
            if constexpr (CHECK) bad |= out_of_range8(v[u], limit);
            store16_any(dst + (k0 + u) * b_stride, v[u]);
        }
    }
    if (fast == (1u << (k1 - k0)) - 1u) return;
    // runs shorter than 8 or reaching into the padding: element by element, +0 past numel
    for (int64_t k = k0; k < k1; ++k) {
        if (fast & (1u << (k - k0))) continue;
        const int64_t e = k * s;
        ZS_GLOBAL uint16_t* d = gptr(dst + k * b_stride);
        uint16_t h[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            h[t] = (t < len && e + t < lim) ? gptr(src)[e + t] : uint16_t(0);
            if (t < len) d[t] = h[t];
        }
        if constexpr (CHECK) bad |= out_of_range8(pack8(h), limit);
    }
}

// One mixed-tile work item: rows [kg * kMixRows, ...) of mixed tile jm.  The parameters that
// overlap the tile are staged with their run counts; each thread takes runs r = tid, tid + 256, ...
template <bool CHECK>
__device__ __forceinline__ void pack_mixed_item(const DevPlan& P, MixMeta* sm, int32_t* s_total, int64_t b_base,
                                                int64_t b_row, int64_t b_stride, const int64_t* __restrict__ tiles,
                                                int64_t jm, int64_t kg, const uint16_t* const* __restrict__ grads,
                                                uint16_t* __restrict__ packed, uint32_t limit, bool& bad) {
    const int64_t j = ld_const(tiles, 2 * jm);
    const int64_t x0 = j << kTileShift, x1 = x0 + kTileCols;
    const int64_t k0 = kg * kMixRows, k1 = k0 + kMixRows < P.nd ? k0 + kMixRows : P.nd;
    // parameters overlapping the tile: [iu, last], last = the tile map's next entry (clamped)
    const int64_t iu = ld_const(tiles, 2 * jm + 1);
    const int64_t inext = ld_const(P.tile_first, j + 1);
    const int64_t last = inext < P.n ? inext : P.n - 1;
    const int64_t cnt = iu < P.n ? last - iu + 1 : 0;
    // the row gap of this bucket, where it falls in the tile: +0 in every row
    const int64_t gap0 = b_base + b_row, gap1 = b_base + b_stride;
    if (gap0 < gap1 && gap0 < x1 && gap1 > x0 && threadIdx.x == 0) {
        const int64_t c0 = gap0 > x0 ? gap0 : x0, c1 = gap1 < x1 ? gap1 : x1;
        for (int64_t k = k0; k < k1; ++k)
            for (int64_t c = c0; c < c1; ++c) gptr(packed)[k * b_stride + (c - b_base)] = 0;
    }
    if (cnt > kStageMax) {  // more parameters than the stage holds: chunk by chunk, unstaged
        const int64_t x = x0 + int64_t(threadIdx.x) * kChunk;
        if (x < b_base || x >= b_base + b_stride) return;
        const int64_t i = param_of_column(P, x);
        for (int64_t k = k0; k < k1; ++k)
            pack_chunk_generic<CHECK>(P, i, k, x, grads, packed + k * b_stride + (x - b_base), limit, bad);
        return;
    }
    __syncthreads();  // the previous item's readers are done with the stage
    for (int64_t t = threadIdx.x; t < cnt; t += kBlock) {
        const int64_t pi = iu + t;
        const int64_t off = P.off[pi], s = P.s[pi];
        const uint16_t* g = grads[pi];
        // run m covers columns off + a_m + [0, 8), a_m = min(8m, s - 8) (s >= 8), or the whole
        // piece (s < 8); a_m never decreases, so the runs meeting [x0, x1) are a range [lo, hi)
        const int64_t nrun = s >= kChunk ? (s + kChunk - 1) / kChunk : (s > 0 ? 1 : 0);
        const int64_t lo = off >= x0 ? 0 : (x0 - off) / kChunk;
        int64_t hi = off >= x1 ? 0 : (x1 - off + kChunk - 1) / kChunk;  // runs starting before x1 at 8m
        if (off < x1 && hi >= nrun - 1) hi = nrun;  // the last run starts at or before its nominal 8(nrun - 1)
        const bool here = g && off >= b_base && off + s <= b_base + b_row && hi > lo;
        sm[t] = MixMeta{off, s, P.numel[pi], g, lo, int32_t(here ? hi - lo : 0)};
    }
    __syncthreads();
    if (threadIdx.x == 0) {  // exclusive scan of the run counts (a handful of parameters per tile)
        int32_t acc = 0;
        for (int t = 0; t < int(cnt); ++t) {
            const int32_t nr = sm[t].run0;
            sm[t].run0 = acc;
            acc += nr;
        }
        *s_total = acc;
    }
    __syncthreads();
    const int32_t total = *s_total;
    for (int32_t r = int32_t(threadIdx.x); r < total; r += kBlock) {
        int lo = 0, hi = int(cnt) - 1;  // last staged parameter whose first run is <= r
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sm[mid].run0 <= r) lo = mid; else hi = mid - 1;
        }
        const MixMeta m = sm[lo];
        pack_run<CHECK>(m, m.mlo + (r - m.run0), k0, k1, packed, b_base, b_stride, limit, bad);
    }
}

// LDS of the pack: the staged parameters of a mixed tile and their run total.
struct PackShared {
    MixMeta sm[kStageMax];
    int32_t total;
};

// The pack of one bucket over virtual blocks vb = vbid, vbid + vgrid, ... (a launch of its own
// passes blockIdx.x and gridDim.x; the ZeRO-3 layer launch passes its share of the grid).
template <bool CHECK>
__device__ __forceinline__ void pack_body(const DevPlan& P, PackShared& sh, int64_t b_base, int64_t b_row,
                                          int64_t b_stride, const int64_t* __restrict__ tiles, int64_t n_whole,
                                          int64_t n_mixed, const uint16_t* const* __restrict__ grads,
                                          uint16_t* __restrict__ packed, uint32_t limit, int32_t* __restrict__ flag,
                                          int64_t vbid, int64_t vgrid) {
    const int64_t n_wrg = (P.nd + kWholeRows - 1) / kWholeRows;
    const int64_t n_wwork = n_whole * n_wrg;
    const int64_t n_mrg = (P.nd + kMixRows - 1) / kMixRows;
    const int64_t n_work = n_wwork + n_mixed * n_mrg;
    bool bad = false;
    // the mixed items (several rows each, heavier) first, so that they do not form the tail;
    // two loops, so that a block with whole items only sets up nothing of the mixed ones
    const int64_t n_mwork = n_work - n_wwork;
    int64_t w = vbid;
    for (; w < n_mwork; w += vgrid) {
        const int64_t kg = w / n_mixed;
        pack_mixed_item<CHECK>(P, sh.sm, &sh.total, b_base, b_row, b_stride, tiles, n_whole + (w - kg * n_mixed), kg,
                               grads, packed, limit, bad);
    }
    for (; w < n_work; w += vgrid) {
        const WholeItem it = whole_item(P, tiles, grads, w - n_mwork, n_wrg, n_whole);
        if (!it.g) continue;  // no gradient this step
        uint4 v[kWholeRows];
        whole_loads<CHECK>(P, it, v, limit, bad);
        whole_stores(P, it, v, packed, b_base, b_stride);
    }
    if constexpr (CHECK) flag_wave(bad, flag);
}

// Number of virtual blocks the pack of one bucket uses (one per work item, capped).
inline int64_t pack_blocks(int64_t nd, int64_t n_whole, int64_t n_mixed) {
    return grid_for(n_whole * ((nd + kWholeRows - 1) / kWholeRows) + n_mixed * ((nd + kMixRows - 1) / kMixRows));
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
// row is read from the aligned granules of the (16-byte aligned) gathered block that hold it
// (load8_two; measured on MI355X 1% faster here than one unaligned load, and 6% faster than
// taking the second granule from the next lane by a DPP shift); a chunk crossing into the next
// row (s >= 8) is two such reads and a merge (a crossing chunk is never in the last row, so
// both stay inside the block); the tail of a parameter and rows shorter than 8 go element by
// element.  The store is one 16-byte store whatever the output's 2-byte alignment.
__device__ __forceinline__ void unpack_chunk(int64_t u, int64_t ucb, int64_t numel, int64_t s, int64_t col,
                                             double inv_s, int64_t b_stride, const uint16_t* __restrict__ gathered,
                                             uint16_t* out) {
    const int64_t e0 = (u - ucb) * kChunk;
    // row k = e0 / s and column j0 = e0 mod s; the double estimate is off by at most one
    int64_t k = int64_t(double(e0) * inv_s);
    int64_t j0 = e0 - k * s;
    if (j0 < 0) { --k; j0 += s; } else if (j0 >= s) { ++k; j0 -= s; }
    if (e0 + kChunk <= numel) {
        if (j0 + kChunk <= s) {
            store16_any(out + e0, load8_two(gathered, k * b_stride + col + j0));
            return;
        }
        if (s >= kChunk) {
            const uint4 a = load8_two(gathered, k * b_stride + col + j0);
            const uint4 b = load8_two(gathered, (k + 1) * b_stride + col);
            store16_any(out + e0, merge_split(a, b, int(s - j0)));
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
__device__ __forceinline__ void unpack_body(const DevPlan& P, int64_t b_base, int64_t b_stride, int64_t u0, int64_t u1,
                                            const uint16_t* __restrict__ gathered, uint16_t* const* __restrict__ outs,
                                            int64_t vbid, int64_t vgrid) {
    const int64_t ut0 = u0 >> kUTileShift;
    const int64_t n_ut = ((u1 + kUTileChunks - 1) >> kUTileShift) - ut0;
    const int64_t n_groups = (n_ut + kUnpackUnroll - 1) / kUnpackUnroll;
    for (int64_t w = vbid; w < n_groups; w += vgrid) {
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
            if (s >= kSpanElems) {
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
                        store16_any(out + e0, load8_two(gathered, k * b_stride + col + j0));
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

// Number of virtual blocks the unpack of chunks [u0, u1) uses.
inline int64_t unpack_blocks(int64_t u0, int64_t u1) {
    const int64_t n_ut = ((u1 + kUTileChunks - 1) >> kUTileShift) - (u0 >> kUTileShift);
    return grid_for((n_ut + kUnpackUnroll - 1) / kUnpackUnroll);
}

// A validated pack of one bucket, ready to run: what pack_body needs, and its block count
// (0 = nothing to do).
struct PackLaunch {
    int64_t b_base, b_row, b_stride;
    const int64_t* tiles;
    int64_t n_whole, n_mixed;
    const uint16_t* const* grads;
    uint16_t* packed;
    uint32_t limit;
    int32_t* flag;
    bool check;
    int64_t blocks;
};
// The same for the unpack of one bucket.
struct UnpackLaunch {
    int64_t b_base, b_stride, u0, u1;
    const uint16_t* gathered;
    uint16_t* const* outs;
    int64_t blocks;
};
// Argument checks of zero_pack_bucket / zero_pack_bucket_check / zero_unpack (errors named after
// `who`), filling the launch record; defined in pack.hip.
zero_status pack_prepare(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs, void* d_packed,
                         int32_t* d_flag, bool check, const char* who, PackLaunch* out);
zero_status unpack_prepare(const zero_plan* plan, int64_t b, const void* d_gathered, void* const* d_param_ptrs,
                           const char* who, UnpackLaunch* out);

}  // namespace zs
