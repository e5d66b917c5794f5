// zs_reduce.h — device code of the Nd-way shard reduce (see reduce.hip): the body that a
// launch of its own (reduce.hip) or the ZeRO-3 layer launch (z3.hip) runs over its blocks.
#pragma once

#include "zs_common.h"

namespace zs {

// x: the thread's first column; rows_u: the rows at the tile's first column (uniform)
template <int DT, int FORM, bool NT>
__device__ __forceinline__ void reduce_chunk(const DevPlan& P, int64_t x, unsigned mask, const uint16_t* rows_u,
                                             int64_t row_stride, float* __restrict__ g32, bool& bad) {
    float acc[8];
    reduce_rows8<DT, FORM, NT>(rows_u, threadIdx.x * kChunk, P.nd, row_stride, acc);
    float* dst = g32 + x;
    if (mask == 0xffu) {
        store4f(dst, make_float4(acc[0], acc[1], acc[2], acc[3]));
        store4f(dst + 4, make_float4(acc[4], acc[5], acc[6], acc[7]));
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            if (mask & (1u << t)) gptr(dst)[t] = acc[t];
    }
    bad |= any_bad8(acc, mask);
}

// WHOLE, MIXED: the row forms of reduce_rows8 for tiles inside one parameter and for the other
// tiles; NT: nontemporal row loads (a launch of its own uses them, the ZeRO-3 layer launch not).
template <int DT, int WHOLE, int MIXED, bool NT>
__device__ __forceinline__ void reduce_body(const DevPlan& P, int64_t b_base, int64_t b_row, int64_t tile0,
                                            int64_t n_tile, const uint16_t* __restrict__ rows, int64_t row_stride,
                                            const uint8_t* __restrict__ live, float* __restrict__ g32,
                                            int32_t* __restrict__ flag, int64_t vbid, int64_t vgrid) {
    bool bad = false;
    for (int64_t w = vbid; w < n_tile; w += vgrid) {
        const int64_t j = tile0 + w;
        const int64_t x0 = j << kTileShift;
        // block-uniform (scalar loads): does the tile lie inside one parameter, hence inside
        // this bucket, and is that parameter live?
        const int64_t iu = ld_const(P.tile_first, j);
        const int64_t ic = iu < P.n ? iu : P.n - 1;
        const int64_t off = ld_const(P.off, ic), end = ld_const(P.end, ic);
        const bool lv = ld_const(live, ic) != 0;
        const bool whole = iu < P.n && off <= x0 && end >= x0 + kTileCols;
        if (whole && !lv) continue;
        const int64_t x = x0 + int64_t(threadIdx.x) * kChunk;
        const int64_t c = x - b_base;
        if (!whole && (c < 0 || c >= b_row)) continue;  // outside the bucket, or entirely in the row gap
        const unsigned mask = whole ? 0xffu : live_mask8(P, live, x, param_of_column(P, x));
        if (mask == 0) continue;
        const uint16_t* rows_u = rows + (x0 - b_base);
        if constexpr (WHOLE == MIXED) reduce_chunk<DT, WHOLE, NT>(P, x, mask, rows_u, row_stride, g32, bad);
        else if (whole) reduce_chunk<DT, WHOLE, NT>(P, x, mask, rows_u, row_stride, g32, bad);
        else reduce_chunk<DT, MIXED, NT>(P, x, mask, rows_u, row_stride, g32, bad);
    }
    if (flag) flag_wave(bad, flag);
}

// Number of virtual blocks the reduce of n_tile tiles uses (one per tile, up to the grid cap).
inline int64_t reduce_blocks(int64_t n_tile) { return grid_for(n_tile); }

// A validated reduce of one bucket, ready to run, and its block count (0 = nothing to do).
struct ReduceLaunch {
    int64_t b_base, b_row, tile0, n_tile;
    const uint16_t* rows;
    int64_t row_stride;
    const uint8_t* live;
    float* g32;
    int32_t* flag;
    int64_t blocks;
};
// Argument checks of zero_reduce_shard (errors named after `who`); defined in reduce.hip.
zero_status reduce_prepare(const zero_plan* plan, int64_t b, const void* d_rows, int64_t row_stride,
                           const uint8_t* d_live, float* d_g32, int32_t* d_flag, const char* who, ReduceLaunch* out);

}  // namespace zs
