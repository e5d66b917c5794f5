// fused.hip — the reduce and the Adam step of one bucket in a single pass: the reduced
// gradient never goes to memory (the g32 write and re-read, 8 of the 50 bytes per shard
// element at Nd = 8, disappear).
//
// Pages: ColossalAI issue "[zero] improving compatibility of low level zero" — BWD (zero2:
// reduce-scatter of the per-rank flats) and Optim (each rank steps its own p32 with the matching
// g, only parameters that have a gradient); upskillscore ZeRO summary — model states and the
// stage-2 bucketed reduce-scatter.
//
// Skipping a step needs the overflow verdict before any state changes, so this path takes it
// from the inputs: each rank flags its own gradients while packing them (zero_pack_bucket_check:
// a non-finite element, or one above 2^126 / Nd in magnitude), and the ranks' flags are ORed
// (an all-reduce MAX of one int).  With every input finite and below that bound, no fp32 sum of
// Nd of them can overflow, so a clear flag means every sum is finite — the same verdict the
// unfused check of the sums gives — and the sums, summed in the same order, and the Adam update,
// computed by the same code, are bit-identical to the unfused path's.
#include "zs_adam.h"

namespace zs {

template <int DT>
__global__ __launch_bounds__(kBlock) void reduce_adam_kernel(DevPlan P, int64_t b_base, int64_t b_row,
                                                             int64_t b_stride, int64_t tile0, int64_t n_tile,
                                                             const uint16_t* __restrict__ rows, int64_t row_stride,
                                                             const uint8_t* __restrict__ live, float* __restrict__ p32,
                                                             float* __restrict__ m, float* __restrict__ v,
                                                             const float2* __restrict__ scal,
                                                             const float* __restrict__ consts,
                                                             const int32_t* __restrict__ flag,
                                                             uint16_t* __restrict__ arena) {
    if (flag && *flag) return;
    __shared__ float4 g_lds[kTileCols / 4];  // the fp32 sums of a whole tile
    const AdamK K = load_adam_consts(consts);
    uint16_t* const lp_row = arena + P.nd * b_base + P.rank * b_stride;  // row r of the bucket's block
    for (int64_t w = blockIdx.x; w < n_tile; w += gridDim.x) {
        const int64_t j = tile0 + w;
        const int64_t x0 = j << kTileShift;
        // block-uniform (scalar loads): the whole tile inside one parameter?
        const int64_t iu = ld_const(P.tile_first, j);
        const int64_t ic = iu < P.n ? iu : P.n - 1;
        const int64_t off = ld_const(P.off, ic), end = ld_const(P.end, ic);
        const bool lv = ld_const(live, ic) != 0;
        const float2 sc_u = ld_const_f2(scal, ic);
        const bool whole = iu < P.n && off <= x0 && end >= x0 + kTileCols;
        if (whole) {
            if (!lv) continue;
            // A whole tile of one live parameter: the rows are summed with nontemporal loads
            // (each wave's load covers whole lines), the sums go through LDS, and Adam takes the
            // tile lane-strided as the unfused step does, its state loaded after the sum with
            // whole-line nontemporal loads.  Measured on MI355X against one thread updating the
            // 8 columns it summed, state loaded before the sum: 7-8% faster on the 7.5B, GPT-2
            // and Llama lists, 3% on the ragged one.  Loading the state before the sum, ordinary
            // row loads, or the reduce's double-buffered row groups here were each slower.
            float acc[8];
            reduce_rows8<DT, kRowsLow, true>(rows + (x0 - b_base), threadIdx.x * kChunk, P.nd, row_stride, acc);
            g_lds[2 * threadIdx.x] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            g_lds[2 * threadIdx.x + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
            float4 p4[2], m4[2], v4[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int64_t xq = x0 + quad_col(q);
                p4[q] = load4f_nt(p32 + xq);
                m4[q] = load4f_nt(m + xq);
                v4[q] = load4f_nt(v + xq);
            }
            __syncthreads();
            float4 g4[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) g4[q] = g_lds[quad_col(q) / 4];
            __syncthreads();  // the LDS is free for the block's next tile
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int64_t xq = x0 + quad_col(q);
                adam_quad<DT>(K, g4[q], p4[q], m4[q], v4[q], sc_u, p32 + xq, m + xq, v + xq,
                              lp_row + (xq - b_base));
            }
            continue;
        }
        const int64_t x = x0 + int64_t(threadIdx.x) * kChunk;
        const int64_t c = x - b_base;
        if (c < 0 || c >= b_row) continue;  // outside the bucket, or entirely in the row gap
        int64_t i = param_of_column(P, x);
        const unsigned mask = live_mask8(P, live, x, i);
        if (mask == 0) continue;
        const bool one_param = i < P.n && P.off[i] <= x && x + kChunk <= P.end[i];
        const bool vec = mask == 0xffu && one_param;
        // the other tiles: two groups of rows in flight, nontemporal row loads (2.5% faster on
        // the ragged list, where these tiles dominate; level on the model lists)
        float acc[8];
        reduce_rows8<DT, kRowsPipe, true>(rows + (x0 - b_base), threadIdx.x * kChunk, P.nd, row_stride, acc);
        if (vec) {
            // eight columns of one live parameter: two 4-column updates
            const float2 sc = scal[i];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int64_t xq = x + 4 * q;
                adam_quad<DT>(K, make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]),
                              load4f(p32 + xq), load4f(m + xq), load4f(v + xq), sc, p32 + xq, m + xq, v + xq,
                              lp_row + c + 4 * q);
            }
            continue;
        }
        // columns of several parameters, dead slots or the row gap: element by element
        ZS_GLOBAL float* gp = gptr(p32);
        ZS_GLOBAL float* gm = gptr(m);
        ZS_GLOBAL float* gv = gptr(v);
        ZS_GLOBAL uint16_t* glp = gptr(lp_row);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (!(mask & (1u << t))) continue;
            const int64_t xt = x + t;
            while (i < P.n && P.end[i] <= xt) ++i;
            const float2 sc = scal[i];
            float pe = gp[xt], me = gm[xt], ve = gv[xt];
            adam_elem(K, acc[t], pe, me, ve, sc.x, sc.y);
            gp[xt] = pe;
            gm[xt] = me;
            gv[xt] = ve;
            glp[c + t] = from_f32<DT>(pe);
        }
    }
}

zero_status launch_adam_prepare(const zero_plan* plan, const uint8_t* d_live, int32_t* d_steps,
                                const zero_adam_hparams* hp, const int32_t* d_flag, hipStream_t s, const char* who);

}  // namespace zs

using namespace zs;

extern "C" zero_status zero_reduce_adam_bucket(const zero_plan* plan, int64_t b, const void* d_rows, int64_t row_stride,
                                               const uint8_t* d_live, float* d_p32, float* d_m, float* d_v,
                                               const int32_t* d_flag, void* d_arena, void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (b < 0 || b >= plan->n_buckets)
        return fail(ZERO_EINVAL, "zero_reduce_adam_bucket: bucket %lld out of range", (long long)b);
    const int64_t* br = plan->h_bucket + b * kBucketFields;
    const int64_t base = br[BF_BASE], row = br[BF_ROW], stride = br[BF_STRIDE];
    if (row == 0) return ZERO_OK;  // empty rows: nothing to read or write, buffers may be NULL
    if (!d_rows || !d_live || !d_p32 || !d_m || !d_v || !d_arena)
        return fail(ZERO_EINVAL, "zero_reduce_adam_bucket: NULL pointer");
    if (!host_aligned16(d_rows) || !host_aligned16(d_p32) || !host_aligned16(d_m) || !host_aligned16(d_v) ||
        !host_aligned16(d_arena))
        return fail(ZERO_EINVAL, "zero_reduce_adam_bucket: rows, shard arrays and arena must be 16-byte aligned");
    if (row_stride < stride || row_stride % kChunk != 0)
        return fail(ZERO_EINVAL, "zero_reduce_adam_bucket: row_stride %lld must be >= %lld and a multiple of 8",
                    (long long)row_stride, (long long)stride);
    const int64_t tile0 = base >> kTileShift;
    const int64_t n_tile = ((base + row + kTileCols - 1) >> kTileShift) - tile0;
    const int g = grid_for(n_tile);
    hipStream_t s = (hipStream_t)stream;
    const uint16_t* rows = static_cast<const uint16_t*>(d_rows);
    const float2* scal = reinterpret_cast<const float2*>(plan->d_adam_scal);
    uint16_t* arena = static_cast<uint16_t*>(d_arena);
    if (plan->dtype == ZERO_BF16)
        reduce_adam_kernel<ZERO_BF16><<<g, kBlock, 0, s>>>(plan->dev, base, row, stride, tile0, n_tile, rows,
                                                           row_stride, d_live, d_p32, d_m, d_v, scal,
                                                           plan->d_adam_const, d_flag, arena);
    else
        reduce_adam_kernel<ZERO_FP16><<<g, kBlock, 0, s>>>(plan->dev, base, row, stride, tile0, n_tile, rows,
                                                           row_stride, d_live, d_p32, d_m, d_v, scal,
                                                           plan->d_adam_const, d_flag, arena);
    return check_launch("zero_reduce_adam_bucket");
}
