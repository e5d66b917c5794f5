// reduce.hip — the Nd-way shard reduce (the arithmetic of the ZeRO-2 reduce-scatter of the
// per-rank flat chunks, ColossalAI issue "[zero] improving compatibility of low level zero",
// BWD; the bucketed reduce-scatter of stage Pos+g in the upskillscore ZeRO summary) and the
// inf/NaN overflow check.
//
// Each thread owns 8 consecutive columns of the bucket row and keeps 8 fp32 accumulators.
// It reads the 16 bytes of every rank's row at those columns (aligned dwordx4: rows start on
// 16-byte boundaries), converts exactly to fp32 and adds in ascending rank order, seeded with
// rank 0's value — the fixed order that makes the sums bit-reproducible.  The rows are read
// in groups of eight with nontemporal loads, each group's loads before its adds.  Two kernels,
// chosen by Nd, measured on MI355X against each other and against two groups in flight:
//   * Nd >= 16: a tile inside one parameter keeps one group in flight and the others two (the
//     ragged list's mixed tiles: 4% faster than one), at two blocks per CU: 0.4-9% faster than
//     two groups everywhere at every Nd from 16 to 128 on the GPT-2 and 7.5B lists;
//   * Nd < 16: one group everywhere, at the occupancy its 77 registers allow (six waves per
//     SIMD): 3-4% faster at Nd = 8 on the GPT-2 and Llama lists than two groups at three waves
//     per SIMD, which were in turn 3-5% faster there than the many-row kernel.
// Columns of parameters without a gradient are skipped before any row is read.  The overflow
// flag is ORed once per wavefront (a ballot, then one atomic), only when a value is found.
#include "zs_reduce.h"

namespace zs {

// Nd from which the reduce runs its many-row kernel (below).
constexpr int64_t kBigNd = 16;

template <int DT, int WHOLE, int MIXED>
__global__ __launch_bounds__(kBlock) void reduce_kernel(DevPlan P, int64_t b_base, int64_t b_row, int64_t tile0,
                                                        int64_t n_tile, const uint16_t* __restrict__ rows,
                                                        int64_t row_stride, const uint8_t* __restrict__ live,
                                                        float* __restrict__ g32, int32_t* __restrict__ flag) {
    reduce_body<DT, WHOLE, MIXED, true>(P, b_base, b_row, tile0, n_tile, rows, row_stride, live, g32, flag, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(kBlock) void overflow_kernel(DevPlan P, const float* __restrict__ g32,
                                                          const uint8_t* __restrict__ live, int32_t* __restrict__ flag) {
    bool bad = false;
    for (int64_t j = blockIdx.x; j < P.n_tiles; j += gridDim.x) {
        const int64_t x = (j << kTileShift) + int64_t(threadIdx.x) * kChunk;
        if (x >= P.shard_numel) continue;
        const unsigned mask = live_mask8(P, live, x, param_of_column(P, x));
        if (mask == 0) continue;
        const float4 a = load4f(g32 + x);
        const float4 b = load4f(g32 + x + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        bad |= any_bad8(v, mask);
    }
    flag_wave(bad, flag);
}

}  // namespace zs

using namespace zs;

namespace zs {
zero_status reduce_prepare(const zero_plan* plan, int64_t b, const void* d_rows, int64_t row_stride,
                           const uint8_t* d_live, float* d_g32, int32_t* d_flag, const char* who, ReduceLaunch* out) {
    *out = ReduceLaunch{};
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "%s: bucket %lld out of range", who, (long long)b);
    const int64_t* br = plan->h_bucket + b * kBucketFields;
    const int64_t base = br[BF_BASE], row = br[BF_ROW], stride = br[BF_STRIDE];
    if (row == 0) return ZERO_OK;  // empty rows: nothing to read or write, buffers may be NULL
    if (!d_rows || !d_live || !d_g32) return fail(ZERO_EINVAL, "%s: NULL pointer", who);
    if (!host_aligned16(d_rows) || !host_aligned16(d_g32))
        return fail(ZERO_EINVAL, "%s: rows and g32 must be 16-byte aligned", who);
    if (row_stride < stride || row_stride % kChunk != 0)
        return fail(ZERO_EINVAL, "%s: row_stride %lld must be >= %lld and a multiple of 8", who, (long long)row_stride,
                    (long long)stride);
    const int64_t tile0 = base >> kTileShift;
    const int64_t n_tile = ((base + row + kTileCols - 1) >> kTileShift) - tile0;
    *out = ReduceLaunch{base, row, tile0, n_tile, static_cast<const uint16_t*>(d_rows), row_stride, d_live, d_g32,
                        d_flag, reduce_blocks(n_tile)};
    return ZERO_OK;
}
}  // namespace zs

extern "C" zero_status zero_reduce_shard(const zero_plan* plan, int64_t b, const void* d_rows, int64_t row_stride,
                                         const uint8_t* d_live, float* d_g32, int32_t* d_flag, void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    ReduceLaunch L;
    if ((st = reduce_prepare(plan, b, d_rows, row_stride, d_live, d_g32, d_flag, "zero_reduce_shard", &L)) != ZERO_OK ||
        L.blocks == 0)
        return st;
    hipStream_t s = (hipStream_t)stream;
    // Nd >= kBigNd: one group in flight on whole tiles, two on the others, at two blocks per CU;
    // below, one group everywhere at the occupancy the registers allow
    const bool big = plan->nd >= kBigNd;
    auto kern = plan->dtype == ZERO_BF16
                    ? (big ? reduce_kernel<ZERO_BF16, kRowsGroup, kRowsPipe> : reduce_kernel<ZERO_BF16, kRowsGroup, kRowsGroup>)
                    : (big ? reduce_kernel<ZERO_FP16, kRowsGroup, kRowsPipe> : reduce_kernel<ZERO_FP16, kRowsGroup, kRowsGroup>);
    kern<<<int(L.blocks), kBlock, big ? kTwoBlocksLds : 0u, s>>>(plan->dev, L.b_base, L.b_row, L.tile0, L.n_tile, L.rows,
                                                                  L.row_stride, L.live, L.g32, L.flag);
    return check_launch("zero_reduce_shard");
}

extern "C" zero_status zero_overflow_check(const zero_plan* plan, const float* d_g32, const uint8_t* d_live,
                                           int32_t* d_flag, void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (plan->shard_numel == 0) return ZERO_OK;  // empty shard: buffers may be NULL
    if (!d_g32 || !d_live || !d_flag) return fail(ZERO_EINVAL, "zero_overflow_check: NULL pointer");
    if (!host_aligned16(d_g32)) return fail(ZERO_EINVAL, "zero_overflow_check: g32 not 16-byte aligned");
    overflow_kernel<<<grid_for(plan->dev.n_tiles), kBlock, 0, (hipStream_t)stream>>>(plan->dev, d_g32, d_live,
                                                                                          d_flag);
    return check_launch("zero_overflow_check");
}
