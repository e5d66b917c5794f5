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
#include "zs_common.h"

namespace zs {

// ------------------------------------------------------------------------------- pack --
// Block w of the grid-stride loop handles tile (w mod n_tile) of row (w / n_tile) of the
// bucket; one thread per 8-column chunk.
__global__ __launch_bounds__(kBlock) void pack_kernel(DevPlan P, int64_t b_base, int64_t b_stride, int64_t tile0,
                                                      int64_t n_tile, const uint16_t* const* __restrict__ grads,
                                                      uint16_t* __restrict__ packed) {
    const int64_t n_work = n_tile * P.nd;
    for (int64_t w = blockIdx.x; w < n_work; w += gridDim.x) {
        const int64_t k = w / n_tile;
        const int64_t j = tile0 + (w - k * n_tile);
        const int64_t x = (j << kTileShift) + int64_t(threadIdx.x) * kChunk;  // shard column
        if (x < b_base || x >= b_base + b_stride) continue;
        uint16_t* dst = packed + k * b_stride + (x - b_base);
        int64_t i = param_of_column(P, x);
        if (i < P.n && P.off[i] <= x && x + kChunk <= P.end[i]) {
            // Chunk inside parameter i.
            const uint16_t* g = grads[i];
            if (!g) continue;  // no gradient this step: leave the slots alone
            const int64_t numel = P.numel[i];
            const int64_t e0 = k * P.s[i] + (x - P.off[i]);
            uint4 v;
            if (e0 + kChunk <= numel && aligned16(g)) {
                v = load8_realigned(g, e0);
            } else {
                uint16_t h[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) h[t] = (e0 + t < numel) ? g[e0 + t] : uint16_t(0);
                v = pack8(h);
            }
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            // Chunk across parameter boundaries, padding or the row gap: element by element.
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
                    if (e < P.numel[i]) h[t] = g[e];
                }
                keep |= 1u << t;
            }
            if (keep == 0xffu) {
                *reinterpret_cast<uint4*>(dst) = pack8(h);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (keep & (1u << t)) dst[t] = h[t];
            }
        }
    }
}

// ----------------------------------------------------------------------------- unpack --
// One thread per 8-element chunk of a parameter's flat; chunks of the bucket's parameters
// are numbered [u0, u1) in the plan's chunk space.
__global__ __launch_bounds__(kBlock) void unpack_kernel(DevPlan P, int64_t b_base, int64_t b_stride, int64_t u0,
                                                        int64_t u1, const uint16_t* __restrict__ gathered,
                                                        uint16_t* const* __restrict__ outs) {
    const int64_t ut0 = u0 >> kUTileShift;
    const int64_t n_tiles = ((u1 + kUTileChunks - 1) >> kUTileShift) - ut0;
    for (int64_t w = blockIdx.x; w < n_tiles; w += gridDim.x) {
        const int64_t u = ((ut0 + w) << kUTileShift) + threadIdx.x;
        if (u < u0 || u >= u1) continue;
        const int64_t i = param_of_chunk(P, u);
        uint16_t* out = outs[i];
        if (!out) continue;
        const int64_t numel = P.numel[i], s = P.s[i];
        const int64_t col = P.off[i] - b_base;
        const int64_t e0 = (u - P.ucb[i]) * kChunk;
        // row k = e0 / s and column j0 = e0 mod s; the double estimate is off by at most one
        int64_t k = int64_t(double(e0) * P.inv_s[i]);
        int64_t j0 = e0 - k * s;
        if (j0 < 0) { --k; j0 += s; } else if (j0 >= s) { ++k; j0 -= s; }
        if (e0 + kChunk <= numel && j0 + kChunk <= s && aligned16(out)) {
            *reinterpret_cast<uint4*>(out + e0) = load8_realigned(gathered, k * b_stride + col + j0);
        } else {
            const int cnt = int(numel - e0 < kChunk ? numel - e0 : kChunk);
            for (int t = 0; t < cnt; ++t) {
                out[e0 + t] = gathered[k * b_stride + col + j0];
                if (++j0 == s) { j0 = 0; ++k; }
            }
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
                    if constexpr (SRC == 0) vals[t] = static_cast<const float*>(src)[e];
                    else vals[t] = to_f32<SRC>(static_cast<const uint16_t*>(src)[e]);
                }
            }
            keep |= 1u << t;
        }
        float* dst = p32 + x;
        if (keep == 0xffu) {
            reinterpret_cast<float4*>(dst)[0] = make_float4(vals[0], vals[1], vals[2], vals[3]);
            reinterpret_cast<float4*>(dst)[1] = make_float4(vals[4], vals[5], vals[6], vals[7]);
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                if (keep & (1u << t)) dst[t] = vals[t];
        }
    }
}

}  // namespace zs

using namespace zs;

static const int64_t* bucket_row(const zero_plan* plan, int64_t b) { return plan->h_bucket + b * kBucketFields; }

extern "C" zero_status zero_pack_bucket(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs, void* d_packed,
                                        void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "zero_pack_bucket: bucket %lld out of range", (long long)b);
    if (!d_grad_ptrs || !d_packed) return fail(ZERO_EINVAL, "zero_pack_bucket: NULL pointer");
    if (!host_aligned16(d_packed)) return fail(ZERO_EINVAL, "zero_pack_bucket: packed buffer not 16-byte aligned");
    const int64_t* br = bucket_row(plan, b);
    const int64_t base = br[BF_BASE], stride = br[BF_STRIDE];
    if (stride == 0) return ZERO_OK;
    const int64_t tile0 = base >> kTileShift;
    const int64_t n_tile = ((base + stride + kTileCols - 1) >> kTileShift) - tile0;
    pack_kernel<<<grid_for(n_tile * plan->nd, 8192), kBlock, 0, (hipStream_t)stream>>>(
        plan->dev, base, stride, tile0, n_tile, reinterpret_cast<const uint16_t* const*>(d_grad_ptrs),
        static_cast<uint16_t*>(d_packed));
    return check_launch("zero_pack_bucket");
}

extern "C" zero_status zero_unpack(const zero_plan* plan, int64_t b, const void* d_gathered, void* const* d_param_ptrs,
                                   void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "zero_unpack: bucket %lld out of range", (long long)b);
    if (!d_gathered || !d_param_ptrs) return fail(ZERO_EINVAL, "zero_unpack: NULL pointer");
    if (!host_aligned16(d_gathered)) return fail(ZERO_EINVAL, "zero_unpack: gathered buffer not 16-byte aligned");
    const int64_t* br = bucket_row(plan, b);
    const int64_t u0 = plan->h_bucket_chunks[2 * b], u1 = plan->h_bucket_chunks[2 * b + 1];
    if (u1 == u0) return ZERO_OK;
    const int64_t n_tiles = ((u1 + kUTileChunks - 1) >> kUTileShift) - (u0 >> kUTileShift);
    unpack_kernel<<<grid_for(n_tiles, 8192), kBlock, 0, (hipStream_t)stream>>>(
        plan->dev, br[BF_BASE], br[BF_STRIDE], u0, u1, static_cast<const uint16_t*>(d_gathered),
        reinterpret_cast<uint16_t* const*>(d_param_ptrs));
    return check_launch("zero_unpack");
}

extern "C" zero_status zero_shard_init(const zero_plan* plan, const void* const* d_src_ptrs, int32_t src_dtype,
                                       float* d_p32, void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (!d_src_ptrs || !d_p32) return fail(ZERO_EINVAL, "zero_shard_init: NULL pointer");
    if (!host_aligned16(d_p32)) return fail(ZERO_EINVAL, "zero_shard_init: p32 not 16-byte aligned");
    if (plan->shard_numel == 0) return ZERO_OK;
    const int g = grid_for(plan->dev.n_tiles, 8192);
    hipStream_t s = (hipStream_t)stream;
    switch (src_dtype) {
        case 0: shard_init_kernel<0><<<g, kBlock, 0, s>>>(plan->dev, d_src_ptrs, d_p32); break;
        case ZERO_BF16: shard_init_kernel<ZERO_BF16><<<g, kBlock, 0, s>>>(plan->dev, d_src_ptrs, d_p32); break;
        case ZERO_FP16: shard_init_kernel<ZERO_FP16><<<g, kBlock, 0, s>>>(plan->dev, d_src_ptrs, d_p32); break;
        default: return fail(ZERO_EINVAL, "zero_shard_init: bad src_dtype %d", src_dtype);
    }
    return check_launch("zero_shard_init");
}
