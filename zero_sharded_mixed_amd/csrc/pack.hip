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
// store is an aligned dwordx4 (rows start 16-byte aligned because L_b is a multiple of 8).  A
// chunk that lies inside one parameter reads its 8 source elements with one 16-byte load at
// whatever alignment the row has in the gradient (k * s_i + column); chunks that straddle
// parameters, padding or a row gap go element by element.  The pack's blocks follow per-bucket
// lists of whole and mixed tiles built with the plan (see pack_kernel).  The unpack is driven
// by its output too, in per-parameter chunk space.
#include <cmath>
#include <cstring>

#include "zs_pack.h"

namespace zs {

template <bool CHECK>
__global__ __launch_bounds__(kBlock) void pack_kernel(DevPlan P, int64_t b_base, int64_t b_row, int64_t b_stride,
                                                      const int64_t* __restrict__ tiles, int64_t n_whole,
                                                      int64_t n_mixed, const uint16_t* const* __restrict__ grads,
                                                      uint16_t* __restrict__ packed, uint32_t limit,
                                                      int32_t* __restrict__ flag) {
    __shared__ PackShared sh;
    pack_body<CHECK>(P, sh, b_base, b_row, b_stride, tiles, n_whole, n_mixed, grads, packed, limit, flag, blockIdx.x,
                     gridDim.x);
}

__global__ __launch_bounds__(kBlock) void unpack_kernel(DevPlan P, int64_t b_base, int64_t b_stride, int64_t u0,
                                                        int64_t u1, const uint16_t* __restrict__ gathered,
                                                        uint16_t* const* __restrict__ outs) {
    unpack_body(P, b_base, b_stride, u0, u1, gathered, outs, blockIdx.x, gridDim.x);
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

namespace zs {
zero_status pack_prepare(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs, void* d_packed,
                         int32_t* d_flag, bool check, const char* who, PackLaunch* out) {
    *out = PackLaunch{};
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "%s: bucket %lld out of range", who, (long long)b);
    const int64_t* br = bucket_row(plan, b);
    if (br[BF_STRIDE] == 0) return ZERO_OK;  // empty rows: nothing to read or write, buffers may be NULL
    if (!d_grad_ptrs || !d_packed || (check && !d_flag)) return fail(ZERO_EINVAL, "%s: NULL pointer", who);
    if (!host_aligned16(d_packed)) return fail(ZERO_EINVAL, "%s: packed buffer not 16-byte aligned", who);
    const int64_t* pt = plan->h_ptile + 3 * b;
    *out = PackLaunch{br[BF_BASE], br[BF_ROW], br[BF_STRIDE], plan->d_ptiles + 2 * pt[0], pt[1], pt[2],
                      reinterpret_cast<const uint16_t* const*>(d_grad_ptrs), static_cast<uint16_t*>(d_packed),
                      check ? check_limit_bits(plan->dtype, plan->nd) : 0u, check ? d_flag : nullptr, check,
                      pack_blocks(plan->nd, pt[1], pt[2])};
    return ZERO_OK;
}

zero_status unpack_prepare(const zero_plan* plan, int64_t b, const void* d_gathered, void* const* d_param_ptrs,
                           const char* who, UnpackLaunch* out) {
    *out = UnpackLaunch{};
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "%s: bucket %lld out of range", who, (long long)b);
    const int64_t* br = bucket_row(plan, b);
    const int64_t u0 = plan->h_bucket_chunks[2 * b], u1 = plan->h_bucket_chunks[2 * b + 1];
    if (u1 == u0) return ZERO_OK;  // only empty parameters: nothing to move, buffers may be NULL
    if (!d_gathered || !d_param_ptrs) return fail(ZERO_EINVAL, "%s: NULL pointer", who);
    if (!host_aligned16(d_gathered)) return fail(ZERO_EINVAL, "%s: gathered buffer not 16-byte aligned", who);
    *out = UnpackLaunch{br[BF_BASE], br[BF_STRIDE], u0, u1, static_cast<const uint16_t*>(d_gathered),
                        reinterpret_cast<uint16_t* const*>(d_param_ptrs), unpack_blocks(u0, u1)};
    return ZERO_OK;
}
}  // namespace zs

static zero_status pack_common(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs, void* d_packed,
                               int32_t* d_flag, bool check, void* stream, const char* who) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    PackLaunch L;
    if ((st = pack_prepare(plan, b, d_grad_ptrs, d_packed, d_flag, check, who, &L)) != ZERO_OK || L.blocks == 0)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (!check)
        pack_kernel<false><<<int(L.blocks), kBlock, 0, s>>>(plan->dev, L.b_base, L.b_row, L.b_stride, L.tiles,
                                                            L.n_whole, L.n_mixed, L.grads, L.packed, L.limit, nullptr);
    else
        pack_kernel<true><<<int(L.blocks), kBlock, 0, s>>>(plan->dev, L.b_base, L.b_row, L.b_stride, L.tiles,
                                                           L.n_whole, L.n_mixed, L.grads, L.packed, L.limit, L.flag);
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
    UnpackLaunch L;
    if ((st = unpack_prepare(plan, b, d_gathered, d_param_ptrs, "zero_unpack", &L)) != ZERO_OK || L.blocks == 0)
        return st;
    unpack_kernel<<<int(L.blocks), kBlock, 0, (hipStream_t)stream>>>(plan->dev, L.b_base, L.b_stride, L.u0, L.u1,
                                                                      L.gathered, L.outs);
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
