// adam.hip — the fused mixed-precision Adam step over rank r's shard, with the 16-bit write of
// the updated parameters into row r of every bucket's all-gather block.
//
// Pages: ColossalAI issue "[zero] improving compatibility of low level zero" — Optim (each rank
// steps its own p32 with the matching g; only parameters that require grad and have a
// gradient take part: the layer-drop mapping); upskillscore ZeRO summary — model states (the
// optimizer keeps an fp32 copy of the parameters, the momentum and the variance); briefia.fr
// "L'IA sur plusieurs GPU : ZeRO et FSDP" — ZeRO-1 step order (update the own partition, then
// all-gather the parameters); llm-engineer "ZeRO-3" — the ZeRO-1/2 all-gather.  The update rule
// itself is textbook bias-corrected Adam without weight decay (the pages give none).
//
// Two launches on the caller's stream.  adam_prepare_kernel (one thread per parameter) reads
// the overflow flag, bumps the step count of every live parameter and forms its step size
// lr / (1 - beta1^t) and 1 / sqrt(1 - beta2^t) in double, rounded to fp32 once; it also forms
// the fp32 hyperparameters (1 - beta computed in double, then rounded).  adam_kernel then
// streams the shard: per thread one 8-column chunk, reading g32, p32, m, v as two dwordx4
// each and writing p32, m, v and 8 16-bit parameters (one dwordx4) — 30 bytes per element.
// Both kernels return at once when the flag is set, so a skipped step changes nothing.
#include <cmath>

#include "zs_common.h"

namespace zs {

enum AdamConst { AC_BETA1, AC_BETA2, AC_C1, AC_C2, AC_EPS, AC_GSCALE, kAdamConsts };

__global__ void adam_prepare_kernel(DevPlan P, const uint8_t* __restrict__ live, int32_t* __restrict__ steps,
                                    const int32_t* __restrict__ flag, double lr, double beta1, double beta2, double eps,
                                    double grad_scale, float2* __restrict__ scal, float* __restrict__ consts) {
    if (flag && *flag) return;
    const int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (gid == 0) {
        consts[AC_BETA1] = float(beta1);
        consts[AC_BETA2] = float(beta2);
        consts[AC_C1] = float(1.0 - beta1);
        consts[AC_C2] = float(1.0 - beta2);
        consts[AC_EPS] = float(eps);
        consts[AC_GSCALE] = float(grad_scale);
    }
    for (int64_t i = gid; i < P.n; i += int64_t(gridDim.x) * blockDim.x) {
        if (!live[i]) continue;
        const int32_t t = steps[i] + 1;
        steps[i] = t;
        const double bc1 = 1.0 - pow(beta1, double(t));
        const double bc2 = 1.0 - pow(beta2, double(t));
        scal[i] = make_float2(float(lr / bc1), float(1.0 / sqrt(bc2)));
    }
}

struct AdamArgs {
    const float* g32;
    float* p32;
    float* m;
    float* v;
    const uint8_t* live;
    const float2* scal;
    const float* consts;
    const int32_t* flag;
    uint16_t* arena;
};

struct AdamK {
    float b1, b2, c1, c2, eps, gs;
};

__device__ __forceinline__ void adam_elem(const AdamK& K, float g32, float& p, float& m, float& v, float step_size,
                                          float inv_sqrt_bc2) {
    const float g = g32 * K.gs;
    m = K.b1 * m + K.c1 * g;
    v = K.b2 * v + K.c2 * (g * g);
    const float denom = sqrtf(v) * inv_sqrt_bc2 + K.eps;
    p = p - step_size * (m / denom);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void adam_kernel(DevPlan P, AdamArgs A) {
    if (A.flag && *A.flag) return;
    const AdamK K{A.consts[AC_BETA1], A.consts[AC_BETA2], A.consts[AC_C1],
                  A.consts[AC_C2],    A.consts[AC_EPS],   A.consts[AC_GSCALE]};
    for (int64_t j = blockIdx.x; j < P.n_tiles; j += gridDim.x) {
        const int64_t x = (j << kTileShift) + int64_t(threadIdx.x) * kChunk;
        if (x >= P.shard_numel) continue;
        int64_t i = param_of_column(P, x);
        if (i < P.n && P.off[i] <= x && x + kChunk <= P.end[i]) {
            // Whole chunk inside live parameter i: the wide path.
            if (!A.live[i]) continue;
            const float2 sc = A.scal[i];
            const int32_t b = P.bucket[i];
            const int64_t O = P.b_base[b];
            const float4* gv = reinterpret_cast<const float4*>(A.g32 + x);
            float4* pv = reinterpret_cast<float4*>(A.p32 + x);
            float4* mv = reinterpret_cast<float4*>(A.m + x);
            float4* vv = reinterpret_cast<float4*>(A.v + x);
            const float4 g0 = gv[0], g1 = gv[1];
            float4 p0 = pv[0], p1 = pv[1], m0 = mv[0], m1 = mv[1], v0 = vv[0], v1 = vv[1];
            float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint16_t h[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                adam_elem(K, g[t], p[t], m[t], v[t], sc.x, sc.y);
                h[t] = from_f32<DT>(p[t]);
            }
            pv[0] = make_float4(p[0], p[1], p[2], p[3]);
            pv[1] = make_float4(p[4], p[5], p[6], p[7]);
            mv[0] = make_float4(m[0], m[1], m[2], m[3]);
            mv[1] = make_float4(m[4], m[5], m[6], m[7]);
            vv[0] = make_float4(v[0], v[1], v[2], v[3]);
            vv[1] = make_float4(v[4], v[5], v[6], v[7]);
            uint16_t* dst = A.arena + P.nd * O + P.rank * P.b_stride[b] + (x - O);
            *reinterpret_cast<uint4*>(dst) = pack8(h);
        } else {
            // Chunk across parameters, dead slots or a row gap: element by element.
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int64_t xt = x + t;
                while (i < P.n && P.end[i] <= xt) ++i;
                if (!(i < P.n && P.off[i] <= xt) || !A.live[i]) continue;
                const float2 sc = A.scal[i];
                const int32_t b = P.bucket[i];
                const int64_t O = P.b_base[b];
                float p = A.p32[xt], m = A.m[xt], v = A.v[xt];
                adam_elem(K, A.g32[xt], p, m, v, sc.x, sc.y);
                A.p32[xt] = p;
                A.m[xt] = m;
                A.v[xt] = v;
                A.arena[P.nd * O + P.rank * P.b_stride[b] + (xt - O)] = from_f32<DT>(p);
            }
        }
    }
}

}  // namespace zs

using namespace zs;

extern "C" zero_status zero_adam_step(const zero_plan* plan, const float* d_g32, float* d_p32, float* d_m, float* d_v,
                                      const uint8_t* d_live, int32_t* d_steps, const zero_adam_hparams* hp,
                                      const int32_t* d_flag, void* d_arena, void* stream) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (!d_g32 || !d_p32 || !d_m || !d_v || !d_live || !d_steps || !hp || !d_arena)
        return fail(ZERO_EINVAL, "zero_adam_step: NULL pointer");
    if (!host_aligned16(d_g32) || !host_aligned16(d_p32) || !host_aligned16(d_m) || !host_aligned16(d_v) ||
        !host_aligned16(d_arena))
        return fail(ZERO_EINVAL, "zero_adam_step: shard arrays and arena must be 16-byte aligned");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->grad_scale) || !(hp->beta1 >= 0.0) ||
        !(hp->beta1 < 1.0) || !(hp->beta2 >= 0.0) || !(hp->beta2 < 1.0))
        return fail(ZERO_EINVAL, "zero_adam_step: hyperparameters out of range");
    hipStream_t s = (hipStream_t)stream;
    float2* scal = reinterpret_cast<float2*>(plan->d_adam_scal);
    adam_prepare_kernel<<<grid_for((plan->n + 255) / 256, 1024), 256, 0, s>>>(
        plan->dev, d_live, d_steps, d_flag, hp->lr, hp->beta1, hp->beta2, hp->eps, hp->grad_scale, scal,
        plan->d_adam_const);
    if ((st = check_launch("adam_prepare_kernel")) != ZERO_OK) return st;
    if (plan->shard_numel == 0) return ZERO_OK;
    AdamArgs A{d_g32, d_p32, d_m, d_v, d_live, scal, plan->d_adam_const, d_flag, static_cast<uint16_t*>(d_arena)};
    const int g = grid_for(plan->dev.n_tiles, 8192);
    if (plan->dtype == ZERO_BF16)
        adam_kernel<ZERO_BF16><<<g, kBlock, 0, s>>>(plan->dev, A);
    else
        adam_kernel<ZERO_FP16><<<g, kBlock, 0, s>>>(plan->dev, A);
    return check_launch("zero_adam_step");
}
