// zs_adam.h — the mixed-precision Adam arithmetic shared by the unfused step (adam.hip) and
// the fused reduce + Adam path (fused.hip), so that both compute bit-identical results.
//
// Textbook bias-corrected Adam without weight decay (the pages name the optimizer's fp32 copy,
// momentum and variance but give no update rule): with g = reduced gradient * grad_scale,
//   m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
//   p -= (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps).
#pragma once

#include <cmath>

#include "zs_common.h"

namespace zs {

enum AdamConst { AC_BETA1, AC_BETA2, AC_C1, AC_C2, AC_EPS, AC_GSCALE, kAdamConsts };

// One thread per parameter.  If the flag is set the step is skipped: nothing is written.
// Otherwise every live parameter's step count advances and its step size lr / (1 - beta1^t)
// and 1 / sqrt(1 - beta2^t) are formed in double and rounded to fp32 once; thread 0 also forms
// the fp32 hyperparameters (1 - beta in double, then rounded) and the gradient multiplier
// grad_scale (/ scaler->scale when a device loss scaler is given).
__global__ void adam_prepare_kernel(DevPlan P, const uint8_t* __restrict__ live, int32_t* __restrict__ steps,
                                    const int32_t* __restrict__ flag, double lr, double beta1, double beta2, double eps,
                                    double grad_scale, const zero_loss_scaler* __restrict__ scaler,
                                    float2* __restrict__ scal, float* __restrict__ consts);

struct AdamK {
    float b1, b2, c1, c2, eps, gs;
};

__device__ __forceinline__ AdamK load_adam_consts(const float* consts) {
    return AdamK{ld_const(consts, AC_BETA1), ld_const(consts, AC_BETA2), ld_const(consts, AC_C1),
                 ld_const(consts, AC_C2),    ld_const(consts, AC_EPS),   ld_const(consts, AC_GSCALE)};
}

// One element, in fp32, with every rounding spelled out (no contraction left to the compiler).
__device__ __forceinline__ void adam_elem(const AdamK& K, float g32, float& p, float& m, float& v, float step_size,
                                          float inv_sqrt_bc2) {
#pragma clang fp contract(off)
    const float g = g32 * K.gs;
    m = __builtin_fmaf(K.b1, m, K.c1 * g);
    v = __builtin_fmaf(K.b2, v, K.c2 * (g * g));
    const float denom = __builtin_fmaf(sqrtf(v), inv_sqrt_bc2, K.eps);
    p = __builtin_fmaf(-step_size, m / denom, p);
}

// Lane-strided layout of a span of columns: in pass q the block's threads take consecutive
// 4-column groups of the span's q-th kBlock * 4 columns, so that every load and store
// instruction of a wavefront covers 1 KB of fp32 (512 B of the 16-bit parameters) of whole
// cache lines.  quad_col(q) is the thread's first column in pass q, relative to the span.
__device__ __forceinline__ int64_t quad_col(int q) { return int64_t(q) * kBlock * 4 + int64_t(threadIdx.x) * 4; }

// The update of 4 consecutive columns of one parameter from g (the reduced gradient) and the
// loaded p, m, v: stores p, m, v at p32, m, v and the four new 16-bit parameters at lp.
template <int DT>
__device__ __forceinline__ void adam_quad(const AdamK& K, const float4& g, float4 p, float4 m, float4 v, float2 sc,
                                          float* p32, float* mm, float* vv, uint16_t* lp) {
    const float* gq = &g.x;
    float* pq = &p.x;
    float* mq = &m.x;
    float* vq = &v.x;
    uint16_t h[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        adam_elem(K, gq[t], pq[t], mq[t], vq[t], sc.x, sc.y);
        h[t] = from_f32<DT>(pq[t]);
    }
    store4f(p32, p);
    store4f(mm, m);
    store4f(vv, v);
    __builtin_nontemporal_store(
        uint64_t(uint32_t(h[0]) | (uint32_t(h[1]) << 16)) | (uint64_t(uint32_t(h[2]) | (uint32_t(h[3]) << 16)) << 32),
        gptr(reinterpret_cast<uint64_t*>(lp)));
}

}  // namespace zs
