// scaler.hip — the dynamic loss scaler, on the device.
//
// The pages do not treat loss scaling (the fp16 workloads need it); this is the usual dynamic
// rule: back off after a step with an overflow, grow after a run of clean steps.  Keeping the
// state in device memory lets the whole step — overflow verdict, skip, step counts, the
// gradient multiplier of the next step — run without a host round trip: the Adam prepare
// kernel reads `scale`, and this update reads the step's flag.
#include <cmath>

#include "zs_common.h"

namespace zs {

__global__ void loss_scaler_init_kernel(zero_loss_scaler cfg, zero_loss_scaler* __restrict__ s) { *s = cfg; }

// One thread.  Products in fp32 with round to nearest even; the clamps keep the scale in
// [min_scale, max_scale].
__global__ void loss_scaler_update_kernel(const int32_t* __restrict__ flag, zero_loss_scaler* __restrict__ s) {
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    zero_loss_scaler st = *s;
    if (*flag) {
        const float x = st.scale * st.backoff_factor;
        st.scale = x < st.min_scale ? st.min_scale : x;
        st.good_steps = 0;
        st.overflows += 1;
    } else {
        st.good_steps += 1;
        if (st.good_steps >= st.growth_interval) {
            const float x = st.scale * st.growth_factor;
            st.scale = x > st.max_scale ? st.max_scale : x;
            st.good_steps = 0;
        }
    }
    *s = st;
}

}  // namespace zs

using namespace zs;

static bool scaler_aligned(const void* p) { return reinterpret_cast<uintptr_t>(p) % alignof(zero_loss_scaler) == 0; }

extern "C" zero_status zero_loss_scaler_init(const zero_loss_scaler* cfg, zero_loss_scaler* d_scaler, void* stream) {
    if (!cfg || !d_scaler) return fail(ZERO_EINVAL, "zero_loss_scaler_init: NULL pointer");
    if (!scaler_aligned(d_scaler)) return fail(ZERO_EINVAL, "zero_loss_scaler_init: scaler not 4-byte aligned");
    const zero_loss_scaler c = *cfg;
    const bool ok = std::isfinite(c.scale) && std::isfinite(c.min_scale) && std::isfinite(c.max_scale) &&
                    c.min_scale > 0.0f && c.min_scale <= c.scale && c.scale <= c.max_scale &&
                    c.growth_interval >= 1 && std::isfinite(c.growth_factor) && c.growth_factor >= 1.0f &&
                    c.backoff_factor > 0.0f && c.backoff_factor <= 1.0f && c.good_steps >= 0 &&
                    c.good_steps < c.growth_interval && c.overflows >= 0;
    if (!ok) return fail(ZERO_EINVAL, "zero_loss_scaler_init: configuration out of range");
    loss_scaler_init_kernel<<<1, 1, 0, (hipStream_t)stream>>>(c, d_scaler);
    return check_launch("zero_loss_scaler_init");
}

extern "C" zero_status zero_loss_scaler_update(const int32_t* d_flag, zero_loss_scaler* d_scaler, void* stream) {
    if (!d_flag || !d_scaler) return fail(ZERO_EINVAL, "zero_loss_scaler_update: NULL pointer");
    if (!scaler_aligned(d_scaler) || reinterpret_cast<uintptr_t>(d_flag) % 4 != 0)
        return fail(ZERO_EINVAL, "zero_loss_scaler_update: pointers not 4-byte aligned");
    loss_scaler_update_kernel<<<1, 64, 0, (hipStream_t)stream>>>(d_flag, d_scaler);
    return check_launch("zero_loss_scaler_update");
}
