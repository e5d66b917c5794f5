// z3.hip — ZeRO-3's per-layer traffic in one launch: the reduce-scatter arithmetic of one layer,
// the pack of another layer's gradients and the all-gather unpack of a third layer's
// parameters, each on its own share of the grid.
//
// Pages: llm-engineer card "ZeRO-3" (every layer's parameters are gathered before it runs and
// freed after; in the backward pass each layer's gradients are reduce-scattered as soon as its
// backward has run, and the layers go L-1, ..., 0); ColossalAI issue "[zero] improving
// compatibility of low level zero", BWD (pack rank-major, reduce-scatter).
//
// Why: with one bucket per layer, a step issues three short kernels per layer, and each loses
// a few microseconds to its ramp-up and its last wave.  The three parts of a backward step are
// independent when they concern different layers -- reduce(l + 1) reads rows packed one step
// earlier, pack(l) reads the gradients layer l's backward just produced, gather(l - 1) reads the
// all-gather block and fills the parameter scratch that layer l no longer needs -- so they can
// share one launch and one tail.
#include "zs_pack.h"
#include "zs_reduce.h"

namespace zs {

// Blocks [0, R.blocks) reduce, the next K.blocks pack, the last U.blocks unpack.  The reduce
// goes first: its blocks read Nd rows each and run longest.
template <int DT, bool CHECK>
__global__ __launch_bounds__(kBlock) void z3_layer_kernel(DevPlan P, ReduceLaunch R, PackLaunch K, UnpackLaunch U) {
    __shared__ PackShared sh;
    int64_t b = blockIdx.x;
    if (b < R.blocks) {
        reduce_body<DT>(P, R.b_base, R.b_row, R.tile0, R.n_tile, R.rows, R.row_stride, R.live, R.g32, R.flag, b,
                        R.blocks);
        return;
    }
    b -= R.blocks;
    if (b < K.blocks) {
        pack_body<CHECK>(P, sh, K.b_base, K.b_row, K.b_stride, K.tiles, K.n_whole, K.n_mixed, K.grads, K.packed,
                         K.limit, K.flag, b, K.blocks);
        return;
    }
    b -= K.blocks;
    unpack_body(P, U.b_base, U.b_stride, U.u0, U.u1, U.gathered, U.outs, b, U.blocks);
}

template <int DT>
static void launch_z3(const zero_plan* plan, const ReduceLaunch& R, const PackLaunch& K, const UnpackLaunch& U,
                      int g, hipStream_t s) {
    if (K.check)
        z3_layer_kernel<DT, true><<<g, kBlock, 0, s>>>(plan->dev, R, K, U);
    else
        z3_layer_kernel<DT, false><<<g, kBlock, 0, s>>>(plan->dev, R, K, U);
}

}  // namespace zs

using namespace zs;

extern "C" zero_status zero_z3_layer_step(const zero_plan* plan, int64_t reduce_b, const void* d_rows,
                                          int64_t row_stride, const uint8_t* d_live, float* d_g32, int64_t pack_b,
                                          const void* const* d_grad_ptrs, void* d_packed, int32_t check,
                                          int64_t gather_b, const void* d_gathered, void* const* d_param_ptrs,
                                          int32_t* d_flag, void* stream) {
    const char* who = "zero_z3_layer_step";
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (reduce_b < -1 || pack_b < -1 || gather_b < -1)
        return fail(ZERO_EINVAL, "%s: a bucket index below -1", who);
    ReduceLaunch R{};
    PackLaunch K{};
    UnpackLaunch U{};
    if (reduce_b >= 0 &&
        (st = reduce_prepare(plan, reduce_b, d_rows, row_stride, d_live, d_g32, d_flag, who, &R)) != ZERO_OK)
        return st;
    if (pack_b >= 0 && (st = pack_prepare(plan, pack_b, d_grad_ptrs, d_packed, d_flag, check != 0, who, &K)) != ZERO_OK)
        return st;
    if (gather_b >= 0 && (st = unpack_prepare(plan, gather_b, d_gathered, d_param_ptrs, who, &U)) != ZERO_OK)
        return st;
    int64_t total = R.blocks + K.blocks + U.blocks;
    if (total == 0) return ZERO_OK;
    if (total > int64_t(ZS_GRID_CAP)) {  // the parts loop over their work: shrink their shares to fit one launch
        for (int64_t* nb : {&R.blocks, &K.blocks, &U.blocks})
            if (*nb > 0) *nb = *nb * (int64_t(ZS_GRID_CAP) / 4) / total + 1;
        total = R.blocks + K.blocks + U.blocks;
    }
    hipStream_t s = (hipStream_t)stream;
    if (plan->dtype == ZERO_BF16)
        launch_z3<ZERO_BF16>(plan, R, K, U, int(total), s);
    else
        launch_z3<ZERO_FP16>(plan, R, K, U, int(total), s);
    return check_launch(who);
}
