// z3.hip — ZeRO-3's per-layer traffic in one launch: the reduce-scatter arithmetic of some
// layers, the pack of other layers' gradients and the all-gather unpack of a third set of
// layers' parameters, each bucket on its own share of the grid.
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
// share one launch and one tail; so can the parts of several consecutive layers.
#include "zs_pack.h"
#include "zs_reduce.h"

namespace zs {

// The buckets of one launch, up to K of each kind, in grid order: the reduces (their blocks
// read Nd rows each and run longest, so they go first), the packs, the unpacks; a part with
// blocks == 0 is absent.  K is a template parameter so that every part's record sits at a fixed
// place in the kernel arguments: measured on MI355X, selecting the part through a run-time
// index into the arguments costs 1-3% of a ZeRO-3 backward step.
template <int K>
struct Z3Parts {
    ReduceLaunch r[K];
    PackLaunch k[K];
    UnpackLaunch u[K];
};

// KINDS: the kinds of parts compiled in (1 reduce, 2 pack, 4 unpack): a launch of gathers
// only (the forward pass) then carries neither the reduce's nor the pack's registers.
template <int DT, bool CHECK, int K, int KINDS>
__global__ __launch_bounds__(kBlock) void z3_kernel(DevPlan P, Z3Parts<K> Z) {
    int64_t b = blockIdx.x;
    if constexpr ((KINDS & 1) != 0) {
#pragma unroll
        for (int p = 0; p < K; ++p) {
            const ReduceLaunch& R = Z.r[p];
            if (b < R.blocks) {
                reduce_body<DT, kRowsLow, kRowsLow, false>(P, R.b_base, R.b_row, R.tile0, R.n_tile, R.rows, R.row_stride, R.live,
                                              R.g32, R.flag, b, R.blocks);
                return;
            }
            b -= R.blocks;
        }
    }
    if constexpr ((KINDS & 2) != 0) {
        __shared__ PackShared sh;
#pragma unroll
        for (int p = 0; p < K; ++p) {
            const PackLaunch& L = Z.k[p];
            if (b < L.blocks) {
                pack_body<CHECK>(P, sh, L.b_base, L.b_row, L.b_stride, L.tiles, L.n_whole, L.n_mixed, L.grads,
                                 L.packed, L.limit, L.flag, b, L.blocks);
                return;
            }
            b -= L.blocks;
        }
    }
#pragma unroll
    for (int p = 0; p < K; ++p) {
        const UnpackLaunch& U = Z.u[p];
        if (b < U.blocks) {
            unpack_body(P, U.b_base, U.b_stride, U.u0, U.u1, U.gathered, U.outs, b, U.blocks);
            return;
        }
        b -= U.blocks;
    }
}

template <int K>
static void launch_z3(const zero_plan* plan, const ReduceLaunch* R, const PackLaunch* L, const UnpackLaunch* U,
                      bool check, int grid, hipStream_t s) {
    Z3Parts<K> Z{};  // absent parts: blocks == 0
    bool gathers_only = true;
    for (int p = 0; p < K; ++p) {
        Z.r[p] = R[p], Z.k[p] = L[p], Z.u[p] = U[p];
        gathers_only &= R[p].blocks == 0 && L[p].blocks == 0;
    }
    if (gathers_only) {  // the unpack body alone (a 16-bit copy: the data type does not matter)
        z3_kernel<ZERO_BF16, false, K, 4><<<grid, kBlock, 0, s>>>(plan->dev, Z);
    } else if (plan->dtype == ZERO_BF16) {
        if (check) z3_kernel<ZERO_BF16, true, K, 7><<<grid, kBlock, 0, s>>>(plan->dev, Z);
        else z3_kernel<ZERO_BF16, false, K, 7><<<grid, kBlock, 0, s>>>(plan->dev, Z);
    } else {
        if (check) z3_kernel<ZERO_FP16, true, K, 7><<<grid, kBlock, 0, s>>>(plan->dev, Z);
        else z3_kernel<ZERO_FP16, false, K, 7><<<grid, kBlock, 0, s>>>(plan->dev, Z);
    }
}

// Validate every piece of *z (errors named after `who`) and launch them together.
static zero_status z3_launch(const zero_plan* plan, const zero_z3_pieces* z, void* stream, const char* who) {
    zero_status st = check_device(plan);
    if (st != ZERO_OK) return st;
    if (!z) return fail(ZERO_EINVAL, "%s: NULL pieces", who);
    const int64_t ns[3] = {z->reduce_n, z->pack_n, z->gather_n};
    const int64_t b0s[3] = {z->reduce_b0, z->pack_b0, z->gather_b0};
    for (int t = 0; t < 3; ++t) {
        if (ns[t] < 0 || ns[t] > ZERO_Z3_MAX_BUCKETS)
            return fail(ZERO_EINVAL, "%s: %lld buckets in one piece, 0 .. %d allowed", who, (long long)ns[t],
                        ZERO_Z3_MAX_BUCKETS);
        if (ns[t] > 0 && (b0s[t] < 0 || b0s[t] + ns[t] > plan->n_buckets))
            return fail(ZERO_EINVAL, "%s: buckets [%lld, %lld) outside [0, %lld)", who, (long long)b0s[t],
                        (long long)(b0s[t] + ns[t]), (long long)plan->n_buckets);
    }
    ReduceLaunch R[ZERO_Z3_MAX_BUCKETS]{};
    PackLaunch L[ZERO_Z3_MAX_BUCKETS]{};
    UnpackLaunch U[ZERO_Z3_MAX_BUCKETS]{};
    for (int64_t j = 0; j < z->reduce_n; ++j)
        if ((st = reduce_prepare(plan, z->reduce_b0 + j, z->rows[j], z->row_stride[j], z->live, z->g32, z->flag, who,
                                 &R[j])) != ZERO_OK)
            return st;
    for (int64_t j = 0; j < z->pack_n; ++j)
        if ((st = pack_prepare(plan, z->pack_b0 + j, z->grad_ptrs, z->packed[j], z->flag, z->check != 0, who, &L[j])) !=
            ZERO_OK)
            return st;
    for (int64_t j = 0; j < z->gather_n; ++j)
        if ((st = unpack_prepare(plan, z->gather_b0 + j, z->gathered[j], z->param_ptrs, who, &U[j])) != ZERO_OK)
            return st;
    int64_t total = 0;
    for (int p = 0; p < ZERO_Z3_MAX_BUCKETS; ++p) total += R[p].blocks + L[p].blocks + U[p].blocks;
    if (total == 0) return ZERO_OK;
    if (total > int64_t(ZS_GRID_CAP)) {  // every part loops over its work: shrink the shares to fit one launch
        const int64_t all = total;
        total = 0;
        for (int p = 0; p < ZERO_Z3_MAX_BUCKETS; ++p)
            for (int64_t* nb : {&R[p].blocks, &L[p].blocks, &U[p].blocks})
                if (*nb > 0) total += (*nb = *nb * (int64_t(ZS_GRID_CAP) / 2) / all + 1);
    }
    const int64_t most = z->reduce_n > z->pack_n ? (z->reduce_n > z->gather_n ? z->reduce_n : z->gather_n)
                                                 : (z->pack_n > z->gather_n ? z->pack_n : z->gather_n);
    const bool check = z->pack_n > 0 && z->check != 0;
    hipStream_t s = (hipStream_t)stream;
    const int g = int(total);
    if (most <= 1) launch_z3<1>(plan, R, L, U, check, g, s);
    else if (most == 2) launch_z3<2>(plan, R, L, U, check, g, s);
    else launch_z3<ZERO_Z3_MAX_BUCKETS>(plan, R, L, U, check, g, s);
    return check_launch(who);
}

}  // namespace zs

using namespace zs;

extern "C" zero_status zero_z3_step(const zero_plan* plan, const zero_z3_pieces* pieces, void* stream) {
    return z3_launch(plan, pieces, stream, "zero_z3_step");
}

extern "C" zero_status zero_z3_layer_step(const zero_plan* plan, int64_t reduce_b, const void* d_rows,
                                          int64_t row_stride, const uint8_t* d_live, float* d_g32, int64_t pack_b,
                                          const void* const* d_grad_ptrs, void* d_packed, int32_t check,
                                          int64_t gather_b, const void* d_gathered, void* const* d_param_ptrs,
                                          int32_t* d_flag, void* stream) {
    const char* who = "zero_z3_layer_step";
    if (reduce_b < -1 || pack_b < -1 || gather_b < -1) {
        const zero_status st = check_device(plan);
        return st != ZERO_OK ? st : fail(ZERO_EINVAL, "%s: a bucket index below -1", who);
    }
    zero_z3_pieces z{};
    z.reduce_b0 = reduce_b, z.reduce_n = reduce_b >= 0, z.rows[0] = d_rows, z.row_stride[0] = row_stride;
    z.live = d_live, z.g32 = d_g32;
    z.pack_b0 = pack_b, z.pack_n = pack_b >= 0, z.grad_ptrs = d_grad_ptrs, z.packed[0] = d_packed, z.check = check;
    z.gather_b0 = gather_b, z.gather_n = gather_b >= 0, z.gathered[0] = d_gathered, z.param_ptrs = d_param_ptrs;
    z.flag = d_flag;
    return z3_launch(plan, &z, stream, who);
}
