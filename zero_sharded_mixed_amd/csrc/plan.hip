// plan.hip — the shard planner: per-parameter padding and shard tables, the bucket walk,
// the row/shard placement and the tile maps the hot kernels search, all computed on the
// device, then copied back so the host can answer info queries.
//
// Follows briefia.fr "L'IA sur plusieurs GPU : ZeRO et FSDP" (Implémentation simplifiée: zero
// padding to a multiple of the world size, the shard size, start and end of every rank's row)
// and the ColossalAI
// issue "[zero] improving compatibility of low level zero" (INIT: split every parameter evenly
// over world_size; BWD: gradients gathered into buckets, flattened per rank).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "zs_common.h"

namespace zs {

static thread_local char g_err[512] = "";

zero_status fail(zero_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

zero_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

zero_status check_device(const zero_plan* plan) {
    if (!plan) return fail(ZERO_EINVAL, "plan is NULL");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ZERO_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev != plan->device) return fail(ZERO_EINVAL, "plan lives on device %d but device %d is current", plan->device, dev);
    return ZERO_OK;
}

// ------------------------------------------------------------------- planner kernels --

struct PlanScratch {
    int64_t* numel;
    int64_t* pad;
    int64_t* padded;
    int64_t* s;
    int64_t* start;
    int64_t* sh_end;
    int64_t* off;
    int64_t* end;
    int64_t* col;
    int64_t* dense;   // exclusive scan of s over the whole list
    int64_t* pp;      // inclusive scan of padded
    int64_t* uc;      // ceil(numel / 8)
    int64_t* ucb;     // exclusive scan of uc
    int64_t* ucend;
    double* inv_s;
    int32_t* bucket;
    int32_t* bfirst;
    int32_t* bcount;
    int64_t* b_row;
    int64_t* b_stride;
    int64_t* b_base;
    int64_t* totals;  // [0] n_buckets [1] shard_numel [2] sum s [3] sum padded [4] total chunks [5] sum numel
};

// Per-parameter closed forms (one thread per parameter).
__global__ void plan_fields_kernel(PlanScratch T, const int64_t* __restrict__ numels, int64_t n, int64_t nd,
                                   int64_t rank) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        // Nd full rows: a row is the quotient of numel by Nd, one longer when a remainder
        // is left; the zeros the rows hold beyond numel are the padding.
        const int64_t numel = numels[i];
        const int64_t q = numel / nd;
        const bool partial = q * nd != numel;
        const int64_t s = partial ? q + 1 : q;
        T.numel[i] = numel;
        T.s[i] = s;
        T.padded[i] = s * nd;
        T.pad[i] = s * nd - numel;
        T.start[i] = rank * s;
        T.sh_end[i] = (rank + 1) * s;
        T.uc[i] = (numel + kChunk - 1) / kChunk;
    }
}

// One block: running scans of s (exclusive), padded (inclusive) and uc (exclusive) over the
// whole list, 1024 parameters at a time through LDS, carrying the totals between chunks.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void plan_scan_kernel(PlanScratch T, int64_t n) {
    __shared__ int64_t sa[kScanThreads], sb[kScanThreads], sc[kScanThreads];
    const int tid = threadIdx.x;
    int64_t ca = 0, cb = 0, cc = 0;
    for (int64_t base = 0; base < n; base += kScanThreads) {
        const int64_t i = base + tid;
        const int64_t a = i < n ? T.s[i] : 0, b = i < n ? T.padded[i] : 0, c = i < n ? T.uc[i] : 0;
        sa[tid] = a;
        sb[tid] = b;
        sc[tid] = c;
        __syncthreads();
        for (int d = 1; d < kScanThreads; d <<= 1) {  // Hillis-Steele inclusive scan
            int64_t xa = 0, xb = 0, xc = 0;
            if (tid >= d) {
                xa = sa[tid - d];
                xb = sb[tid - d];
                xc = sc[tid - d];
            }
            __syncthreads();
            sa[tid] += xa;
            sb[tid] += xb;
            sc[tid] += xc;
            __syncthreads();
        }
        if (i < n) {
            T.dense[i] = ca + sa[tid] - a;
            T.pp[i] = cb + sb[tid];
            T.ucb[i] = cc + sc[tid] - c;
        }
        ca += sa[kScanThreads - 1];
        cb += sb[kScanThreads - 1];
        cc += sc[kScanThreads - 1];
        __syncthreads();
    }
    if (tid == 0) {
        T.totals[2] = ca;
        T.totals[3] = cb;
        T.totals[4] = cc;
    }
}

// One thread: walk the list into buckets.  A bucket starting at i0 takes the longest run
// i0..i1 that stays inside i0's group (i1 <= gend[i0], the last index of that group) and whose
// padded total fits the capacity (found by binary search over the inclusive scan), and at
// least i0 itself.  capacity < 0 means unbounded.
__global__ void plan_buckets_kernel(PlanScratch T, const int64_t* __restrict__ gend, int64_t n, int64_t capacity) {
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    int64_t i0 = 0, nb = 0, base = 0;
    const int64_t total_s = T.totals[2];
    while (i0 < n) {
        int64_t i1;
        const int64_t last = gend[i0];
        if (capacity < 0) {
            i1 = last;
        } else {
            const int64_t prev = i0 > 0 ? T.pp[i0 - 1] : 0;
            int64_t lo = i0, hi = last + 1;  // first i in [i0, last] with pp[i] - prev > capacity
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (T.pp[mid] - prev > capacity) hi = mid; else lo = mid + 1;
            }
            i1 = lo == i0 ? i0 : lo - 1;
        }
        const int64_t row = (i1 + 1 < n ? T.dense[i1 + 1] : total_s) - T.dense[i0];
        const int64_t stride = (row + kChunk - 1) / kChunk * kChunk;
        T.bfirst[nb] = int32_t(i0);
        T.bcount[nb] = int32_t(i1 - i0 + 1);
        T.b_row[nb] = row;
        T.b_stride[nb] = stride;
        T.b_base[nb] = base;
        base += stride;
        ++nb;
        i0 = i1 + 1;
    }
    T.totals[0] = nb;
    T.totals[1] = base;
}

// Per parameter: its bucket, its column in the bucket rows and its shard range.
__global__ void plan_place_kernel(PlanScratch T, int64_t n) {
    const int64_t nb = T.totals[0];
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        int64_t lo = 0, hi = nb - 1;  // last bucket whose first parameter is <= i
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (T.bfirst[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int64_t s = T.s[i];
        const int64_t col = T.dense[i] - T.dense[T.bfirst[lo]];
        T.bucket[i] = int32_t(lo);
        T.col[i] = col;
        T.off[i] = T.b_base[lo] + col;
        T.end[i] = T.b_base[lo] + col + s;
        T.inv_s[i] = s > 0 ? 1.0 / double(s) : 0.0;
        T.ucend[i] = T.ucb[i] + T.uc[i];
    }
}

// tile_first[j] = first i with key[i] > (j << shift), n if none; j in [0, n_tiles].
__global__ void plan_tile_map_kernel(const int64_t* __restrict__ key, int64_t n, int shift, int32_t* __restrict__ out,
                                     int64_t n_entries) {
    for (int64_t j = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; j < n_entries;
         j += int64_t(gridDim.x) * blockDim.x) {
        out[j] = int32_t(first_greater(key, 0, n, j << shift));
    }
}

}  // namespace zs

using namespace zs;

// --------------------------------------------------------------------- host entry points --

namespace {

zero_status hip_fail(const char* what, hipError_t e) {
    return fail(e == hipErrorOutOfMemory ? ZERO_ENOMEM : ZERO_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define ZS_HIP(call, what)                                   \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) { st = hip_fail(what, e_); goto done; } \
    } while (0)

}  // namespace

extern "C" void zero_plan_destroy(zero_plan* plan) {
    if (!plan) return;
    if (plan->d_mem) (void)hipFree(plan->d_mem);
    free(plan->h_param);
    free(plan->h_bucket);
    free(plan->h_bucket_chunks);
    free(plan->h_ptile);
    delete plan;
}

extern "C" zero_status zero_plan_create_grouped(const int64_t* numels, const int32_t* groups, int64_t n_params,
                                                int32_t nd, int32_t rank, int64_t bucket_bytes, int32_t dtype,
                                                zero_plan** out) {
    if (!out) return fail(ZERO_EINVAL, "zero_plan_create: out is NULL");
    *out = nullptr;
    if (!numels) return fail(ZERO_EINVAL, "zero_plan_create: numels is NULL");
    if (n_params < 1 || n_params > INT32_MAX / 2) return fail(ZERO_EINVAL, "zero_plan_create: n_params %lld out of range", (long long)n_params);
    if (nd < 1 || nd > kMaxNd) return fail(ZERO_EINVAL, "zero_plan_create: nd %d outside [1, %d]", nd, kMaxNd);
    if (rank < 0 || rank >= nd) return fail(ZERO_EINVAL, "zero_plan_create: rank %d outside [0, %d)", rank, nd);
    if (bucket_bytes < 0) return fail(ZERO_EINVAL, "zero_plan_create: bucket_bytes < 0");
    if (dtype != ZERO_BF16 && dtype != ZERO_FP16) return fail(ZERO_EINVAL, "zero_plan_create: bad dtype %d", dtype);
    // Size validation: every parameter below 2^48 elements and the padded total below 2^62
    // (bounded here by sum(numel) + n * (nd - 1), which is never smaller than it).
    {
        int64_t bound = 0;
        for (int64_t i = 0; i < n_params; ++i) {
            if (numels[i] < 0) return fail(ZERO_EINVAL, "zero_plan_create: numel[%lld] < 0", (long long)i);
            if (numels[i] >= kMaxNumel) return fail(ZERO_ERANGE, "zero_plan_create: numel[%lld] >= 2^48", (long long)i);
            bound += numels[i] + (nd - 1);
            if (bound >= (int64_t(1) << 62)) return fail(ZERO_ERANGE, "zero_plan_create: padded total exceeds 2^62");
        }
    }

    zero_status st = ZERO_OK;
    zero_plan* P = new (std::nothrow) zero_plan();
    if (!P) return fail(ZERO_ENOMEM, "zero_plan_create: host allocation");
    const int64_t n = n_params;
    P->n = n;
    P->nd = nd;
    P->rank = rank;
    P->dtype = dtype;
    P->bucket_elems = bucket_bytes / 2;

    PlanScratch T{};
    int64_t totals[6] = {0, 0, 0, 0, 0, 0};
    int64_t* d_numels_in = nullptr;
    std::vector<int64_t> tmp;
    {
        // Layout of the single device allocation.  Tables the hot kernels read come first;
        // the planner's scratch (scans, inputs) is not kept apart since it is small.
        const int64_t n8 = (n + 1);
        size_t bytes = 0;
        auto take = [&](size_t sz) { size_t o = bytes; bytes += (sz + 255) / 256 * 256; return o; };
        const size_t o_numel = take(8 * n8), o_pad = take(8 * n8), o_padded = take(8 * n8), o_s = take(8 * n8),
                     o_start = take(8 * n8), o_shend = take(8 * n8), o_off = take(8 * n8), o_end = take(8 * n8),
                     o_col = take(8 * n8), o_dense = take(8 * n8), o_pp = take(8 * n8), o_uc = take(8 * n8),
                     o_ucb = take(8 * n8), o_ucend = take(8 * n8), o_invs = take(8 * n8), o_bucket = take(4 * n8),
                     o_bfirst = take(4 * n8), o_bcount = take(4 * n8), o_brow = take(8 * n8), o_bstride = take(8 * n8),
                     o_bbase = take(8 * n8), o_totals = take(8 * 8), o_in = take(8 * n8), o_gend = take(8 * n8),
                     o_scal = take(8 * n8),
                     o_const = take(4 * 8);
        // Tile maps are sized once the totals are known; reserve a generous upper bound now
        // so everything lives in one allocation: shard columns <= padded total / nd + 8 * n.
        int64_t padded_bound = 0;
        for (int64_t i = 0; i < n; ++i) padded_bound += numels[i] + (nd - 1);
        const int64_t shard_bound = padded_bound / nd + 8 * n + 8;
        const int64_t tiles_bound = shard_bound / kTileCols + 2;
        int64_t chunks_bound = 0;
        for (int64_t i = 0; i < n; ++i) chunks_bound += (numels[i] + 7) / 8;
        const int64_t utiles_bound = chunks_bound / kUTileChunks + 2;
        const size_t o_tile = take(4 * size_t(tiles_bound)), o_utile = take(4 * size_t(utiles_bound));
        // every bucket's tiles (a tile shared by two buckets is listed for both)
        const size_t o_ptile = take(16 * size_t(tiles_bound + n + 2));

        ZS_HIP(hipGetDevice(&P->device), "hipGetDevice");
        ZS_HIP(hipMalloc(&P->d_mem, bytes), "hipMalloc(plan tables)");
        char* m = static_cast<char*>(P->d_mem);
        T.numel = (int64_t*)(m + o_numel);
        T.pad = (int64_t*)(m + o_pad);
        T.padded = (int64_t*)(m + o_padded);
        T.s = (int64_t*)(m + o_s);
        T.start = (int64_t*)(m + o_start);
        T.sh_end = (int64_t*)(m + o_shend);
        T.off = (int64_t*)(m + o_off);
        T.end = (int64_t*)(m + o_end);
        T.col = (int64_t*)(m + o_col);
        T.dense = (int64_t*)(m + o_dense);
        T.pp = (int64_t*)(m + o_pp);
        T.uc = (int64_t*)(m + o_uc);
        T.ucb = (int64_t*)(m + o_ucb);
        T.ucend = (int64_t*)(m + o_ucend);
        T.inv_s = (double*)(m + o_invs);
        T.bucket = (int32_t*)(m + o_bucket);
        T.bfirst = (int32_t*)(m + o_bfirst);
        T.bcount = (int32_t*)(m + o_bcount);
        T.b_row = (int64_t*)(m + o_brow);
        T.b_stride = (int64_t*)(m + o_bstride);
        T.b_base = (int64_t*)(m + o_bbase);
        T.totals = (int64_t*)(m + o_totals);
        d_numels_in = (int64_t*)(m + o_in);
        int64_t* d_gend = (int64_t*)(m + o_gend);
        P->d_adam_scal = (float*)(m + o_scal);
        P->d_adam_const = (float*)(m + o_const);
        int32_t* d_tile = (int32_t*)(m + o_tile);
        int32_t* d_utile = (int32_t*)(m + o_utile);
        P->d_ptiles = (int64_t*)(m + o_ptile);

        hipStream_t s = nullptr;
        ZS_HIP(hipMemcpy(d_numels_in, numels, 8 * size_t(n), hipMemcpyHostToDevice), "upload numels");
        // gend[i]: the last index of the run of equal group ids holding i (n - 1 without groups)
        tmp.assign(static_cast<size_t>(n), n - 1);
        if (groups)
            for (int64_t i = n - 2; i >= 0; --i) tmp[i] = groups[i] == groups[i + 1] ? tmp[i + 1] : i;
        ZS_HIP(hipMemcpy(d_gend, tmp.data(), 8 * size_t(n), hipMemcpyHostToDevice), "upload groups");
        const int g = grid_for((n + 255) / 256, 1024);
        plan_fields_kernel<<<g, 256, 0, s>>>(T, d_numels_in, n, nd, rank);
        if ((st = check_launch("plan_fields_kernel")) != ZERO_OK) goto done;
        plan_scan_kernel<<<1, kScanThreads, 0, s>>>(T, n);
        if ((st = check_launch("plan_scan_kernel")) != ZERO_OK) goto done;
        plan_buckets_kernel<<<1, 64, 0, s>>>(T, d_gend, n, bucket_bytes > 0 ? bucket_bytes / 2 : -1);
        if ((st = check_launch("plan_buckets_kernel")) != ZERO_OK) goto done;
        plan_place_kernel<<<g, 256, 0, s>>>(T, n);
        if ((st = check_launch("plan_place_kernel")) != ZERO_OK) goto done;
        ZS_HIP(hipMemcpy(totals, T.totals, sizeof totals, hipMemcpyDeviceToHost), "download totals");
        for (int64_t i = 0; i < n; ++i) P->numel_total += numels[i];

        P->n_buckets = totals[0];
        P->shard_numel = totals[1];
        P->shard_elems = totals[2];
        P->padded_total = totals[3];
        P->total_chunks = totals[4];
        const int64_t n_tiles = (P->shard_numel + kTileCols - 1) / kTileCols;
        const int64_t n_utiles = (P->total_chunks + kUTileChunks - 1) / kUTileChunks;
        if (n_tiles + 1 > tiles_bound || n_utiles + 1 > utiles_bound) {
            st = fail(ZERO_EHIP, "zero_plan_create: planner produced sizes beyond their bounds");
            goto done;
        }
        plan_tile_map_kernel<<<grid_for((n_tiles + 256) / 256, 1024), 256, 0, s>>>(T.end, n, kTileShift, d_tile,
                                                                                   n_tiles + 1);
        if ((st = check_launch("plan_tile_map_kernel")) != ZERO_OK) goto done;
        plan_tile_map_kernel<<<grid_for((n_utiles + 256) / 256, 1024), 256, 0, s>>>(T.ucend, n, kUTileShift, d_utile,
                                                                                    n_utiles + 1);
        if ((st = check_launch("plan_tile_map_kernel")) != ZERO_OK) goto done;

        // Host copies of the tables.
        P->h_param = (int64_t*)calloc(size_t(n) * kParamFields, 8);
        P->h_bucket = (int64_t*)calloc(size_t(P->n_buckets) * kBucketFields, 8);
        if (!P->h_param || !P->h_bucket) { st = fail(ZERO_ENOMEM, "zero_plan_create: host tables"); goto done; }
        tmp.resize(size_t(n));
        {
            int64_t* const cols[] = {T.numel, T.pad, T.padded, T.s, T.start, T.sh_end, T.off, nullptr, T.col};
            for (int f = 0; f < kParamFields; ++f) {
                if (!cols[f]) continue;
                ZS_HIP(hipMemcpy(tmp.data(), cols[f], 8 * size_t(n), hipMemcpyDeviceToHost), "download tables");
                for (int64_t i = 0; i < n; ++i) P->h_param[i * kParamFields + f] = tmp[i];
            }
            std::vector<int32_t> b32(static_cast<size_t>(n));
            ZS_HIP(hipMemcpy(b32.data(), T.bucket, 4 * size_t(n), hipMemcpyDeviceToHost), "download buckets");
            for (int64_t i = 0; i < n; ++i) P->h_param[i * kParamFields + PF_BUCKET] = b32[i];
            const int64_t nb = P->n_buckets;
            std::vector<int32_t> f32v(static_cast<size_t>(nb)), c32v(static_cast<size_t>(nb));
            std::vector<int64_t> rowv(static_cast<size_t>(nb)), strv(static_cast<size_t>(nb)), basev(static_cast<size_t>(nb));
            ZS_HIP(hipMemcpy(f32v.data(), T.bfirst, 4 * size_t(nb), hipMemcpyDeviceToHost), "download buckets");
            ZS_HIP(hipMemcpy(c32v.data(), T.bcount, 4 * size_t(nb), hipMemcpyDeviceToHost), "download buckets");
            ZS_HIP(hipMemcpy(rowv.data(), T.b_row, 8 * size_t(nb), hipMemcpyDeviceToHost), "download buckets");
            ZS_HIP(hipMemcpy(strv.data(), T.b_stride, 8 * size_t(nb), hipMemcpyDeviceToHost), "download buckets");
            ZS_HIP(hipMemcpy(basev.data(), T.b_base, 8 * size_t(nb), hipMemcpyDeviceToHost), "download buckets");
            for (int64_t b = 0; b < nb; ++b) {
                int64_t* r = P->h_bucket + b * kBucketFields;
                r[BF_FIRST] = f32v[b];
                r[BF_COUNT] = c32v[b];
                r[BF_ROW] = rowv[b];
                r[BF_STRIDE] = strv[b];
                r[BF_BASE] = basev[b];
            }
        }
        ZS_HIP(hipDeviceSynchronize(), "plan kernels");
        // Unpack chunk range of every bucket (chunk bases are the running sum of ceil(numel / 8)).
        P->h_bucket_chunks = (int64_t*)calloc(size_t(2 * P->n_buckets), 8);
        if (!P->h_bucket_chunks) { st = fail(ZERO_ENOMEM, "zero_plan_create: host tables"); goto done; }
        {
            int64_t u = 0;
            for (int64_t b = 0; b < P->n_buckets; ++b) {
                const int64_t* r = P->h_bucket + b * kBucketFields;
                P->h_bucket_chunks[2 * b] = u;
                for (int64_t i = r[BF_FIRST]; i < r[BF_FIRST] + r[BF_COUNT]; ++i)
                    u += (P->h_param[i * kParamFields + PF_NUMEL] + kChunk - 1) / kChunk;
                P->h_bucket_chunks[2 * b + 1] = u;
            }
        }

        // Tile lists of the pack: per bucket, the tiles of [O_b, O_b + L_b) that lie inside one
        // parameter, then the others.  Parameters are in shard order, so one walk suffices.
        {
            const int64_t nb = P->n_buckets;
            P->h_ptile = (int64_t*)calloc(size_t(3 * nb), 8);
            if (!P->h_ptile) { st = fail(ZERO_ENOMEM, "zero_plan_create: host tables"); goto done; }
            std::vector<int64_t> whole, mixed, all;  // (tile, first parameter ending after its start)
            int64_t i = 0;
            for (int64_t b = 0; b < nb; ++b) {
                const int64_t* r = P->h_bucket + b * kBucketFields;
                whole.clear();
                mixed.clear();
                if (r[BF_STRIDE] > 0) {
                    const int64_t j0 = r[BF_BASE] >> kTileShift, j1 = (r[BF_BASE] + r[BF_STRIDE] - 1) >> kTileShift;
                    for (int64_t j = j0; j <= j1; ++j) {
                        const int64_t x0 = j << kTileShift;
                        while (i < n && P->h_param[i * kParamFields + PF_OFFSET] + P->h_param[i * kParamFields + PF_SHARD] <= x0)
                            ++i;  // first parameter whose range ends after x0
                        const bool in_one = i < n && P->h_param[i * kParamFields + PF_OFFSET] <= x0 &&
                                            P->h_param[i * kParamFields + PF_OFFSET] +
                                                    P->h_param[i * kParamFields + PF_SHARD] >= x0 + kTileCols;
                        std::vector<int64_t>& to = in_one ? whole : mixed;
                        to.push_back(j);
                        to.push_back(i);
                    }
                }
                P->h_ptile[3 * b] = int64_t(all.size() / 2);
                P->h_ptile[3 * b + 1] = int64_t(whole.size() / 2);
                P->h_ptile[3 * b + 2] = int64_t(mixed.size() / 2);
                all.insert(all.end(), whole.begin(), whole.end());
                all.insert(all.end(), mixed.begin(), mixed.end());
            }
            if (int64_t(all.size() / 2) > tiles_bound + n + 2) {
                st = fail(ZERO_EHIP, "zero_plan_create: tile lists beyond their bound");
                goto done;
            }
            if (!all.empty())
                ZS_HIP(hipMemcpy(P->d_ptiles, all.data(), 8 * all.size(), hipMemcpyHostToDevice), "upload tile lists");
        }

        DevPlan& D = P->dev;
        D.n = n;
        D.nd = nd;
        D.rank = rank;
        D.shard_numel = P->shard_numel;
        D.n_tiles = n_tiles;
        D.n_utiles = n_utiles;
        D.numel = T.numel;
        D.s = T.s;
        D.off = T.off;
        D.end = T.end;
        D.inv_s = T.inv_s;
        D.bucket = T.bucket;
        D.ucb = T.ucb;
        D.ucend = T.ucend;
        D.b_base = T.b_base;
        D.b_stride = T.b_stride;
        D.b_row = T.b_row;
        D.tile_first = d_tile;
        D.utile_first = d_utile;
        P->d_bfirst = T.bfirst;
        P->d_bcount = T.bcount;
    }
done:
    if (st != ZERO_OK) {
        zero_plan_destroy(P);
        return st;
    }
    *out = P;
    return ZERO_OK;
}

extern "C" zero_status zero_plan_create(const int64_t* numels, int64_t n_params, int32_t nd, int32_t rank,
                                        int64_t bucket_bytes, int32_t dtype, zero_plan** out) {
    return zero_plan_create_grouped(numels, nullptr, n_params, nd, rank, bucket_bytes, dtype, out);
}

extern "C" zero_status zero_plan_get_summary(const zero_plan* plan, zero_plan_summary* out) {
    if (!plan || !out) return fail(ZERO_EINVAL, "zero_plan_get_summary: NULL argument");
    out->n_params = plan->n;
    out->nd = plan->nd;
    out->rank = plan->rank;
    out->n_buckets = plan->n_buckets;
    out->shard_numel = plan->shard_numel;
    out->shard_elems = plan->shard_elems;
    out->numel_total = plan->numel_total;
    out->padded_total = plan->padded_total;
    out->bucket_elems = plan->bucket_elems;
    out->arena_numel = plan->nd * plan->shard_numel;
    out->dtype = plan->dtype;
    out->device = plan->device;
    return ZERO_OK;
}

extern "C" zero_status zero_plan_param_info(const zero_plan* plan, int64_t i, zero_param_info* out) {
    if (!plan || !out) return fail(ZERO_EINVAL, "zero_plan_param_info: NULL argument");
    if (i < 0 || i >= plan->n) return fail(ZERO_EINVAL, "zero_plan_param_info: index %lld out of range", (long long)i);
    const int64_t* r = plan->h_param + i * kParamFields;
    out->numel = r[PF_NUMEL];
    out->pad = r[PF_PAD];
    out->padded_numel = r[PF_PADDED];
    out->shard_size = r[PF_SHARD];
    out->shard_start = r[PF_START];
    out->shard_end = r[PF_END];
    out->shard_offset = r[PF_OFFSET];
    out->bucket = r[PF_BUCKET];
    out->bucket_col = r[PF_COL];
    return ZERO_OK;
}

extern "C" zero_status zero_plan_bucket_info(const zero_plan* plan, int64_t b, zero_bucket_info* out) {
    if (!plan || !out) return fail(ZERO_EINVAL, "zero_plan_bucket_info: NULL argument");
    if (b < 0 || b >= plan->n_buckets) return fail(ZERO_EINVAL, "zero_plan_bucket_info: bucket %lld out of range", (long long)b);
    const int64_t* r = plan->h_bucket + b * kBucketFields;
    out->first_param = r[BF_FIRST];
    out->n_params = r[BF_COUNT];
    out->row_elems = r[BF_ROW];
    out->row_stride = r[BF_STRIDE];
    out->shard_base = r[BF_BASE];
    out->block_offset = plan->nd * r[BF_BASE];
    return ZERO_OK;
}

// Model-state accounting of the upskillscore ZeRO summary (model states; ZeRO-DP stages):
// 2 bytes of 16-bit parameters + 2 of 16-bit gradients + 12 of fp32 optimizer state per
// parameter; stage k partitions the first k of {optimizer state, gradients, parameters}.
extern "C" zero_status zero_model_state_bytes(double psi, double nd, int32_t stage, double* out) {
    if (!out) return fail(ZERO_EINVAL, "zero_model_state_bytes: out is NULL");
    if (!(psi >= 0.0) || !(nd >= 1.0) || stage < 0 || stage > 3)
        return fail(ZERO_EINVAL, "zero_model_state_bytes: bad arguments");
    const double params_b = 2.0 * psi, grads_b = 2.0 * psi, optim_b = 12.0 * psi;
    *out = (stage >= 3 ? params_b / nd : params_b) + (stage >= 2 ? grads_b / nd : grads_b) +
           (stage >= 1 ? optim_b / nd : optim_b);
    return ZERO_OK;
}

extern "C" zero_status zero_plan_model_state_bytes(const zero_plan* plan, int32_t stage, double* out) {
    if (!plan) return fail(ZERO_EINVAL, "zero_plan_model_state_bytes: plan is NULL");
    return zero_model_state_bytes(double(plan->padded_total), double(plan->nd), stage, out);
}

extern "C" const char* zero_last_error(void) { return g_err; }
