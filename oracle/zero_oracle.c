/*
 * zero_oracle.c — plain, slow CPU oracle of the ZeRO-1/2 per-rank shard pipeline.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load this file's library.  It shares no code, header, table or
 * helper with the GPU library; every function is written from the definitions on the
 * pages below, in the order the pages state them, with no blocking or reordering.
 * Built with gcc -O2 -fno-fast-math -ffp-contract=off (SSE2 scalar arithmetic), so every
 * float operation below is one IEEE-754 operation with round-to-nearest-even.
 *
 * Pages (title, section):
 *   [LLZ] ColossalAI issue "[zero] improving compatibility of low level zero" — Design
 *         (Notion, INIT, BWD, Optim)
 *   [FR]  briefia.fr "L'IA sur plusieurs GPU : ZeRO et FSDP" — "Implémentation simplifiée",
 *         "ZeRO-1 : Partitionnement des états de l'optimiseur", "Problème de mémoire dans DDP"
 *   [Z3]  llm-engineer card "ZeRO-3" — the section contrasting the ZeRO-1/2 all-gather
 *   [ZP]  upskillscore summary of "ZeRO: Memory Optimizations Toward Training Trillion
 *         Parameter Models" — model states; the three ZeRO-DP stages
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - parameter order is list order; buckets are contiguous runs of the list, closed
 *     before a parameter that would overflow the capacity (counted in padded 16-bit
 *     elements), a parameter larger than the capacity alone in its bucket;
 *   - a bucket's rank rows are stored L_b = S_b rounded up to 8 elements apart (the row
 *     contents are the pages' concatenation; the gap [S_b, L_b) is zero), and rank r's fp32
 *     shard is the concatenation of its bucket rows at those same strides;
 *   - the reduce is a sum (not a mean), accumulated in fp32 in ascending rank order seeded
 *     with rank 0's value; averaging and loss-scale removal are the Adam grad_scale;
 *   - Adam is textbook bias-corrected Adam without weight decay; dead parameters (no
 *     gradient) and skipped steps leave every piece of state untouched, step count
 *     included; the model parameter is the fp32 master rounded to 16 bits by
 *     round-to-nearest-even.
 *
 * Parity status of each function: see the tests that pin them (plan: closed form and brute
 * force; pack/unpack: the [LLZ BWD] worked layout and identity; reduce: exact integer sums,
 * two-term correctly rounded sums, the ordering example; Adam: library Adam and closed
 * forms; conversions: library conversions; accounting: the [ZP] worked figures).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Field indices of one parameter record (int64 each). */
enum {
    ORP_NUMEL = 0,
    ORP_PAD,
    ORP_PADDED,
    ORP_SHARD,
    ORP_START,
    ORP_END,
    ORP_OFFSET,
    ORP_BUCKET,
    ORP_COL,
    ORP_NFIELDS
};
/* Field indices of one bucket record (int64 each). */
enum { ORB_FIRST = 0, ORB_COUNT, ORB_ROW, ORB_STRIDE, ORB_BASE, ORB_NFIELDS };

#define OR_BF16 1
#define OR_FP16 2

int oracle_param_fields(void) { return ORP_NFIELDS; }

/*
 * Threads for the element loops (1 unless set).  With more than one thread, a loop over the
 * columns (or elements) of one parameter is split into disjoint contiguous ranges, one per
 * thread; every element is still computed by the same operations in the same order, so the
 * results are identical for any thread count.  Used only to time the oracle on all host cores.
 */
static int g_threads = 1;
void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int oracle_get_threads(void) { return g_threads; }
#define OR_PARALLEL _Pragma("omp parallel for num_threads(g_threads) if(g_threads > 1) schedule(static)")
#define OR_PARALLEL2 _Pragma("omp parallel for collapse(2) num_threads(g_threads) if(g_threads > 1) schedule(static)")
int oracle_bucket_fields(void) { return ORB_NFIELDS; }

/* ------------------------------------------------------------------ plan (O1) ------ */
/*
 * [FR Implémentation simplifiée]: every flat parameter is zero-padded to a multiple of the
 * world size, viewed as [world_size, -1], and rank r owns row r (its shard_start and
 * shard_end in the padded flat).  [LLZ INIT]: every parameter is split evenly over the ranks.
 * Here a row holds ceil(numel / Nd) elements; the padding is whatever the Nd full rows hold
 * beyond numel (the tests check it against the page's pad formula for every numel up to 3Nd).
 * [LLZ BWD]: gradients go into buckets; when full, each one is viewed as [Nd, -1] and the
 * rows of one rank are flattened together.
 * [Z3]: ZeRO-3 gathers and frees the parameters one layer (unit) at a time; with groups (one
 * id per parameter, NULL = a single group), a bucket also ends where the group id changes, so
 * that every bucket lies inside one unit.
 * Returns the number of buckets, or -1 on an invalid argument.  params: n * ORP_NFIELDS,
 * buckets: n * ORB_NFIELDS (n is an upper bound on the bucket count).
 */
int64_t oracle_plan(const int64_t* numels, const int32_t* groups, int64_t n, int64_t nd, int64_t rank,
                    int64_t bucket_bytes, int64_t* params, int64_t* buckets, int64_t* shard_len) {
    if (n < 1 || nd < 1 || rank < 0 || rank >= nd || bucket_bytes < 0) return -1;
    for (int64_t i = 0; i < n; i++) {
        if (numels[i] < 0) return -1;
        int64_t* p = params + i * ORP_NFIELDS;
        int64_t row_len = (numels[i] + nd - 1) / nd; /* elements of one rank's row */
        p[ORP_NUMEL] = numels[i];
        p[ORP_SHARD] = row_len;
        p[ORP_PADDED] = nd * row_len;
        p[ORP_PAD] = nd * row_len - numels[i];
        p[ORP_START] = rank * row_len;
        p[ORP_END] = (rank + 1) * row_len;
    }

    /* Greedy buckets over the list, capacity in 16-bit elements (0 bytes = unbounded). */
    int64_t capacity = bucket_bytes / 2;
    int64_t nb = 0;
    int64_t fill = 0;
    for (int64_t i = 0; i < n; i++) {
        int64_t padded = params[i * ORP_NFIELDS + ORP_PADDED];
        int open_nonempty = nb > 0 && buckets[(nb - 1) * ORB_NFIELDS + ORB_COUNT] > 0;
        int new_group = groups != NULL && i > 0 && groups[i] != groups[i - 1];
        if (nb == 0 || new_group || (bucket_bytes > 0 && open_nonempty && fill + padded > capacity)) {
            int64_t* bk = buckets + nb * ORB_NFIELDS;
            bk[ORB_FIRST] = i;
            bk[ORB_COUNT] = 0;
            nb++;
            fill = 0;
        }
        buckets[(nb - 1) * ORB_NFIELDS + ORB_COUNT] += 1;
        params[i * ORP_NFIELDS + ORP_BUCKET] = nb - 1;
        fill += padded;
    }

    /* Row r of a bucket: the shards of its parameters one after the other. */
    int64_t base = 0;
    for (int64_t b = 0; b < nb; b++) {
        int64_t* bk = buckets + b * ORB_NFIELDS;
        int64_t col = 0;
        for (int64_t i = bk[ORB_FIRST]; i < bk[ORB_FIRST] + bk[ORB_COUNT]; i++) {
            params[i * ORP_NFIELDS + ORP_COL] = col;
            params[i * ORP_NFIELDS + ORP_OFFSET] = base + col;
            col += params[i * ORP_NFIELDS + ORP_SHARD];
        }
        bk[ORB_ROW] = col;
        bk[ORB_STRIDE] = ((col + 7) / 8) * 8;
        bk[ORB_BASE] = base;
        base += bk[ORB_STRIDE];
    }
    *shard_len = base;
    return nb;
}

/* ------------------------------------------------------- 16-bit <-> fp32 ---------- */
/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    if (expo == 31) {
        if (frac == 0) return sign ? -INFINITY : INFINITY;
        /* NaN: quiet, payload moved to the top of the binary32 fraction */
        uint32_t bits = ((uint32_t)sign << 31) | 0x7fc00000u | ((uint32_t)frac << 13);
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
    else
        mag = ldexp(1024.0 + (double)frac, expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return (float)(sign ? -mag : mag); /* exact: at most 11 significant bits */
}

/* bfloat16 is the top half of a binary32. */
float oracle_bf16_to_f32(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even on the 16 dropped bits. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0)
        return (uint16_t)(((bits >> 16) & 0x8000u) | 0x7fc0u); /* NaN -> quiet NaN */
    uint32_t upper = bits >> 16;
    uint32_t lower = bits & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1; /* carries into exponent */
    return (uint16_t)upper;
}

/* binary32 -> binary16, round to nearest, ties to even; subnormals kept; overflow to inf. */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    double x = fabs((double)f);
    if (x >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* at or past the midpoint above 65504 */
    if (x < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-24 */
        double q = rint(x * ldexp(1.0, 24)); /* default rounding mode: nearest, ties to even */
        return (uint16_t)(sign | (uint16_t)q); /* q == 1024 encodes the smallest normal */
    }
    int ex;
    frexp(x, &ex); /* x = m * 2^ex, m in [0.5, 1): x in [2^(ex-1), 2^ex) */
    int e = ex - 1;
    double q = rint(ldexp(x, 10 - e)); /* significand scaled to [1024, 2048] */
    uint32_t enc = ((uint32_t)(e + 15) << 10) + (uint32_t)(q - 1024.0); /* q == 2048 carries */
    return (uint16_t)(sign | enc);
}

static float to_f32(uint16_t h, int dtype) { return dtype == OR_FP16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h); }
static uint16_t from_f32(float f, int dtype) { return dtype == OR_FP16 ? oracle_f32_to_f16(f) : oracle_f32_to_bf16(f); }

void oracle_convert_to_f32(const uint16_t* in, float* out, int64_t count, int dtype) {
    for (int64_t i = 0; i < count; i++) out[i] = to_f32(in[i], dtype);
}
void oracle_convert_from_f32(const float* in, uint16_t* out, int64_t count, int dtype) {
    for (int64_t i = 0; i < count; i++) out[i] = from_f32(in[i], dtype);
}

/* ------------------------------------------------------------------ pack (O2) ------ */
/*
 * [LLZ BWD]: each gradient of the bucket is viewed as [Nd, -1]; row k of every gradient
 * goes to rank k, and rank k's rows are flattened into one buffer, in list order.  With
 * the padding of [FR Implémentation simplifiée] being zeros, element j of row k of
 * parameter i is g_i[k*s_i + j] when that index is below numel_i and +0 otherwise.
 * grads[i] == NULL marks a parameter without a gradient ([LLZ Optim] layer drop): its
 * columns are left as they were.  The row gap [S_b, L_b) is set to zero.
 */
void oracle_pack_bucket(const int64_t* params, const int64_t* buckets, int64_t nd, int64_t b,
                        const uint16_t* const* grads, uint16_t* packed) {
    const int64_t* bk = buckets + b * ORB_NFIELDS;
    int64_t L = bk[ORB_STRIDE];
    for (int64_t i = bk[ORB_FIRST]; i < bk[ORB_FIRST] + bk[ORB_COUNT]; i++) {
        const uint16_t* g = grads[i];
        if (g == NULL) continue;
        const int64_t* p = params + i * ORP_NFIELDS;
        int64_t s = p[ORP_SHARD], numel = p[ORP_NUMEL], col = p[ORP_COL];
        OR_PARALLEL2
        for (int64_t k = 0; k < nd; k++)
            for (int64_t j = 0; j < s; j++) {
                int64_t e = k * s + j;
                packed[k * L + col + j] = (e < numel) ? g[e] : (uint16_t)0;
            }
    }
    for (int64_t k = 0; k < nd; k++)
        for (int64_t c = bk[ORB_ROW]; c < L; c++) packed[k * L + c] = 0;
}

/* ---------------------------------------------------------------- reduce (O3) ------ */
/*
 * The reduce-scatter of [LLZ BWD] (ZeRO-2) and [ZP stage Pos+g] leaves on rank r the sum
 * over ranks of row r.  One column: start from rank 0's value converted to fp32 (exact),
 * then add ranks 1..Nd-1 in ascending order, one fp32 addition each.
 */
float oracle_reduce_column(const uint16_t* vals, int64_t nd, int64_t stride, int dtype) {
    float acc = to_f32(vals[0], dtype);
    for (int64_t k = 1; k < nd; k++) acc = acc + to_f32(vals[k * stride], dtype);
    return acc;
}

/* Row k is rows[k*row_stride ...]; writes g32[O_b + c] for columns of live parameters. */
void oracle_reduce_bucket(const int64_t* params, const int64_t* buckets, int64_t nd, int64_t b,
                          const uint16_t* rows, int64_t row_stride, int dtype, const uint8_t* live, float* g32) {
    const int64_t* bk = buckets + b * ORB_NFIELDS;
    for (int64_t i = bk[ORB_FIRST]; i < bk[ORB_FIRST] + bk[ORB_COUNT]; i++) {
        if (!live[i]) continue;
        const int64_t* p = params + i * ORP_NFIELDS;
        OR_PARALLEL
        for (int64_t j = 0; j < p[ORP_SHARD]; j++) {
            int64_t c = p[ORP_COL] + j;
            g32[bk[ORB_BASE] + c] = oracle_reduce_column(rows + c, nd, row_stride, dtype);
        }
    }
}

/* -------------------------------------------------------------- overflow (O4) ------ */
/* 1 if any value in a live parameter's slice is inf or NaN (all exponent bits set). */
int oracle_overflow(const int64_t* params, int64_t n, const float* g32, const uint8_t* live) {
    int flag = 0;
    for (int64_t i = 0; i < n; i++) {
        if (!live[i]) continue;
        const int64_t* p = params + i * ORP_NFIELDS;
        _Pragma("omp parallel for num_threads(g_threads) if(g_threads > 1) schedule(static) reduction(|:flag)")
        for (int64_t e = p[ORP_OFFSET]; e < p[ORP_OFFSET] + p[ORP_SHARD]; e++) {
            uint32_t bits;
            memcpy(&bits, &g32[e], 4);
            if ((bits & 0x7f800000u) == 0x7f800000u) flag = 1;
        }
    }
    return flag;
}

/*
 * The input-side verdict of the fused path (a reading: the pages do not treat overflow).  1 if
 * a gradient element of a parameter of bucket b that has a gradient (grads[i] != NULL) is inf
 * or NaN, or if |x| * nd > 2^126.  The product of a 16-bit value (at most 11 significant bits)
 * and nd (at most 16 bits) is exact in double, so the comparison is exact.  Padding is not a
 * gradient element and is not examined.
 */
int oracle_input_check(const int64_t* params, const int64_t* buckets, int64_t nd, int64_t b,
                       const uint16_t* const* grads, int dtype) {
    const int64_t* bk = buckets + b * ORB_NFIELDS;
    const double limit = ldexp(1.0, 126);
    int flag = 0;
    for (int64_t i = bk[ORB_FIRST]; i < bk[ORB_FIRST] + bk[ORB_COUNT]; i++) {
        const uint16_t* g = grads[i];
        if (g == NULL) continue;
        const int64_t numel = params[i * ORP_NFIELDS + ORP_NUMEL];
        for (int64_t e = 0; e < numel; e++) {
            double x = (double)to_f32(g[e], dtype);
            if (!isfinite(x) || fabs(x) * (double)nd > limit) flag = 1;
        }
    }
    return flag;
}

/* ------------------------------------------------------------------ Adam (O5) ------ */
/*
 * One element of textbook Adam (bias-corrected, no weight decay), in double from the
 * fp32 state; the state is stored back rounded to fp32.  t is the parameter's step count
 * after this step.  [ZP model states]: the optimizer keeps an fp32 copy of the
 * parameters, the momentum and the variance.
 */
void oracle_adam_element(float g32, float* p32, float* m, float* v, int64_t t, double lr, double beta1,
                         double beta2, double eps, double grad_scale) {
    double g = (double)g32 * grad_scale;
    double mm = beta1 * (double)(*m) + (1.0 - beta1) * g;
    double vv = beta2 * (double)(*v) + (1.0 - beta2) * g * g;
    double m_hat = mm / (1.0 - pow(beta1, (double)t));
    double v_hat = vv / (1.0 - pow(beta2, (double)t));
    double p = (double)(*p32) - lr * m_hat / (sqrt(v_hat) + eps);
    *m = (float)mm;
    *v = (float)vv;
    *p32 = (float)p;
}

/*
 * [LLZ Optim]: each rank steps its own p32 with the matching g, only for parameters that
 * have a gradient this step; then [Z3] / [FR ZeRO-1 step order] the updated parameters are
 * all-gathered, so row r of every bucket's gathered block receives the 16-bit rounding of
 * the new p32.  flag != 0 skips the whole step (overflow somewhere).
 */
void oracle_adam(const int64_t* params, const int64_t* buckets, int64_t n, int64_t nd, int64_t rank,
                 const float* g32, float* p32, float* m, float* v, const uint8_t* live, int32_t* steps, double lr,
                 double beta1, double beta2, double eps, double grad_scale, int flag, uint16_t* arena, int dtype) {
    if (flag) return;
    for (int64_t i = 0; i < n; i++) {
        if (!live[i]) continue;
        const int64_t* p = params + i * ORP_NFIELDS;
        const int64_t* bk = buckets + p[ORP_BUCKET] * ORB_NFIELDS;
        steps[i] += 1;
        OR_PARALLEL
        for (int64_t e = p[ORP_OFFSET]; e < p[ORP_OFFSET] + p[ORP_SHARD]; e++) {
            oracle_adam_element(g32[e], &p32[e], &m[e], &v[e], steps[i], lr, beta1, beta2, eps, grad_scale);
            int64_t c = e - bk[ORB_BASE];
            arena[nd * bk[ORB_BASE] + rank * bk[ORB_STRIDE] + c] = from_f32(p32[e], dtype);
        }
    }
}

/* ------------------------------------------------------ dynamic loss scaling ------ */
/*
 * Not on the pages (a reading: the usual dynamic rule for 16-bit gradients).  State: the
 * current scale, the count of clean steps since it last changed, and the steps skipped.  A
 * step with the overflow flag set multiplies the scale by the back-off factor (not below the
 * minimum) and restarts the count; a clean step adds one to the count, and when the count
 * reaches the growth interval the scale is multiplied by the growth factor (not above the
 * maximum) and the count restarts.  Products in binary32.
 */
typedef struct {
    float scale;
    int32_t good_steps;
    int32_t growth_interval;
    float growth_factor;
    float backoff_factor;
    float min_scale;
    float max_scale;
    int32_t overflows;
} oracle_scaler;

void oracle_loss_scaler_update(oracle_scaler* s, int flag) {
    if (flag) {
        float backed = s->scale * s->backoff_factor;
        s->scale = (backed < s->min_scale) ? s->min_scale : backed;
        s->good_steps = 0;
        s->overflows += 1;
        return;
    }
    s->good_steps += 1;
    if (s->good_steps == s->growth_interval) {
        float grown = s->scale * s->growth_factor;
        s->scale = (grown > s->max_scale) ? s->max_scale : grown;
        s->good_steps = 0;
    }
}

/* ---------------------------------------------------------------- unpack (O6) ------ */
/*
 * [Z3]: after the ZeRO-1/2 all-gather every rank holds the full updated parameters.
 * Element e of parameter i sits in row e / s_i at column col_i + e mod s_i of the bucket's
 * gathered block; padding (e >= numel_i) is dropped.  outs[i] == NULL skips parameter i.
 */
void oracle_unpack_bucket(const int64_t* params, const int64_t* buckets, int64_t b, const uint16_t* gathered,
                          uint16_t* const* outs) {
    const int64_t* bk = buckets + b * ORB_NFIELDS;
    int64_t L = bk[ORB_STRIDE];
    for (int64_t i = bk[ORB_FIRST]; i < bk[ORB_FIRST] + bk[ORB_COUNT]; i++) {
        uint16_t* out = outs[i];
        if (out == NULL) continue;
        const int64_t* p = params + i * ORP_NFIELDS;
        int64_t s = p[ORP_SHARD];
        OR_PARALLEL
        for (int64_t e = 0; e < p[ORP_NUMEL]; e++) {
            int64_t k = e / s, j = e % s;
            out[e] = gathered[k * L + p[ORP_COL] + j];
        }
    }
}

/* ------------------------------------------------------------ accounting (O7) ------ */
/*
 * [ZP model states]: mixed-precision Adam keeps 2 bytes of 16-bit parameters, 2 of 16-bit
 * gradients and K = 12 of fp32 optimizer state (copy, momentum, variance) per parameter.
 * [ZP ZeRO-DP stages]: stage 1 partitions the optimizer state over Nd, stage 2 also the
 * gradients, stage 3 also the parameters.  Stage 0 is plain data parallelism.
 */
double oracle_model_state_bytes(double psi, double nd, int stage) {
    double params_b = 2.0 * psi, grads_b = 2.0 * psi, optim_b = 12.0 * psi;
    switch (stage) {
        case 0: return params_b + grads_b + optim_b;
        case 1: return params_b + grads_b + optim_b / nd;
        case 2: return params_b + grads_b / nd + optim_b / nd;
        case 3: return params_b / nd + grads_b / nd + optim_b / nd;
        default: return -1.0;
    }
}

/* ------------------------------------------------------------ shard init (O1) ------ */
/*
 * [LLZ INIT] / [FR Implémentation simplifiée]: rank r's p32 for parameter i is row r of
 * the zero-padded flat parameter, cloned: element j is master_i[r*s_i + j] when that
 * index is below numel_i and +0 otherwise.  masters[i] == NULL leaves the slice as it
 * was; the row gaps are set to zero.  src_dtype 0 = fp32 source, else a 16-bit source
 * converted exactly.
 */
void oracle_shard_init(const int64_t* params, const int64_t* buckets, int64_t n, int64_t nb,
                       const void* const* masters, int src_dtype, float* p32) {
    for (int64_t i = 0; i < n; i++) {
        if (masters[i] == NULL) continue;
        const int64_t* p = params + i * ORP_NFIELDS;
        for (int64_t j = 0; j < p[ORP_SHARD]; j++) {
            int64_t e = p[ORP_START] + j;
            float val = 0.0f;
            if (e < p[ORP_NUMEL]) {
                if (src_dtype == 0)
                    val = ((const float*)masters[i])[e];
                else
                    val = to_f32(((const uint16_t*)masters[i])[e], src_dtype);
            }
            p32[p[ORP_OFFSET] + j] = val;
        }
    }
    for (int64_t b = 0; b < nb; b++) {
        const int64_t* bk = buckets + b * ORB_NFIELDS;
        for (int64_t c = bk[ORB_ROW]; c < bk[ORB_STRIDE]; c++) p32[bk[ORB_BASE] + c] = 0.0f;
    }
}

/* ------------------------------------------------- element-wise layout queries ------ */
/*
 * Where a packed element comes from (the definition of O2 read backwards, for sampled
 * checks of big buffers): column c of row k of bucket b.  Returns 0 for the row gap,
 * 1 for gradient element (*i_out, *e_out), 2 for a padding element of parameter *i_out.
 */
int oracle_pack_locate(const int64_t* params, const int64_t* buckets, int64_t b, int64_t k, int64_t c,
                       int64_t* i_out, int64_t* e_out) {
    const int64_t* bk = buckets + b * ORB_NFIELDS;
    for (int64_t i = bk[ORB_FIRST]; i < bk[ORB_FIRST] + bk[ORB_COUNT]; i++) {
        const int64_t* p = params + i * ORP_NFIELDS;
        if (c >= p[ORP_COL] && c < p[ORP_COL] + p[ORP_SHARD]) {
            int64_t e = k * p[ORP_SHARD] + (c - p[ORP_COL]);
            *i_out = i;
            *e_out = e;
            return e < p[ORP_NUMEL] ? 1 : 2;
        }
    }
    return 0;
}

/* Row and column of a bucket block that element e of parameter i is unpacked from (O6). */
void oracle_unpack_locate(const int64_t* params, int64_t i, int64_t e, int64_t* row, int64_t* col) {
    const int64_t* p = params + i * ORP_NFIELDS;
    *row = e / p[ORP_SHARD];
    *col = p[ORP_COL] + e % p[ORP_SHARD];
}
