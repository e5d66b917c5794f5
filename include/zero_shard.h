/*
 * zero_shard.h — C ABI of the ZeRO-1/2 per-rank shard pipeline for one MI355X (gfx950).
 *
 * Sources cited below (page title, then the section on that page):
 *   [LLZ]  ColossalAI issue "[zero] improving compatibility of low level zero"
 *          (sections Overview, Goal, Design: Notion / INIT / BWD / Optim)
 *   [FR]   briefia.fr "L'IA sur plusieurs GPU : ZeRO et FSDP"
 *          (sections "Problème de mémoire dans DDP", "ZeRO-1 : Partitionnement des états
 *          de l'optimiseur", "Implémentation simplifiée")
 *   [Z3]   llm-engineer card "ZeRO-3" (section on how the ZeRO-1/2 all-gather differs)
 *   [ZP]   upskillscore summary of "ZeRO: Memory Optimizations Toward Training Trillion
 *          Parameter Models" (sections on model states and on the three ZeRO-DP stages)
 *
 * Vocabulary (the pages' notation):
 *   Nd      number of data-parallel ranks ("world_size" in [LLZ], "Nd" in [ZP]); here the
 *           ranks are virtual: every rank's data lives in the one GPU's memory.
 *   r       this rank.
 *   p32     the fp32 master copy of a parameter held by the optimizer [LLZ Notion];
 *   p       the low-precision (bf16 or fp16) model parameter; g its gradient.
 *   s_i     shard_size of parameter i = padded_numel / Nd  [FR Implémentation simplifiée].
 *
 * Data layout (all sizes in elements):
 *   Parameter i is zero-padded to padded_numel_i = numel_i + pad_i (a multiple of Nd) and
 *   viewed as [Nd, s_i]; row k is the part owned by rank k [LLZ INIT].  Parameters are
 *   grouped, in list order, into buckets [LLZ BWD].  A bucket's rank row k is the
 *   concatenation, in list order, of row k of each of its parameters (the "flatten by rank"
 *   of [LLZ BWD]): row_elems S_b = sum of s_i over the bucket; parameter i starts at column
 *   bucket_col_i.  Rows are stored row_stride L_b apart, L_b = S_b rounded up to a multiple
 *   of 8 elements so that every row starts on a 16-byte boundary; columns [S_b, L_b) of a
 *   row are a zero gap.  A bucket's packed (or gathered) block is therefore [Nd][L_b].
 *   Rank r's flat fp32 shard (p32, m, v, reduced gradient g32) is the concatenation of
 *   row r of every bucket, each starting at shard_base O_b = sum of L over earlier
 *   buckets; parameter i's slice is [shard_offset_i, shard_offset_i + s_i) with
 *   shard_offset_i = O_b + bucket_col_i.  shard_numel = sum of L_b over all buckets.
 *   An all-gather "arena" holds every bucket's [Nd][L_b] block back to back; bucket b's
 *   block starts at element Nd * O_b.
 *
 * Ownership and threading:
 *   The caller owns every data buffer and pointer table (device memory).  A pointer table
 *   and every buffer it names must stay allocated until all work that reads or writes
 *   through them has finished: the calls only enqueue kernels, and a kernel dereferences the
 *   table's pointers when it runs -- after the call returned, and again at every replay of a
 *   captured graph.  Freeing a named buffer earlier (or letting a caching allocator hand its
 *   memory back to the driver) makes a later kernel access unmapped memory.  A plan owns its
 *   host tables, its device copies of them and a small device scratch used by
 *   zero_adam_step.  Hot calls (pack, reduce, overflow, adam, unpack) never allocate and
 *   never synchronise the host; they enqueue on `stream` (a hipStream_t; NULL = the null
 *   stream) and return.  They must be called with the plan's device current.  A plan is
 *   read-only after creation except for the Adam scratch, so hot calls on different
 *   streams are safe when their outputs are disjoint and at most one zero_adam_step per
 *   plan is in flight at a time.
 *
 * Errors:
 *   Every call returns a zero_status and never aborts or prints.  ZERO_EINVAL: a bad
 *   argument (the call did nothing).  ZERO_ERANGE: a size overflow.  ZERO_ENOMEM: a
 *   device or host allocation failed (plan creation only).  ZERO_EHIP: a HIP call failed.
 *   zero_last_error() returns a thread-local message for the last failing call.
 *   A plan stays valid after any failed hot call.
 *
 * Aliasing:
 *   The buffers a call writes must not overlap one another or any buffer the same call reads,
 *   except the arrays a call updates in place (p32, m, v, step counts, the flag, the loss
 *   scaler): the kernels are compiled on the assumption that distinct pointers do not alias.
 *   The per-parameter flats one zero_unpack writes must not overlap each other (tables that
 *   are only read, such as the gradients of a pack, may name overlapping or shared buffers).
 *
 * Empty work:
 *   A call with nothing to move -- a per-bucket call on a bucket whose rows are empty
 *   (L_b = 0: only parameters of numel 0), or a shard-wide call on a plan whose shard has no
 *   elements -- checks the plan and the bucket index and returns ZERO_OK; its buffer pointers
 *   may then be NULL (a zero-length tensor often has a NULL data pointer).  zero_adam_step on
 *   an empty shard still advances the step counts of live parameters, so it still needs
 *   d_live, d_steps and hp.
 *
 * Alignment:
 *   Block buffers (packed, gathered, all-gather arena, receive rows) and the fp32 shard
 *   arrays must be 16-byte aligned (ZERO_EINVAL otherwise).  Per-parameter gradient and
 *   parameter buffers only need 2-byte alignment; 16-byte aligned ones take the wide path.
 *   Kernels may read (never write) up to the end of the 16-byte granule that holds a
 *   buffer's last element, which every hipMalloc / torch allocation provides.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum zero_status {
    ZERO_OK = 0,
    ZERO_EINVAL = -1,
    ZERO_ENOMEM = -2,
    ZERO_EHIP = -3,
    ZERO_ERANGE = -4
} zero_status;

/* Low-precision type of gradients and model parameters [ZP model states: 16-bit params
 * and grads in mixed-precision training]. */
typedef enum zero_dtype { ZERO_BF16 = 1, ZERO_FP16 = 2 } zero_dtype;

typedef struct zero_plan zero_plan; /* opaque */

/* One row of the per-parameter metadata record [FR Implémentation simplifiée: the
 * record of original shape, padded_numel, shard_size, shard_start, shard_end], plus the
 * placement of the rank-r slice in the bucket rows and in the flat shard. */
typedef struct zero_param_info {
    int64_t numel;        /* elements of the flat parameter                              */
    int64_t pad;          /* (Nd - numel % Nd) % Nd zero elements appended               */
    int64_t padded_numel; /* numel + pad                                                 */
    int64_t shard_size;   /* s_i = padded_numel / Nd                                     */
    int64_t shard_start;  /* r * s_i: first element of rank r's row in the padded flat   */
    int64_t shard_end;    /* shard_start + s_i                                           */
    int64_t shard_offset; /* start of the slice in rank r's flat fp32 shard              */
    int64_t bucket;       /* bucket index                                                */
    int64_t bucket_col;   /* column of the slice inside every rank row of its bucket     */
} zero_param_info;

typedef struct zero_bucket_info {
    int64_t first_param;  /* index of the bucket's first parameter                      */
    int64_t n_params;     /* parameters in the bucket (a contiguous run of the list)     */
    int64_t row_elems;    /* S_b                                                         */
    int64_t row_stride;   /* L_b = S_b rounded up to a multiple of 8                     */
    int64_t shard_base;   /* O_b                                                         */
    int64_t block_offset; /* Nd * O_b: start of the bucket's block in an all-gather arena */
} zero_bucket_info;

typedef struct zero_plan_summary {
    int64_t n_params;
    int64_t nd;
    int64_t rank;
    int64_t n_buckets;
    int64_t shard_numel;    /* sum of L_b: length of each fp32 shard array               */
    int64_t shard_elems;    /* sum of s_i (shard_numel minus the row gaps)               */
    int64_t numel_total;    /* sum of numel_i                                            */
    int64_t padded_total;   /* Psi = sum of padded_numel_i                               */
    int64_t bucket_elems;   /* bucket capacity in padded 16-bit elements (0 = unbounded) */
    int64_t arena_numel;    /* Nd * shard_numel: length of an all-gather arena           */
    int32_t dtype;          /* zero_dtype                                                */
    int32_t device;         /* HIP device the plan lives on                              */
} zero_plan_summary;

/* Dynamic loss scaler, kept in device memory so that a step never waits for the host.  The
 * pages do not treat loss scaling; this is the usual dynamic rule for 16-bit gradients: after
 * a step whose overflow flag is set, scale = max(scale * backoff_factor, min_scale) and the
 * step is counted in `overflows`; after growth_interval consecutive clean steps, scale =
 * min(scale * growth_factor, max_scale) (fp32 products, round to nearest even).  The caller
 * multiplies its loss by `scale` before the backward pass (reading it on the device) and
 * passes the scaler to the Adam step through zero_adam_hparams.loss_scaler.  The caller owns
 * the memory: sizeof(zero_loss_scaler) bytes, 4-byte aligned. */
typedef struct zero_loss_scaler {
    float scale;              /* the loss scale the current step's gradients carry       */
    int32_t good_steps;       /* clean steps since the scale last changed                 */
    int32_t growth_interval;  /* clean steps before the scale grows (>= 1)                */
    float growth_factor;      /* >= 1                                                     */
    float backoff_factor;     /* in (0, 1]                                                */
    float min_scale;          /* 0 < min_scale <= scale <= max_scale, all finite          */
    float max_scale;
    int32_t overflows;        /* steps skipped so far                                     */
} zero_loss_scaler;

/* Adam hyperparameters.  The pages name Adam's momentum and variance as the optimizer
 * state [ZP model states; FR Problème de mémoire dans DDP] but give no update rule; the
 * step is textbook bias-corrected Adam without weight decay.  grad_scale multiplies the
 * reduced gradient before use: 1 / (Nd * loss_scale) turns the rank sum into the mean
 * of unscaled gradients.  With a dynamic loss scale, loss_scaler points to the device
 * zero_loss_scaler and the multiplier is grad_scale / loss_scaler->scale (then grad_scale is
 * 1 / Nd), formed in double on the device when the step runs and rounded to fp32 once;
 * NULL = a static scale folded into grad_scale. */
typedef struct zero_adam_hparams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double grad_scale;
    const zero_loss_scaler* loss_scaler;  /* device pointer or NULL */
} zero_adam_hparams;

/* ---------------------------------------------------------------- plan ---------- */

/* Build the sharding plan for rank `rank` of `nd` over parameters numels[0..n_params)
 * (host array, list order).  Follows [LLZ INIT] (pad each parameter to a multiple of Nd,
 * view as [Nd, -1], rank r keeps row r) with the formulas of [FR Implémentation
 * simplifiée], and [LLZ BWD] for buckets: walking the list in order, a bucket is closed
 * before a parameter whose padded_numel would take its total above bucket_bytes / 2
 * elements (one 16-bit gradient element = 2 bytes); a parameter larger than that gets a
 * bucket of its own; bucket_bytes = 0 puts everything in one bucket.  The per-parameter
 * tables are computed on the current HIP device by the planner kernels and copied back,
 * so this call synchronises.  dtype is a zero_dtype.
 * Errors: ZERO_EINVAL for n_params < 1, nd < 1, nd > 65535, rank outside [0, nd),
 * numel < 0, bucket_bytes < 0, bad dtype or out == NULL; ZERO_ERANGE when the padded
 * total exceeds 2^62 or a parameter reaches 2^48 elements; ZERO_ENOMEM / ZERO_EHIP.
 * On failure *out is set to NULL. */
zero_status zero_plan_create(const int64_t* numels, int64_t n_params, int32_t nd, int32_t rank,
                             int64_t bucket_bytes, int32_t dtype, zero_plan** out);

/* zero_plan_create with parameter groups [Z3: ZeRO-3 gathers, uses and frees the parameters
 * one layer at a time]: groups[i] is parameter i's group id (any int32; host array), and a
 * bucket is also closed before every parameter whose id differs from its predecessor's, so
 * every bucket lies inside one run of equal ids; inside a run the capacity rule above holds.
 * With one bucket per layer, a layer's gather is zero_unpack of its bucket and its
 * reduce-scatter is zero_pack_bucket + zero_reduce_shard.  groups == NULL is zero_plan_create.
 * Errors: as zero_plan_create. */
zero_status zero_plan_create_grouped(const int64_t* numels, const int32_t* groups, int64_t n_params, int32_t nd,
                                     int32_t rank, int64_t bucket_bytes, int32_t dtype, zero_plan** out);

/* Free a plan (NULL is a no-op).  Call only after work using it has finished. */
void zero_plan_destroy(zero_plan* plan);

zero_status zero_plan_get_summary(const zero_plan* plan, zero_plan_summary* out);
zero_status zero_plan_param_info(const zero_plan* plan, int64_t i, zero_param_info* out);
zero_status zero_plan_bucket_info(const zero_plan* plan, int64_t b, zero_bucket_info* out);

/* Model-state bytes per device for mixed-precision Adam over psi parameters at nd ranks
 * [ZP model states; ZeRO-DP stages]: stage 0 (plain data parallel) 16*psi; stage 1
 * (optimizer states partitioned) 4*psi + 12*psi/nd; stage 2 (+ gradients) 2*psi +
 * 14*psi/nd; stage 3 (+ parameters) 16*psi/nd.  ZERO_EINVAL for stage outside 0..3,
 * nd < 1, psi < 0 or out == NULL. */
zero_status zero_model_state_bytes(double psi, double nd, int32_t stage, double* out);

/* The same for the plan's padded total Psi and Nd. */
zero_status zero_plan_model_state_bytes(const zero_plan* plan, int32_t stage, double* out);

/* ---------------------------------------------------------------- hot path ------ */

/* Pack bucket b of one rank's gradients rank-major [LLZ BWD]: for every parameter i of
 * the bucket whose d_grad_ptrs[i] is not NULL (a NULL entry is a parameter without a
 * gradient this step, [LLZ Optim] layer drop) and every row k < Nd, column
 * bucket_col_i + j of row k receives element k*s_i + j of the gradient, or +0 where that
 * element is padding.  Columns of NULL parameters are not written; the row gap
 * [S_b, L_b) is written with zeros.  Bits are copied, not converted.
 *   d_grad_ptrs  device array of n_params pointers to 16-bit flat gradients (numel_i each)
 *   d_packed     device [Nd][L_b] 16-bit, 16-byte aligned
 * Errors: ZERO_EINVAL for a bad bucket index or NULL/misaligned pointers. */
zero_status zero_pack_bucket(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs,
                             void* d_packed, void* stream);

/* Reduce bucket b into rank r's fp32 shard: the arithmetic of a reduce-scatter
 * [LLZ BWD: reduce-scatter of the per-rank flat chunks; ZP stage Pos+g].  Row k
 * (k = 0..Nd-1) is virtual rank k's packed row r, at d_rows + k*row_stride elements.  For
 * every column c of a live parameter (d_live[i] != 0):
 *     acc = float(row_0[c]); for k = 1..Nd-1: acc = acc + float(row_k[c])   (fp32, RNE)
 *     d_g32[O_b + c] = acc
 * The 16-bit to fp32 conversions are exact (fp16 subnormals kept); the order is fixed,
 * so results are bit-reproducible.  Columns of dead parameters and the row gap are not
 * written.  If d_flag is not NULL, the call also ORs 1 into *d_flag when any written
 * value is inf or NaN (the fused overflow check); it never clears the flag.
 *   d_rows      device 16-bit, 16-byte aligned, (Nd-1)*row_stride + L_b elements;
 *               row_stride >= L_b and a multiple of 8
 *   d_live      device uint8[n_params]
 *   d_g32       device float[shard_numel], 16-byte aligned
 * Errors: ZERO_EINVAL for bad index, pointers, alignment or row_stride. */
zero_status zero_reduce_shard(const zero_plan* plan, int64_t b, const void* d_rows, int64_t row_stride,
                              const uint8_t* d_live, float* d_g32, int32_t* d_flag, void* stream);

/* OR 1 into *d_flag if any element of a live parameter's slice of d_g32 is inf or NaN.
 * The pages do not describe overflow handling; this is the usual mixed-precision guard
 * before the step.  Never clears the flag (the caller zeroes it once per step, and may
 * preset it to stand for another rank's overflow). */
zero_status zero_overflow_check(const zero_plan* plan, const float* d_g32, const uint8_t* d_live,
                                int32_t* d_flag, void* stream);

/* One mixed-precision Adam step over rank r's shard [LLZ Optim: each rank steps its own
 * p32 with the matching g; only parameters with a gradient take part], writing the
 * updated low-precision parameters into row r of every bucket's all-gather block
 * [Z3: the ZeRO-1/2 all-gather restores full updated parameters; FR ZeRO-1 step order].
 * If d_flag is not NULL and *d_flag != 0 the whole step is skipped: nothing is written
 * and step counts stay.  Otherwise, for every live parameter i: d_steps[i] += 1,
 * t = d_steps[i], and for every element e of its slice (fp32 arithmetic):
 *     g = g32[e] * grad_scale        (grad_scale / loss_scaler->scale with a dynamic scaler)
 *     m = beta1*m + (1-beta1)*g ;  v = beta2*v + (1-beta2)*g*g
 *     p32 -= (lr / (1-beta1^t)) * m / (sqrt(v) / sqrt(1-beta2^t) + eps)
 *     arena[Nd*O_b + r*L_b + (e - O_b)] = round_to_nearest_even_16(p32)
 * (the bias corrections are formed in double on the device and rounded to fp32 once).
 * Dead parameters and the row gaps are not touched.
 *   d_g32, d_p32, d_m, d_v   device float[shard_numel], 16-byte aligned
 *   d_live                   device uint8[n_params];  d_steps device int32[n_params]
 *   hp                       host pointer, read during the call
 *   d_arena                  device 16-bit [Nd * shard_numel], 16-byte aligned
 * Errors: ZERO_EINVAL for NULL/misaligned pointers (hp->loss_scaler 4-byte aligned if set) or
 * hyperparameters that are not finite (lr, eps, grad_scale) or betas outside [0, 1). */
zero_status zero_adam_step(const zero_plan* plan, const float* d_g32, float* d_p32, float* d_m, float* d_v,
                           const uint8_t* d_live, int32_t* d_steps, const zero_adam_hparams* hp,
                           const int32_t* d_flag, void* d_arena, void* stream);

/* Unpack bucket b's gathered block back to per-parameter flats without the padding
 * [Z3 ZeRO-1/2 all-gather; FR Implémentation simplifiée: parameter sync after the
 * step]: element e < numel_i of parameter i receives column bucket_col_i + (e mod s_i) of
 * row e / s_i.  Parameters whose d_param_ptrs[i] is NULL are skipped.
 *   d_gathered    device [Nd][L_b] 16-bit, 16-byte aligned (e.g. arena + Nd*O_b)
 *   d_param_ptrs  device array of n_params pointers to 16-bit flats (numel_i each) */
zero_status zero_unpack(const zero_plan* plan, int64_t b, const void* d_gathered, void* const* d_param_ptrs,
                        void* stream);

/* Initialise rank r's fp32 master shard from full flat parameters [LLZ INIT: pad each
 * parameter, view it as [Nd, -1] and clone row r as p32; FR Implémentation simplifiée: the
 * padding is zeros]: d_p32[shard_offset_i + j] = src_i[shard_start_i + j] when that index is
 * below numel_i, else +0; the row gaps are set to +0.  Parameters whose d_src_ptrs[i] is NULL
 * are left as they were.
 *   d_src_ptrs  device array of n_params pointers to flat parameters
 *   src_dtype   0 = fp32 sources, ZERO_BF16 / ZERO_FP16 = 16-bit sources (converted exactly)
 *   d_p32       device float[shard_numel], 16-byte aligned */
zero_status zero_shard_init(const zero_plan* plan, const void* const* d_src_ptrs, int32_t src_dtype, float* d_p32,
                            void* stream);

/* ------------------------------------------------- allocation-free Adam step ------ */

/* Largest plan (in parameters) that zero_adam_step_noalloc serves. */
#define ZERO_ADAM_NOALLOC_MAX_PARAMS 131072

/* zero_adam_step for callers that cannot allocate device memory or use the plan's scratch
 * (code under graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and the same results, bit for bit, but the per-parameter step sizes and the
 * fp32 hyperparameters are staged in a static device array of 1 MiB + 256 bytes
 * (ZERO_ADAM_NOALLOC_MAX_PARAMS * 8 + 256) that the library holds on every GPU it runs on
 * until the process ends.  The call allocates nothing and calls no allocating routine; its
 * first use on a device looks up the array's address there (hipGetSymbolAddress).  Every
 * call on one GPU shares that GPU's array, which keeps the last call's contents (every value
 * a step reads is written earlier in the same step): calls that overlap in time on one GPU
 * -- on different streams, or from different plans -- race and must not be issued.
 * Arguments and errors as zero_adam_step, plus ZERO_ERANGE when the plan has more than
 * ZERO_ADAM_NOALLOC_MAX_PARAMS parameters (nothing is launched). */
zero_status zero_adam_step_noalloc(const zero_plan* plan, const float* d_g32, float* d_p32, float* d_m, float* d_v,
                                   const uint8_t* d_live, int32_t* d_steps, const zero_adam_hparams* hp,
                                   const int32_t* d_flag, void* d_arena, void* stream);

/* ------------------------------------------- fused path: reduce + check + Adam ------ */
/* The same step with the reduced gradient kept on chip (in registers, or in the block's LDS
 * for a tile inside one parameter): the sum of the Nd rows goes straight into the Adam update,
 * so the fp32 gradient shard is neither written nor read.
 * Because the step must be skipped before any state changes, the overflow verdict comes
 * from the inputs rather than from the sums.  Per step, on one stream:
 *   1. *d_flag = 0; zero_pack_bucket_check for every bucket (this rank's gradients);
 *   2. the ranks OR their flags (an all-reduce of one int; nothing to do on one process);
 *   3. zero_adam_prepare (step counts and step sizes, or nothing if the flag is set);
 *   4. per bucket, once its rows have arrived: zero_reduce_adam_bucket.
 * With the flag clear, p32, m, v, the step counts and the 16-bit parameters are
 * bit-identical to zero_reduce_shard + zero_adam_step on the same rows. */

/* zero_pack_bucket, and OR 1 into *d_flag when a gradient element that the call reads is
 * inf or NaN or has |x| > 2^126 / Nd.  Below that bound no fp32 sum of Nd such values can
 * overflow: with rounding, a partial sum of k terms stays below k * (2^126 / Nd) *
 * (1 + 2^-24)^k < 2^126 * 1.004 < 2^128 for every Nd a plan allows (Nd <= 65535), so a flag
 * that is clear on every rank means every reduced sum is finite.  The comparison is exact:
 * the threshold is the largest 16-bit magnitude whose value times Nd is at most 2^126.  A
 * finite value above the bound flags the step although the sums might not overflow: a conservative skip, which
 * needs |g| near 2^126 / Nd (never reached by fp16; for bf16 a scaled gradient already
 * beyond any usable loss scale).  Never clears the flag.
 *   d_flag   device int32
 * Errors: as zero_pack_bucket, and ZERO_EINVAL for d_flag == NULL. */
zero_status zero_pack_bucket_check(const zero_plan* plan, int64_t b, const void* const* d_grad_ptrs,
                                   void* d_packed, int32_t* d_flag, void* stream);

/* The first launch of zero_adam_step on its own: if d_flag is NULL or *d_flag == 0, every
 * live parameter's step count advances and its step size lr / (1 - beta1^t) and
 * 1 / sqrt(1 - beta2^t) are stored in the plan (double, rounded to fp32 once), with the fp32
 * hyperparameters; if the flag is set, nothing changes.  The stored values serve the
 * zero_reduce_adam_bucket calls that follow on the same stream; the plan holds one set, so
 * do not interleave two steps of one plan on different streams.
 * Errors: ZERO_EINVAL as for zero_adam_step. */
zero_status zero_adam_prepare(const zero_plan* plan, const uint8_t* d_live, int32_t* d_steps,
                              const zero_adam_hparams* hp, const int32_t* d_flag, void* stream);

/* Reduce bucket b and take the Adam step on its columns in one pass [LLZ BWD reduce-scatter,
 * then LLZ Optim on the matching shard; Z3 ZeRO-1/2 all-gather row]: for every column c of a
 * live parameter of the bucket, acc is formed as in zero_reduce_shard and used as g32 in the
 * update of zero_adam_step, which writes p32, m, v at O_b + c and the 16-bit parameter at
 * arena[Nd*O_b + r*L_b + c].  Dead parameters and the row gap are not touched.  If d_flag is
 * not NULL and *d_flag != 0 nothing is written.  Needs zero_adam_prepare earlier on the same
 * stream in this step, with the same d_live and d_flag.
 *   d_rows, row_stride   as zero_reduce_shard
 *   d_p32, d_m, d_v      device float[shard_numel], 16-byte aligned
 *   d_arena              device 16-bit [Nd * shard_numel], 16-byte aligned
 * Errors: ZERO_EINVAL for bad index, NULL/misaligned pointers or row_stride. */
zero_status zero_reduce_adam_bucket(const zero_plan* plan, int64_t b, const void* d_rows, int64_t row_stride,
                                    const uint8_t* d_live, float* d_p32, float* d_m, float* d_v,
                                    const int32_t* d_flag, void* d_arena, void* stream);

/* ------------------------------------------------------- ZeRO-3 layer step ------ */

/* One launch holding up to three independent pieces of ZeRO-3's per-layer traffic [Z3: each
 * layer's parameters are all-gathered before it runs and freed after it; in the backward pass,
 * layers L-1 .. 0, each layer's gradients are reduce-scattered once its backward has run]:
 *   reduce_b >= 0:  zero_reduce_shard(plan, reduce_b, d_rows, row_stride, d_live, d_g32, d_flag)
 *   pack_b   >= 0:  zero_pack_bucket(plan, pack_b, d_grad_ptrs, d_packed), or with check != 0
 *                   zero_pack_bucket_check(..., d_flag)
 *   gather_b >= 0:  zero_unpack(plan, gather_b, d_gathered, d_param_ptrs)
 * (-1 = that piece is absent; its pointers are not read).  Each piece computes exactly what its
 * own entry point computes, with the same arguments, errors and conventions; the pieces share
 * the grid and run concurrently, so no piece may read or write what another writes.  With one
 * bucket per layer (zero_plan_create_grouped), a backward step of layer l is reduce_b = l + 1,
 * pack_b = l, gather_b = l - 1: the reduce reads rows packed one step earlier, the pack reads the
 * gradients layer l just produced, the gather fills the scratch that layer l no longer needs --
 * one launch (and one launch tail) per layer instead of three.
 * Errors: as the three entry points (the first failing piece's), and ZERO_EINVAL for an index
 * below -1. */
zero_status zero_z3_layer_step(const zero_plan* plan, int64_t reduce_b, const void* d_rows, int64_t row_stride,
                               const uint8_t* d_live, float* d_g32, int64_t pack_b, const void* const* d_grad_ptrs,
                               void* d_packed, int32_t check, int64_t gather_b, const void* d_gathered,
                               void* const* d_param_ptrs, int32_t* d_flag, void* stream);

/* Most buckets in one piece of a zero_z3_step call. */
#define ZERO_Z3_MAX_BUCKETS 4

/* The pieces of one zero_z3_step launch: up to ZERO_Z3_MAX_BUCKETS consecutive buckets of each
 * kind.  A count of 0 leaves the kind out (its fields are not read).  Host struct, read during
 * the call; the pointers in it are device pointers. */
typedef struct zero_z3_pieces {
    int64_t reduce_b0, reduce_n;                  /* reduce buckets [reduce_b0, reduce_b0 + reduce_n) */
    const void* rows[ZERO_Z3_MAX_BUCKETS];        /* rows of bucket reduce_b0 + j (zero_reduce_shard's d_rows) */
    int64_t row_stride[ZERO_Z3_MAX_BUCKETS];      /* and its row stride */
    const uint8_t* live;                          /* as zero_reduce_shard */
    float* g32;                                   /* as zero_reduce_shard */
    int64_t pack_b0, pack_n;                      /* pack buckets [pack_b0, pack_b0 + pack_n) */
    const void* const* grad_ptrs;                 /* as zero_pack_bucket */
    void* packed[ZERO_Z3_MAX_BUCKETS];            /* packed block of bucket pack_b0 + j */
    int32_t check;                                /* != 0: the checked pack (zero_pack_bucket_check) */
    int64_t gather_b0, gather_n;                  /* unpack buckets [gather_b0, gather_b0 + gather_n) */
    const void* gathered[ZERO_Z3_MAX_BUCKETS];    /* all-gather block of bucket gather_b0 + j */
    void* const* param_ptrs;                      /* as zero_unpack */
    int32_t* flag;                                /* overflow flag of the reduces and the checked packs */
} zero_z3_pieces;

/* zero_z3_layer_step over ranges of buckets [Z3: the forward pass gathers layers in order and
 * the backward pass goes back through them, reduce-scattering each layer's gradients once its
 * backward has run; consecutive layers can be handled together]: every bucket of every piece
 * computes exactly what its own entry point computes (zero_reduce_shard, zero_pack_bucket or
 * zero_pack_bucket_check, zero_unpack) with that bucket's pointers from *pieces; all buckets
 * share one grid and run concurrently, so no bucket's work may read or write what another's
 * writes.  With one bucket per layer and k layers per step, a backward step packs layers
 * [l, l + k), gathers [l - k, l) and reduces [l + k, l + 2k); a forward step gathers k layers.
 * Errors: ZERO_EINVAL for NULL pieces, a count outside 0 .. ZERO_Z3_MAX_BUCKETS, a range
 * outside [0, n_buckets), or whatever a bucket's own entry point rejects (nothing is launched
 * then). */
zero_status zero_z3_step(const zero_plan* plan, const zero_z3_pieces* pieces, void* stream);

/* ------------------------------------------------------- dynamic loss scaling ------ */

/* Write the host configuration *cfg (every field, good_steps and overflows included) to the
 * device scaler d_scaler, in stream order.  *cfg is read during the call.
 * Errors: ZERO_EINVAL for NULL or misaligned pointers, or a configuration outside the
 * ranges stated in zero_loss_scaler. */
zero_status zero_loss_scaler_init(const zero_loss_scaler* cfg, zero_loss_scaler* d_scaler, void* stream);

/* After a step: apply the rule of zero_loss_scaler to d_scaler from the step's overflow flag
 * *d_flag (read on the device; the flag is not changed).  Call once per step, after the Adam
 * launches that read the scale, before the flag is cleared for the next step.
 * Errors: ZERO_EINVAL for NULL or misaligned pointers. */
zero_status zero_loss_scaler_update(const int32_t* d_flag, zero_loss_scaler* d_scaler, void* stream);

/* Thread-local text of the last error ("" if none). */
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_SHARD_H */
