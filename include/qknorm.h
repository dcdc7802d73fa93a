/*
 * qknorm.h -- C ABI of the MI355X (gfx950) layerwise QK-Norm library.
 *
 * Layerwise QK-Norm is RMSNorm over the FULL projected Q and K vector of
 * each token: one factor per vector, from the sum of squares over all H
 * columns, then an elementwise scale by gamma:
 *
 *   y[t][j] = x[t][j] / sqrt( (1/H) * sum_j x[t][j]^2 + eps ) * gamma[j]
 *
 * ("SwiftQK: Fast and Communication-Efficient Tensor Parallelism for
 * Query-Key Normalization", Section II-A, Eq. (1).) Q and K are two
 * independent normalisations (Fig. 1(a): one Norm per tensor) executed in one
 * fused pass.
 *
 * The library computes it with the letter's decomposition (Section III,
 * Algorithm 1): the hidden dimension is split into n_shards contiguous
 * column blocks ("logical shards"); each shard reduces only a scalar fp32
 * partial sum of squares (Phase A); the partials are exchanged and combined
 * in ascending shard order while the independent x*gamma product proceeds
 * (Phase B); the combined factor scales the product (Phase C). All shards run
 * on one GPU: the shards of a token tile are workgroups of one persistent,
 * co-resident grid that exchange their scalars through device memory.
 *
 * Conventions for every entry point:
 *  - Tensors are device pointers, row-major [T][H] with row stride H
 *    elements, contiguous; gamma is [H]. bf16 means IEEE binary32 truncated
 *    to its upper 16 bits (stored as 16-bit words); f32 is IEEE binary32;
 *    e4m3 is the OCP 8-bit floating point E4M3 encoding (one byte: sign,
 *    4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111
 *    is NaN; largest finite magnitude 448). The caller owns every tensor it
 *    passes.
 *  - Calls are asynchronous and stream-ordered on `stream` (0 = the null
 *    stream of the current device); pointers must belong to the current
 *    device. Nothing is synchronised except where stated.
 *  - Argument errors are detected synchronously and launch nothing.
 *    Return value: QKN_OK (0) or a negative qknorm_status.
 *  - T == 0 is a no-op returning QKN_OK.
 *  - An output may alias its own input exactly (in place); any other
 *    overlap between an output and an input or another output is
 *    QKN_EOVERLAP.
 *  - 16-byte aligned pointers with (H / n_shards) * elem_size a multiple of
 *    16 bytes take 128-bit memory paths; other layouts are still correct.
 *  - Rounding to a 16-bit or 8-bit output is to nearest, ties to even. An
 *    e4m3 output saturates magnitudes above 448 (infinities included) to
 *    +-448 and keeps NaN.
 */
#ifndef QKNORM_H
#define QKNORM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qknorm_status {
    QKN_OK = 0,
    QKN_EINVAL = -1,     /* bad argument: null pointer, T < 0, H < 1,
                            n_shards outside [1, QKN_MAX_SHARDS],
                            H % n_shards != 0, eps negative or not finite */
    QKN_EOVERLAP = -2,   /* an output partially overlaps an input/output */
    QKN_ENOMEM = -3,     /* the library could not allocate its workspace */
    QKN_EHIP = -4,       /* a HIP runtime call or launch failed */
    QKN_ERESIDENCY = -5, /* not even n_shards workgroups can be co-resident */
    QKN_ETIMEOUT = -6,   /* (qknorm_check_fault) a shard exchange timed out */
    QKN_ECAPTURE = -7,   /* fused call under graph capture with the cooperative
                            launch option (not recordable) */
    QKN_ESCRATCH = -8    /* (qknorm_layerwise_fwd_bf16_noalloc) the launch needs more
                            exchange slots than the static scratch holds */
} qknorm_status;

typedef enum qknorm_dtype { QKN_BF16 = 0, QKN_F32 = 1, QKN_E4M3 = 2 } qknorm_dtype;

/* Formats of the fused and split kernels: input x / scale gamma / output y.
 * The `dtype` argument of the planning, occupancy and measurement calls
 * below is a format; formats 0 and 1 are QKN_BF16 and QKN_F32 throughout. */
enum {
    QKN_FMT_BF16 = 0,       /* bf16 / bf16 / bf16 */
    QKN_FMT_F32 = 1,        /* f32 / f32 / f32 */
    QKN_FMT_E4M3_BF16 = 2,  /* e4m3 / bf16 / bf16 */
    QKN_FMT_E4M3_E4M3 = 3,  /* e4m3 / bf16 / e4m3 */
    QKN_FMT_LN_BF16 = 4,    /* LayerNorm, bf16 / bf16 (gamma, beta) / bf16 */
    QKN_FMT_LN_F32 = 5,     /* LayerNorm, f32 / f32 (gamma, beta) / f32 */
    QKN_NUM_FORMATS = 6
};

/* Up to 64 logical shards. The fused kernel's exchange wave holds shards x
 * segments x statistics <= 64 slots: mixed Q+K tiles (two segments per token)
 * take at most 32 shards, single-tensor tiles of one row up to 64 (RMSNorm);
 * other wide splits run the split kernels from the same entry point. */
#define QKN_MAX_SHARDS 64

/* ------------------------------------------------------------------ fused
 * Fused Q+K layerwise RMSNorm (Algorithm 1, Phases A-C, persistent grid of
 * Section III-D). q [T][Hq], k [T][Hk], gamma_q [Hq], gamma_k [Hk] in, out_q
 * [T][Hq], out_k [T][Hk] out, all of the suffix dtype; fp32 accumulation.
 * n_shards must divide both Hq and Hk; shard s of Q and shard s of K belong
 * to the same logical rank. eps is added to the mean square inside the
 * square root.
 *
 * The library owns a small per-(device, stream) workspace (exchange slots,
 * fault word), allocated on first use and reused by later calls; calls on
 * different streams use different workspaces. A shard exchange that does not
 * complete within the spin limit (default 1 s) abandons the wait, leaves the
 * outputs unspecified and records a fault that qknorm_check_fault reports.
 *
 * Under stream capture a fused call allocates nothing and records two kernel
 * nodes: one that clears the exchange slots the launch uses, then the fused
 * kernel. Their scratch is a static per-device array reserved for recorded
 * launches (about 3 MiB), so every replay starts from cleared slots. Replays
 * of recorded fused launches that overlap in time on one device race on that
 * array; so do two graphs replayed concurrently. A recorded launch refused
 * for size (QKN_ESCRATCH) would need more than 2^18 slots. The cooperative
 * launch option is not recordable (QKN_ECAPTURE). The split path below is
 * capturable as well.
 */
int qknorm_layerwise_fwd_bf16(const void* q, const void* k, const void* gamma_q,
                              const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk,
                              int n_shards, float eps, void* out_q, void* out_k,
                              hipStream_t stream);
int qknorm_layerwise_fwd_f32(const void* q, const void* k, const void* gamma_q,
                             const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk,
                             int n_shards, float eps, void* out_q, void* out_k,
                             hipStream_t stream);

/* The bf16 fused call without any device allocation, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels, results and errors as
 * qknorm_layerwise_fwd_bf16, except that the exchange slots, the fault word
 * and the split fallback's statistics live in a static device array of the
 * library (2 MiB of slots, 256 B, 1 MiB of fp32 statistics; about 3 MiB per
 * device, held until the process ends) instead of a per-stream workspace:
 *  - No hipMalloc, hipFree or other device allocation is made. The first call
 *    on a device binds that device's copy of the array, clears it with a
 *    kernel on `stream` and synchronises `stream` once. Host-side bookkeeping
 *    (launch plans per shape) still lives in host memory.
 *  - Every call on one device shares that device's array. Calls on the same
 *    stream are ordered and safe; calls that overlap in time on one device
 *    (different streams) race on the slots and give unspecified results.
 *  - The 2^18 slots hold every launch the planner makes on a 256-CU device.
 *    A launch that needs more (a larger device, or the QKN_OPT_STATIC_SLOTS
 *    test limit) is refused with QKN_ESCRATCH before anything is launched.
 *    The split fallback (unaligned or very wide shards) runs over token
 *    chunks that fit the 1 MiB of statistics, so no token count is refused.
 *  - A timed-out exchange sets the device's static fault word, which
 *    qknorm_check_fault(stream) reports (and clears) like a workspace's.
 *  - Under stream capture it records, like the allocating call, a clearing
 *    kernel and the fused kernel on the array reserved for recorded launches. */
int qknorm_layerwise_fwd_bf16_noalloc(const void* q, const void* k, const void* gamma_q,
                                      const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk,
                                      int n_shards, float eps, void* out_q, void* out_k,
                                      hipStream_t stream);

/* The same for FP8 activations (the letter's FP8-E4M3 evaluation, Section
 * IV-C: FP32 accumulation for FP8-E4M3 inputs as for BF16): q and k are e4m3
 * codes, gamma_q and gamma_k are bf16, and out_q / out_k are `out_dtype`
 * (QKN_BF16 or QKN_E4M3; anything else is QKN_EINVAL). The 128-bit path
 * needs H / n_shards to be a multiple of 16. In place (out aliasing the
 * input) is only possible with out_dtype = QKN_E4M3. */
int qknorm_layerwise_fwd_e4m3(const void* q, const void* k, const void* gamma_q,
                              const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk,
                              int n_shards, float eps, void* out_q, void* out_k,
                              int out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------ LayerNorm
 * The same decomposition applied to LayerNorm (the reading notes' extension,
 * Section 5e): mean and variance of the full vector follow from two additive
 * statistics per shard, sum x and sum x^2, exchanged and combined (ascending
 * shard order) like the RMSNorm partial while x*gamma proceeds:
 *
 *   mu = S1 / H,  var = max(S2 / H - mu^2, 0),  rstd = 1 / sqrt(var + eps),
 *   y[t][j] = (x[t][j] - mu) * rstd * gamma[j] + beta[j]
 *
 * computed as (x*gamma)*rstd + (beta - mu*rstd*gamma) in fp32. Arguments as
 * for the fused RMSNorm entry points, plus beta_q [Hq] and beta_k [Hk] in the
 * suffix dtype; a null beta means no shift. Shards of one token exchange
 * 2 x 2 x n_shards scalars, so the fused kernel holds at most 16 shards (more
 * run the split kernels below from the same entry point). The variance is
 * formed from the two sums in fp32: rows whose mean is large against their
 * spread lose relative accuracy in rstd (cancellation in S2/H - mu^2).
 */
int qknorm_layernorm_fwd_bf16(const void* q, const void* k, const void* gamma_q,
                              const void* gamma_k, const void* beta_q, const void* beta_k,
                              int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                              void* out_q, void* out_k, hipStream_t stream);
int qknorm_layernorm_fwd_f32(const void* q, const void* k, const void* gamma_q,
                             const void* gamma_k, const void* beta_q, const void* beta_k,
                             int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                             void* out_q, void* out_k, hipStream_t stream);

/* LayerNorm split into three launches for one tensor:
 * qknorm_shard_stats_*: sums[s * T + t] and sumsq[s * T + t], fp32 [n_shards][T]
 *   each, over shard s's columns.
 * qknorm_combine_stats: mean[t] and rstd[t] (fp32 [T]) from them, as above.
 * qknorm_apply_norm_*: out = (x*gamma)*rstd + (beta - mean*rstd*gamma); beta may
 *   be null. */
int qknorm_shard_stats_bf16(const void* x, int64_t T, int64_t H, int n_shards, float* sums,
                            float* sumsq, hipStream_t stream);
int qknorm_shard_stats_f32(const void* x, int64_t T, int64_t H, int n_shards, float* sums,
                           float* sumsq, hipStream_t stream);
int qknorm_combine_stats(const float* sums, const float* sumsq, int64_t T, int64_t H,
                         int n_shards, float eps, float* mean, float* rstd, hipStream_t stream);
int qknorm_apply_norm_bf16(const void* x, const void* gamma, const void* beta,
                           const float* mean, const float* rstd, int64_t T, int64_t H,
                           void* out, hipStream_t stream);
int qknorm_apply_norm_f32(const void* x, const void* gamma, const void* beta,
                          const float* mean, const float* rstd, int64_t T, int64_t H,
                          void* out, hipStream_t stream);

/* ------------------------------------------------------------------ headwise
 * Headwise QK-Norm ("SwiftQK", Section II-A): one factor per attention head
 * instead of one per full vector. Row t of q holds heads_q heads of head_dim
 * columns (head h = columns [h*head_dim, (h+1)*head_dim)), and likewise k;
 * gamma_q and gamma_k are [head_dim], each shared by all heads of its tensor:
 *
 *   y[t][h*D + j] = x[t][h*D + j] / sqrt((1/D) sum_{i<D} x[t][h*D+i]^2 + eps) * gamma[j]
 *
 * When tensor parallelism splits the heads (not the columns of a head) across
 * ranks, no shard exchange is needed: this is the method's degenerate case,
 * one streaming pass with the reduction inside each head's lanes, and it takes
 * no shard count. Conventions as above (in place allowed, T == 0 no-op). The
 * 128-bit path needs 16-byte aligned pointers and a head of 1, 2, 4, ... or 64
 * 16-byte vectors (bf16 head_dim 8..512, f32 4..256); other shapes are still
 * correct (one wave per head).
 */
int qknorm_headwise_fwd_bf16(const void* q, const void* k, const void* gamma_q,
                             const void* gamma_k, int64_t T, int64_t heads_q, int64_t heads_k,
                             int64_t head_dim, float eps, void* out_q, void* out_k,
                             hipStream_t stream);
int qknorm_headwise_fwd_f32(const void* q, const void* k, const void* gamma_q,
                            const void* gamma_k, int64_t T, int64_t heads_q, int64_t heads_k,
                            int64_t head_dim, float eps, void* out_q, void* out_k,
                            hipStream_t stream);

/* ------------------------------------------------------------------ split
 * The same computation for one tensor as three stream-ordered launches, with
 * the intermediate statistics in caller-owned device buffers (the unfused
 * "scalar aggregation, then normalise" order the letter compares against,
 * Section IV-A).
 *
 * qknorm_shard_sumsq_*: Phase A. partials [n_shards][T] fp32, shard-major
 *   (partials[s * T + t] = sum of x[t][j]^2 over shard s's columns).
 * qknorm_combine_scale: Phase B combine. rms_inv[t] =
 *   1 / sqrt( (sum_{s=0}^{n_shards-1} partials[s*T+t]) / H + eps ), the sum in
 *   fp32 in ascending s. rms_inv is [T] fp32.
 * qknorm_apply_scale_*: Phases B (x*gamma) and C. out[t][j] =
 *   round(x[t][j] * gamma[j] * rms_inv[t]) in the suffix dtype (for e4m3
 *   inputs: in out_dtype, with gamma in bf16).
 */
int qknorm_shard_sumsq_bf16(const void* x, int64_t T, int64_t H, int n_shards,
                            float* partials, hipStream_t stream);
int qknorm_shard_sumsq_f32(const void* x, int64_t T, int64_t H, int n_shards,
                           float* partials, hipStream_t stream);
int qknorm_shard_sumsq_e4m3(const void* x, int64_t T, int64_t H, int n_shards,
                            float* partials, hipStream_t stream);
int qknorm_combine_scale(const float* partials, int64_t T, int64_t H, int n_shards,
                         float eps, float* rms_inv, hipStream_t stream);
int qknorm_apply_scale_bf16(const void* x, const void* gamma, const float* rms_inv,
                            int64_t T, int64_t H, void* out, hipStream_t stream);
int qknorm_apply_scale_f32(const void* x, const void* gamma, const float* rms_inv,
                           int64_t T, int64_t H, void* out, hipStream_t stream);
/* e4m3 x, bf16 gamma, out of `out_dtype` (QKN_BF16 or QKN_E4M3). */
int qknorm_apply_scale_e4m3(const void* x, const void* gamma, const float* rms_inv,
                            int64_t T, int64_t H, void* out, int out_dtype,
                            hipStream_t stream);

/* ------------------------------------------------------------------ service */

/* Synchronises `stream`, then reports and clears the fault words of that
 * stream's workspace, of the current device's static scratch arrays (the
 * no-allocation call's and the recorded launches') and the device's timeout
 * flag: QKN_OK, QKN_ETIMEOUT (any was set), or QKN_EHIP. */
int qknorm_check_fault(hipStream_t stream);

/* Whether a fused launch on the current device has timed out since the last
 * qknorm_check_fault, without synchronising anything: 1 or 0. A launch sets
 * the device's flag (a word of pinned host memory) when it abandons an
 * exchange, so this turns 1 once that launch has reached its timeout; launches
 * still running are not seen. The flag exists from the first fused call made
 * outside stream capture; launches recorded under capture do not set it (their
 * timeouts are reported by qknorm_check_fault only). */
int qknorm_fault_pending(void);

/* Host address of the current device's timeout flag (allocated here if needed;
 * NULL if pinned memory is unavailable): nonzero once a fused launch timed out,
 * cleared by qknorm_check_fault. Lets a binding poll it without a call. */
const uint32_t* qknorm_fault_flag(void);

/* Static English text for a status code (never NULL). */
const char* qknorm_strerror(int status);

/* Text of the last HIP error the calling thread saw inside the library, or
 * "" (thread-local, valid until the thread's next library call). */
const char* qknorm_last_hip_error(void);

/* Workgroups of the fused kernel that the current device can hold at once
 * for this format (QKN_FMT_*) and shape (occupancy x compute units); *out
 * receives it. */
int qknorm_max_coresident_workgroups(int dtype, int64_t Hq, int64_t Hk, int n_shards,
                                     int* out);

/* Occupancy of the current device for format `dtype` (QKN_FMT_*):
 * blocks_per_cu[v * (QKN_MAX_DATA_WAVES + 1)
 * + w] = workgroups of fused variant v with w data waves that one compute
 * unit can hold (0 = not launchable), an array of QKN_NUM_VARIANTS x
 * (QKN_MAX_DATA_WAVES + 1) ints; *cu_count = compute units. Feeds
 * qknorm_plan_fused with the numbers the library itself plans with. A variant
 * built for single-tensor tiles only (10) reports that kernel's occupancy. */
int qknorm_device_occupancy(int dtype, int* blocks_per_cu, int* cu_count);

/* Frees every workspace the library allocated (all devices and streams).
 * The caller must ensure no library work is still in flight. */
int qknorm_release_workspace(void);

/* Host-only launch planning, exposed for tests and tools. Fills *plan for a
 * device with `cu_count` compute units, of which each holds
 * `blocks_per_cu[v * (QKN_MAX_DATA_WAVES + 1) + w]` workgroups of kernel
 * variant v with w data waves (the layout of qknorm_device_occupancy; the
 * real path queries the occupancy API). Variants 0-5 hold 1, 2, 3, 4, 6, 9
 * 16-byte vectors per data thread (5: fp32 only) and scale a tile one
 * iteration after reducing it; variants 6-9 hold 1, 2, 3, 4 and scale it two
 * iterations later, which decouples the shards of a group further; variant 10
 * (bf16 on single-tensor tiles only, at most four data waves: one per SIMD
 * with the exchange wave) holds 5 with the two-iteration lag and is planned
 * only by the tuned table or QKN_OPT_FORCE_VARIANT. The e4m3
 * formats have variants 0, 1, 2, 6 and 7 (a 16-byte vector is 16 columns);
 * the LayerNorm formats have all but variant 5.
 * A tile is `rows` tokens of Q and of K (mixed layout), or, with Hq == Hk,
 * `rows` rows of one tensor (single-tensor layout, st = 1: the first
 * ceil(T/rows) tiles hold Q's rows, the rest K's, so that every access of an
 * iteration falls in one tensor; up to 8 rows). Measured launches of the
 * prefill-sized shards use the single-tensor layout where it was faster; the
 * scoring rule plans mixed tiles, and moves streaming RMSNorm launches (bf16,
 * fp32) of shards split 4 to 8 ways to single-tensor tiles of twice the
 * rows, unless QKN_OPT_TILE_LAYOUT asks otherwise.
 * Here the single-tensor kernels are taken to occupy the device like the mixed
 * ones (the real path queries both).
 * `dtype` is a format (QKN_FMT_*). */
#define QKN_NUM_VARIANTS 11
#define QKN_MAX_DATA_WAVES 15
typedef struct qknorm_plan {
    int variant;        /* fused kernel variant, or -1: shape uses the split kernels */
    int threads;        /* workgroup size: 64 x (data_waves + 1) */
    int data_waves;     /* data waves per workgroup (one more wave exchanges) */
    int slots;          /* 16-byte vectors per data thread */
    int rows;           /* tokens per tile (single-tensor layout: rows of one tensor) */
    int64_t n_tiles;    /* ceil(T / rows); twice that in the single-tensor layout */
    int n_groups;       /* workgroup groups; each group = n_shards workgroups */
    int grid;           /* n_groups * n_shards */
    int xcd_map;        /* 1: members of a group share blockIdx % 8 */
    int iters;          /* tiles per group (ceil(n_tiles / n_groups)) */
    int st;             /* 1: single-tensor tiles; 0: mixed Q+K tiles */
    int pace_gbs;       /* pacing rate in GB/s (0: none; see QKN_OPT_PACE for the
                           kernels that have one): no workgroup passes its k-th
                           barrier before k periods after its start, one period being
                           the time the whole grid's tile bytes of one iteration take
                           at that rate (launches of more than two iterations). The
                           staggered builds (bf16 variant 10, E4M3 -> bf16 variant 7
                           and LayerNorm bf16 variant 7 on single-tensor tiles,
                           LayerNorm bf16 variant 7 on mixed tiles) start group g's
                           first loads a lead (5/8 of a period for bf16 RMSNorm,
                           3/8 for E4M3 -> bf16, one period for LayerNorm) plus g / n_groups
                           of a period after entry and count barrier k's period from
                           barrier 0, so tiles are loaded in tile order; their drain
                           barriers are not held */
} qknorm_plan;
int qknorm_plan_fused(int dtype, int64_t T, int64_t Hq, int64_t Hk, int n_shards,
                      int cu_count, const int* blocks_per_cu, int aligned,
                      qknorm_plan* plan);

/* Tuning and test options (process-wide, not thread-safe against running
 * calls). Keys: */
enum {
    QKN_OPT_SPIN_LIMIT_NS = 1,  /* exchange spin budget in ns (default 1e9) */
    QKN_OPT_FORCE_VARIANT = 2,  /* -1 = planner's choice, else a variant id */
    QKN_OPT_ROWS = 3,           /* 0 = planner's choice, else rows per tile (<= 4; single-tensor
                                   tiles <= 8) */
    QKN_OPT_XCD_MAP = 4,        /* -1 = planner's choice (a group's members on one XCD,
                                   except for the tuned launches measured faster
                                   without and for streaming fp32 shards split
                                   4-8 ways and bf16 shards split 4 ways with
                                   rows of at least 1 KiB), 0 = off, 1 = on when
                                   possible */
    QKN_OPT_COOPERATIVE = 5,    /* 1 = hipLaunchCooperativeKernel, 0 = plain */
    QKN_OPT_MAX_GROUPS = 6,     /* 0 = no cap, else cap on workgroup groups */
    QKN_OPT_FORCE_SPLIT = 7,    /* 1 = fused entry points run the split kernels */
    QKN_OPT_DATA_WAVES = 9,     /* 0 = planner's choice, else data waves per workgroup */
    QKN_OPT_SPLIT_VECTORS = 10, /* 0 = library's choice, else 1, 2, 4 or 8: 16-byte vectors
                                   each thread of the split kernels' 16-byte paths loads
                                   at once (the apply kernels take at most 4) */
    QKN_OPT_TILE_LAYOUT = 11,   /* 0 = planner's choice, 1 = mixed Q+K tiles only,
                                   2 = single-tensor tiles wherever allowed */
    QKN_OPT_WPC = 12,           /* 0 = planner's choice, else workgroups per CU the
                                   planner's search must use (launch timing) */
    QKN_OPT_PACE = 14,          /* -1 = planner's choice (the tuned launches measured
                                   faster paced), 0 = no pacing, else a pacing rate in
                                   GB/s (qknorm_plan.pace_gbs) for launches whose kernel
                                   has a paced build: bf16 variant 8 on mixed tiles and
                                   variant 10 on single-tensor tiles (staggered:
                                   see qknorm_plan.pace_gbs), E4M3 -> bf16 variants 0
                                   (single-tensor tiles) and 7 (mixed; single-tensor
                                   tiles: staggered), E4M3 -> E4M3
                                   variant 7 (single-tensor), LayerNorm bf16 variant 7
                                   (both layouts, staggered) */
    QKN_OPT_STATIC_SLOTS = 13,  /* test hook: 0 = the no-allocation call may use all of
                                   its static slots, else at most this many (so that
                                   QKN_ESCRATCH can be exercised) */
    QKN_OPT_TEST_SKIP_PUBLISH = 8 /* test hook: 1 = fused workgroups never publish
                                     their partial, so every exchange with n_shards
                                     > 1 ends at the spin limit (kernel still exits) */
};
int qknorm_set_option(int key, int64_t value);
int64_t qknorm_get_option(int key);

/* Bandwidth ceiling for measurements: copies q -> out_q and k -> out_k
 * (bytes_q, bytes_k bytes) with a one-shot grid of one-wave workgroups, each
 * thread moving one 16-byte vector (the fastest simple pattern measured on
 * this part). Pointers must be 16-byte aligned; an output overlapping any
 * input or the other output is QKN_EOVERLAP; a tensor above 2^31 - 2^16
 * bytes is QKN_EINVAL. */
int qknorm_bench_copy(const void* q, const void* k, void* out_q, void* out_k,
                      int64_t bytes_q, int64_t bytes_k, hipStream_t stream);

/* Bandwidth ceiling for byte mixes that write twice what they read (E4M3
 * inputs with bf16 outputs): every byte of q (bytes_q of them) becomes one
 * 16-bit word of out_q, the byte zero-extended (out_q holds 2 * bytes_q
 * bytes), and likewise k -> out_k; one-wave workgroups, each thread loading
 * 8 bytes and storing 16. Pointers must be 16-byte aligned; an output
 * overlapping any input or the other output is QKN_EOVERLAP; an output above
 * 2^31 - 2^16 bytes is QKN_EINVAL. A tensor of 0 bytes may be passed as a
 * null pointer (also for qknorm_bench_copy). */
int qknorm_bench_widen(const void* q, const void* k, void* out_q, void* out_k,
                       int64_t bytes_q, int64_t bytes_k, hipStream_t stream);

/* Ceiling of the persistent streaming structure for measurements: launches,
 * for format `dtype` (QKN_FMT_*) and this shape, the fused call's own plan
 * (grid, workgroup size, tiles, slot layout, groups, XCD mapping, one barrier
 * per tile and one-tile prefetch) with no arithmetic and no exchange, storing
 * every byte of q and k unchanged to out_q and out_k (formats whose output
 * element is twice the input's: each byte zero-extended to a 16-bit word).
 * Pointers 16-byte aligned; outputs overlapping an input or each other are
 * QKN_EOVERLAP; a shape the fused kernel does not run (split kernels) or a
 * tensor of 2^31 - 2^16 bytes or more is QKN_EINVAL. */
int qknorm_bench_skeleton(int dtype, const void* q, const void* k, void* out_q, void* out_k,
                          int64_t T, int64_t Hq, int64_t Hk, int n_shards, hipStream_t stream);

/* Measurement helper: issues `repeats` back-to-back fused calls with the same
 * arguments (as the fused entry point of format `dtype`, a QKN_FMT_* value)
 * from C, so that launch-rate-bound shapes can be timed without a host
 * language's per-call overhead. Returns the first non-OK status. */
int qknorm_bench_fused(int dtype, const void* q, const void* k, const void* gamma_q,
                       const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk, int n_shards,
                       float eps, void* out_q, void* out_k, int repeats, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QKNORM_H */
