/*
 * santa.h -- C ABI of the decode-step stochastic sparse attention library
 * (libsanta.so, gfx950 / MI355X).
 *
 * The method is SANTA as described on the web page "Stochastic Sparse
 * Attention for Memory-Bound Inference" (ICML 2026 paper notes).  For each
 * query head of one decode step the library scores the whole KV cache, forms
 * the softmax distribution A, and instead of the full A.V product draws S
 * indices from A by systematic sampling (one offset U in [0, 1/S), thresholds
 * U + m/S, m = 0..S-1; "key design 1") and averages the S matching V rows.
 * Two GPU schedules are offered: S2ANTA-prop ("key design 2": exact scores
 * and a stash in pass 1, a global reducer that gives every tile a budget
 * equal to the number of thresholds falling in its CDF interval, sampling
 * and the V gather in pass 2) and S2ANTA-flash ("key design 3": every tile
 * samples S/n_t tokens from its own softmax, partial means are rescaled by
 * the true tile mass at merge time).  exact_decode_ref is the same GPU's
 * exact split-KV decode, the baseline the pages compare against
 * (FlashDecoding-style, "key design 2" and related work).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless its comment says host.
 *   - The caller owns all memory.  The library allocates nothing, keeps no
 *     global state except the optional timing hook and the static scratch
 *     of santa_decode_prop_static (both below), and is reentrant.
 *   - Work is launched asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Results are valid once the stream has synchronised.
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error nothing is launched and no output is written.
 *   - For identical inputs results are bitwise identical from run to run:
 *     every reduction has a fixed order, and the only floating-point atomics
 *     (prop with at most 256 heads in the batch, 128 with the list
 *     generators) add a head's two partial outputs onto its zeroed row,
 *     a sum that does not depend on which arrives first.  A head's output
 *     can differ in its last bits between calls on either side of those
 *     head counts (its partial sums are grouped differently); its indices
 *     and budgets do not.
 *   - No output may share memory with an input or with another output.  The
 *     host rejects an `out` that overlaps `q` or the first B*Hq floats of `u`
 *     with SANTA_ERR_INVALID (prop clears output rows while other
 *     workgroups of the same call still read the query).
 *   - No C++ exception crosses this boundary.
 *
 * Layouts (row-major, last index fastest)
 *   q     [B, Hq, d]                          q_dtype
 *   k, v  contiguous: [B, Hkv, max_seq_len, d]   kv_dtype
 *         paged:      [num_pages, Hkv, page_size, d]; token j of request b
 *                     is row (j % page_size) of page page_table[b][j / page_size]
 *   u     [B*Hq] fp32, u[b*Hq+h] in [0, 1/S)  (one offset per head; a caller
 *         wanting one offset per request replicates it over the heads).
 *         The device clamps any other value into [0, u_max], u_max the
 *         largest float below 1/S (NaN and -0 count as 0), so every call
 *         places S thresholds in [0, 1)
 *   out   [B, Hq, d] fp32
 *   q head h reads KV head h / (Hq / Hkv)     (grouped-query attention)
 */
#ifndef SANTA_H
#define SANTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
    SANTA_OK = 0,
    SANTA_ERR_INVALID = -1,      /* null required pointer, bad size, bad combination */
    SANTA_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim, dtype, group, tile */
    SANTA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required        */
    SANTA_ERR_HIP = -4,          /* a HIP launch reported an error                    */
    SANTA_ERR_TOO_LARGE = -5     /* santa_decode_prop_static: the problem needs more
                                    than SANTA_STATIC_SCRATCH_BYTES of workspace     */
} santa_status;

/* Storage types.  SANTA_FP8_E4M3 is OCP e4m3 (1 sign, 4 exponent bits with
   bias 7, 3 mantissa bits, no infinities; 0x7F/0xFF are NaN), for K and V
   only: with it, q is bf16.  Every e4m3 value is exact in bf16, and the
   kernels widen K to bf16 before scoring and V to fp32 before summing. */
typedef enum { SANTA_F32 = 0, SANTA_BF16 = 1, SANTA_FP8_E4M3 = 2 } santa_dtype;

typedef enum {
    SANTA_VARIANT_PROP = 0,
    SANTA_VARIANT_FLASH = 1,
    SANTA_VARIANT_EXACT = 2
} santa_variant;

/* Shapes and layout of one decode-attention call. */
typedef struct {
    int32_t batch;            /* B >= 0; B == 0 is a no-op that returns SANTA_OK   */
    int32_t num_q_heads;      /* Hq >= 1                                           */
    int32_t num_kv_heads;     /* Hkv >= 1, Hq % Hkv == 0, group Hq/Hkv in {1,2,4,8} */
    int32_t head_dim;         /* d; only 128 is built                              */
    int32_t max_seq_len;      /* n_k (contiguous) or the longest request (ragged)  */
    const int32_t *seq_lens;  /* device [B] keys per request, or NULL: every
                                 request has max_seq_len keys.  A value <= 0 makes
                                 that request empty: its output rows are 0, its
                                 sample indices -1 and its budgets 0.  Values
                                 above max_seq_len are clamped to it.              */
    int32_t q_dtype;          /* santa_dtype; equal to kv_dtype, or SANTA_BF16
                                 when kv_dtype is SANTA_FP8_E4M3                   */
    int32_t kv_dtype;         /* santa_dtype                                       */
    int32_t page_size;        /* 0: contiguous K/V.  Else a multiple of 16: paged
                                 pools                                             */
    const int32_t *page_table;/* device [B, max_pages_per_seq] (paged only)        */
    int32_t max_pages_per_seq;/* >= ceil(max_seq_len / page_size) (paged only)     */
    float scale;              /* softmax scale, normally (float)(1/sqrt(d))        */
    int32_t tile_len;         /* T, tokens per tile: 64, 128, 256, 512 or 1024;
                                 ceil(max_seq_len / T) must not exceed 1024        */
} santa_problem;

/*
 * Bytes of device workspace the given variant needs for this problem and S
 * (S is ignored for SANTA_VARIANT_EXACT).  Writes *bytes; returns a status
 * (the same validation as the decode calls).  The workspace must be 256-byte
 * aligned.  Every variant's workspace starts with SANTA_SYNC_BYTES of arrival
 * counters that only santa_decode_prop_fused uses: they must be zero before
 * a workspace is first passed to it (allocate the workspace zeroed, or zero
 * that prefix once), and every call leaves them zero; no other call reads
 * or writes them.  The rest of the workspace need not be initialised.
 */
#define SANTA_SYNC_BYTES (64u << 10)
int santa_workspace_size(const santa_problem *p, int32_t variant, int32_t S, size_t *bytes);

/*
 * S2ANTA-prop ("key design 2").  Pass 1 streams K once per tile of T tokens,
 * computes the group's scores, the per-tile max and partition function and
 * writes the exponentiated scores to a stash; a reducer per head forms the
 * tile CDF and gives tile t a budget S_t equal to the number of thresholds
 * U + m/S inside its CDF interval (so sum_t S_t = S and tiles of low mass
 * get 0 and are never read again); pass 2 scans the stash of each tile with
 * S_t > 0, inverts its CDF at its thresholds, gathers those V rows and
 * divides the sum by S.  This equals untiled systematic sampling.
 *
 *   S            samples per head, 1 <= S <= 4096 (larger: SANTA_ERR_UNSUPPORTED)
 *   u            [B*Hq] offsets in [0, 1/S) (clamped into it on the device,
 *                see the layouts above)
 *   out          [B, Hq, d] fp32 estimate
 *   sample_idx   [B, Hq, S] int32 or NULL: token selected by threshold m,
 *                in threshold order (repeats mean multiplicity)
 *   tile_budget  [B, Hq, ceil(max_seq_len/T)] int32 or NULL: S_t per tile
 *   workspace    santa_workspace_size(p, SANTA_VARIANT_PROP, S) bytes
 */
int santa_decode_prop(const santa_problem *p, const void *q, const void *k, const void *v,
                      int32_t S, const float *u, float *out, int32_t *sample_idx,
                      int32_t *tile_budget, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * S2ANTA-prop in a single launch ("key design 2" with its global step as a
 * per-group arrival count instead of a kernel boundary).  Every workgroup
 * scores its tile and writes its stash and tile statistics as in
 * santa_decode_prop, publishes them (an agent-scope release) and increments
 * its (request, KV group)'s counter; the workgroup that completes the count
 * runs the reducer and pass 2 of the group's heads and resets the counter.
 * No workgroup waits for another.  Results: the same indices and budgets as
 * santa_decode_prop (the same arithmetic); the output sums the same rows in
 * another order (4 waves per head instead of 16), so it may differ in the
 * last bits.
 *   arguments    as for santa_decode_prop (systematic thresholds)
 *   workspace    santa_workspace_size(p, SANTA_VARIANT_PROP, S) bytes whose
 *                first SANTA_SYNC_BYTES are zero (see above); calls sharing
 *                a workspace must not overlap in time
 *   B * Hkv must not exceed 1024 (else SANTA_ERR_UNSUPPORTED)
 */
int santa_decode_prop_fused(const santa_problem *p, const void *q, const void *k, const void *v,
                            int32_t S, const float *u, float *out, int32_t *sample_idx,
                            int32_t *tile_budget, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Threshold generators of prop ("key design 1"). */
typedef enum {
    SANTA_SAMPLER_SYS = 0,     /* S2ANTA-sys: t_m = U + m/S, one offset U per head   */
    SANTA_SAMPLER_STRAT = 1,   /* S2ANTA-strat: t_m = (m + u_m)/S, one uniform per
                                  stratum [m/S, (m+1)/S)                            */
    SANTA_SAMPLER_IID = 2      /* plain SANTA: t = the S uniforms, sorted (i.i.d.
                                  draws from A, as in the Eq. (4) estimator)         */
} santa_sampler;

/*
 * S2ANTA-prop with a choice of threshold generator ("key design 1"; the
 * schedule is that of santa_decode_prop, which is this call with
 * SANTA_SAMPLER_SYS).  Tile budgets are the numbers of thresholds in each
 * tile's CDF interval for every generator, so sum_t S_t = S.
 *
 *   sampler      a santa_sampler value (else SANTA_ERR_INVALID)
 *   u            SANTA_SAMPLER_SYS: [B*Hq] offsets in [0, 1/S) (clamped as
 *                for santa_decode_prop);
 *                STRAT and IID: [B*Hq, S] uniforms in [0, 1).  The device
 *                does not check them: values outside the range are clamped
 *                into it (NaN counts as 0).  STRAT and IID thresholds are
 *                formed in fp64 (IID sorted on the device).
 *   other arguments and the workspace as for santa_decode_prop; the
 *   threshold list lives in LDS (S doubles, a power of two for IID).
 */
int santa_decode_prop_sampler(const santa_problem *p, const void *q, const void *k, const void *v,
                              int32_t S, int32_t sampler, const float *u, float *out,
                              int32_t *sample_idx, int32_t *tile_budget, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * S2ANTA-flash ("key design 3").  No global step between scoring and
 * sampling: each tile of T tokens takes S_f = S / n_t samples from its own
 * softmax with thresholds u_f + m/S_f, u_f = U * n_t (one offset per head,
 * scaled to the tile budget), and averages those V rows; the merge weighs
 * every tile's mean by its true share of the mass.  Requires seq_lens ==
 * NULL (every request has max_seq_len keys) and S % n_t == 0 with
 * n_t = ceil(max_seq_len / T), else SANTA_ERR_INVALID.
 *
 *   sample_idx   [B, Hq, S] int32 or NULL, tile-major: tile t's samples are
 *                entries t*S_f .. t*S_f + S_f - 1
 *   tile_budget  ignored (every tile's budget is S_f); may be NULL
 *   workspace    santa_workspace_size(p, SANTA_VARIANT_FLASH, S) bytes
 */
int santa_decode_flash(const santa_problem *p, const void *q, const void *k, const void *v,
                       int32_t S, const float *u, float *out, int32_t *sample_idx,
                       int32_t *tile_budget, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * S2ANTA-flash with a choice of threshold generator ("key design 1" applied
 * to each tile's own softmax; santa_decode_flash is this call with
 * SANTA_SAMPLER_SYS).  Each tile takes S_f = S / n_t samples:
 *   SANTA_SAMPLER_SYS    u [B*Hq] offsets in [0, 1/S); local thresholds
 *                        u_f + m/S_f with u_f = U * n_t
 *   SANTA_SAMPLER_STRAT  u [B*Hq, S] uniforms in [0, 1), tile-major (tile t's
 *                        at t*S_f .. t*S_f + S_f - 1); local thresholds
 *                        (m + u_m)/S_f
 *   SANTA_SAMPLER_IID    u as for STRAT; local thresholds: the tile's
 *                        uniforms, sorted on the device
 * Uniforms outside [0, 1) are clamped into it (NaN counts as 0).  Other
 * arguments, requirements and the workspace as for santa_decode_flash.
 */
int santa_decode_flash_sampler(const santa_problem *p, const void *q, const void *k, const void *v,
                               int32_t S, int32_t sampler, const float *u, float *out,
                               int32_t *sample_idx, int32_t *tile_budget, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Exact split-KV decode on the same GPU: out = softmax(scale * q K^T) V per
 * head, computed per tile (max, sum, weighted V sum) and merged.  This is
 * the baseline that S2ANTA is measured against.
 *   workspace    santa_workspace_size(p, SANTA_VARIANT_EXACT, 0) bytes
 */
int exact_decode_ref(const santa_problem *p, const void *q, const void *k, const void *v,
                     float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * S2ANTA-prop on Bernoulli qK^T scores ("key design 4", the score-stage
 * sparsification, composed with "key design 2"; the mean group query is the
 * one of the ablation table).  Pass 1 replaces the exact scores by an
 * unbiased estimate from ternary queries: a query is scaled into [-1, 1] by
 * a = max_i |q_i|, and each of `draws` independent draws keeps feature i,
 * with the sign of q_i, when fl32(u * a) < |q_i| (u: that draw's uniform for
 * feature i).  With c_i the sum of the draws, the score of key j is
 * scale * (a / draws) * sum_i c_i K[j][i], whose expectation is the exact
 * score.  Only features with c_i != 0 are read from K, which is therefore
 * passed feature-major.  The reducer and pass 2 are those of
 * santa_decode_prop (systematic thresholds).
 *
 * Built for (else SANTA_ERR_UNSUPPORTED): q_dtype = SANTA_BF16 with kv_dtype
 * SANTA_BF16 or SANTA_FP8_E4M3, page_size = 0 (seq_lens may be given),
 * max_seq_len % 4 == 0.
 *   k_features   [B, Hkv, d, max_seq_len] kv_dtype, 8-byte (bf16) or 4-byte
 *                (e4m3) aligned (else SANTA_ERR_INVALID): K transposed per
 *                KV head
 *   v            [B, Hkv, max_seq_len, d] kv_dtype (the usual layout)
 *   draws        ternary draws per query, 1..64 (else SANTA_ERR_INVALID)
 *   group_mean   0: every q head draws its own ternary query, and its KV
 *                group reads the union of their kept features.  1: the fp32
 *                mean of the group's Hq/Hkv queries (summed in head order,
 *                then multiplied by Hkv/Hq) is drawn once and every head of
 *                the group takes its scores.  Other values: SANTA_ERR_INVALID
 *   u_bern       fp32 uniforms in [0, 1): [B*Hq, draws, d] (group_mean 0) or
 *                [B*Hkv, draws, d] (group_mean 1).  Not checked on the device:
 *                the comparison above is applied to whatever is given
 *   features_read [B*Hkv] int32 or NULL: the number of features of K the
 *                group reads (kept by any of its draws), also for empty
 *                requests
 *   other arguments and the workspace (santa_workspace_size with
 *   SANTA_VARIANT_PROP) as for santa_decode_prop
 */
int santa_decode_prop_bernoulli(const santa_problem *p, const void *q, const void *k_features,
                                const void *v, int32_t S, const float *u, int32_t draws,
                                int32_t group_mean, const float *u_bern, float *out,
                                int32_t *sample_idx, int32_t *tile_budget, int32_t *features_read,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * santa_decode_prop without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  The call allocates nothing: its
 * workspace is a static device array of SANTA_STATIC_SCRATCH_BYTES (32 MiB)
 * inside the library, which every GPU the library runs on holds until the
 * process ends (its address is looked up once per device, on the first call
 * made with that device current).
 *   - Problems whose santa_workspace_size(p, SANTA_VARIANT_PROP, S) exceeds
 *     SANTA_STATIC_SCRATCH_BYTES return SANTA_ERR_TOO_LARGE, launching
 *     nothing (e.g. the 32k-token, 32/8-head layer fits up to batch 7).
 *   - All calls on one GPU share that GPU's array.  Calls that overlap in
 *     time on one GPU (other streams, other threads) race on it and give
 *     undefined results; calls in one stream are ordered and safe.  Nothing
 *     in the array has to start at zero: each call writes every entry it
 *     reads.
 *   - Arguments, results and every other convention as for
 *     santa_decode_prop (same kernels, bitwise the same results).
 */
#define SANTA_STATIC_SCRATCH_BYTES (32u << 20)
int santa_decode_prop_static(const santa_problem *p, const void *q, const void *k, const void *v,
                             int32_t S, const float *u, float *out, int32_t *sample_idx,
                             int32_t *tile_budget, void *stream);

/*
 * Optional timing hook for benchmarks.  When both events are non-NULL
 * (hipEvent_t), every later decode call made from the calling thread
 * records `begin` just before and `end` just after its dominant kernel (the
 * one that streams K: pass 1 for prop, the tile kernel for flash, the
 * partial kernel for exact, the Bernoulli pass 1 for
 * santa_decode_prop_bernoulli) on the call's stream.  Pass NULL, NULL to
 * turn it off.  Thread-local; returns SANTA_OK.
 */
int santa_set_timing_events(void *begin_event, void *end_event);

/* Static description of a status code. */
const char *santa_status_string(int status);

/* Library ABI version (increments on any signature or layout change). */
int santa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SANTA_H */
