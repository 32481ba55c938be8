/* kvc.h -- attention-matching KV-cache compaction on AMD Instinct MI355X (gfx950).
 *
 * Method: "Fast KV Compaction via Attention Matching" (Zweiger, Fu, Guo, Kim),
 * technical summary, section 2.  Per (layer, KV head) the library builds a
 * compact cache (C_k, beta, C_v) of t << T entries from the full cache (K, V)
 * and a set of reference queries Q_ref so that, on those queries, attention
 * over the compact cache reproduces both the attention output and the
 * attention mass of the full cache (the output- and mass-matching equations of
 * the "main objective" paragraph):
 *
 *   1. s = Q_ref K^T (no extra scale: Q_ref carries 1/sqrt(d)), lse per query,
 *      p = exp(s - lse), full-cache output O = P V;
 *   2. importance of key j = RMS over the reference queries of p_ij (or the
 *      mean, KVC_AGG_MEAN); keep the t most important ORIGINAL keys
 *      ("highest-attention keys" in the algorithmic pipeline); equal
 *      importances go to the lower index; kept indices ascend;
 *   3. bias: w = argmin_{w >= 0} ||P_S w - 1||^2 + lam_w ||w - 1||^2 (each
 *      query's kept mass, re-weighted, equals its full mass; the pipeline's
 *      NNLS bias fit), beta = log(max(w, 1e-30));
 *   4. values: C_v = argmin ||X C - O||^2 + lam_v ||C - V_S||^2 with X the
 *      softmax over the kept keys with the fitted bias (the pipeline's
 *      least-squares value fit given keys and bias).
 *   lam_w = ridge_rel * trace(P_S^T P_S) / t and lam_v = ridge_rel *
 *   trace(X^T X) / t: a vanishing ridge toward the prior (w = 1, C_v = V_S).
 *   ridge_rel = 0 is the pipeline's literal NNLS and least squares; it needs
 *   the Grams to be positive definite (n >= t, no duplicated kept keys).
 *
 * Conventions for every entry point below:
 *   - every array pointer is a DEVICE pointer to row-major, contiguous data,
 *     aligned to 16 bytes; the caller owns every buffer; the library
 *     allocates no device memory in these calls;
 *   - work is enqueued on `stream` and is asynchronous: outputs are valid once
 *     the stream has completed;
 *   - argument errors (KVC_EINVAL, KVC_EWORKSPACE, KVC_EUNSUPPORTED) are
 *     detected before anything is enqueued;
 *   - the library keeps no state between calls (apart from the benchmark
 *     instrumentation and the wait limit below), so calls with distinct
 *     workspaces may be issued from several host threads; two calls that
 *     share a workspace must be ordered on one stream;
 *   - the fits run as launches whose grid is sized to what the whole device
 *     holds at once (their teams of workgroups wait for each other), which
 *     assumes the device is not busy with other long-running work meanwhile:
 *     compactions that should all succeed must not overlap in time on the
 *     device (issue them on one stream, or synchronize between streams).  If
 *     they do overlap, a fit team's wait may run out: every wait is bounded,
 *     so the call still ends, and the affected heads report
 *     KVC_STATUS_SYNC_TIMEOUT.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_OK            0
#define KVC_EINVAL       -1   /* null pointer, misalignment, bad size or enum     */
#define KVC_EWORKSPACE   -2   /* workspace smaller than kvc_workspace_bytes()     */
#define KVC_EHIP         -3   /* a HIP launch or query failed                     */
#define KVC_EUNSUPPORTED -4   /* head dim other than 64/128, or sizes past limits */

/* Per-head numerical status written to out_status[b] (0 = ok). */
#define KVC_STATUS_OK            0
#define KVC_STATUS_NOT_SPD       1  /* a sweep pivot had the wrong sign or
                                       vanished (the regularized Gram is not
                                       numerically positive definite)          */
#define KVC_STATUS_NNLS_CAP      2  /* NNLS stopped at max_nnls_iters           */
#define KVC_STATUS_NONFINITE     4  /* a non-finite value reached the fits      */
#define KVC_STATUS_SYNC_TIMEOUT  8  /* a fit team's barrier wait ran out (the
                                       head's fit is incomplete)               */
#define KVC_STATUS_BUDGET       16  /* kvc_compact_ragged: the head's budget was
                                       outside [1, p->t] and was clamped       */
#define KVC_STATUS_PROTECT      32  /* kvc_compact_protected: more than t - 1
                                       keys were marked; only the first t - 1
                                       (by position) were kept as protected    */
#define KVC_STATUS_RIDGE_RAISED 64  /* a failed pivot in the bias NNLS made the
                                       head restart with the ridge raised
                                       tenfold (relative ridge max(10^e ridge,
                                       10^(e-1) 1e-9) at the e-th raise, at
                                       most 3); the count e is in bits 8-9
                                       (KVC_STATUS_RAISES), the values are
                                       fitted with the raised ridge, and
                                       KVC_STATUS_NOT_SPD remains only if the
                                       third raise still failed                */
#define KVC_STATUS_RAISES(s)    (((s) >> 8) & 3)

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype_t;
typedef enum { KVC_AGG_RMS = 0, KVC_AGG_MEAN = 1 } kvc_agg_t;

typedef struct {
  int64_t B;              /* independent (layer, KV head) problems, >= 1          */
  int64_t T;              /* cache length per head, >= 1                          */
  int64_t n;              /* reference queries per head, >= 1                     */
  int64_t d;              /* head dim: 64 or 128                                  */
  int64_t t;              /* kept keys per head, 1 <= t <= T, t <= 4096           */
  int32_t in_dtype;       /* kvc_dtype_t of Q_ref, K, V (out_K has the same)      */
  int32_t agg;            /* kvc_agg_t, default KVC_AGG_RMS                       */
  double  ridge_rel;      /* ridge weight relative to the Gram's mean diagonal,
                             default 1e-6; >= 0 (0: no ridge)                     */
  int32_t max_nnls_iters; /* cap on NNLS pivoting rounds, default 32              */
  int32_t out_v_dtype;    /* kvc_dtype_t of out_V, default KVC_F32; KVC_BF16
                             stores the float32 result rounded to nearest-even   */
  int32_t refine_steps;   /* refinement steps of the value fit, 0..4, default 0.
                             Each step is one corrected semi-normal-equation
                             step: E = O - X_F C, C += (G + lam_v I)^-1
                             (X_F^T E - lam_v (C - V_S)), with the inverse the
                             value sweep leaves when refinement is on.  It
                             takes the residual against O itself, so it
                             recovers accuracy the normal equations lose when
                             X_F is ill-conditioned.  Needs workspace for E
                             (B n d doubles) and two B t d double buffers      */
  int32_t reserved;       /* must be 0                                            */
} kvc_params_t;

/* Fill *p with the defaults above (sizes zeroed). */
void kvc_params_default(kvc_params_t* p);

/* Bytes of device workspace kvc_compact / kvc_fit need for these parameters,
 * or 0 if the parameters are invalid.  Depends on B, T, n, d, t only. */
size_t kvc_workspace_bytes(const kvc_params_t* p);

/* Compact B independent heads.
 *   Q_ref   [B, n, d]  in_dtype   reference queries (scaled by the caller)
 *   K, V    [B, T, d]  in_dtype   full cache (keys as stored, e.g. post-RoPE)
 *   out_K   [B, t, d]  in_dtype   kept keys: exact copies of K rows
 *   out_bias[B, t]     float32    beta, an additive logit bias per kept key
 *   out_V   [B, t, d]  out_v_dtype fitted values
 *   out_idx [B, t]     int32      kept indices, ascending; may be NULL
 *   out_status [B]     int32      per-head KVC_STATUS_* bits; may be NULL
 *   workspace          >= kvc_workspace_bytes(p) bytes of device memory
 * Returns KVC_OK once everything is enqueued, or a negative KVC_E* code. */
int kvc_compact(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
                void* out_K, float* out_bias, void* out_V, int32_t* out_idx,
                int32_t* out_status, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* kvc_compact for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and outputs, with the workspace taken from a device array
 * of KVC_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends.  Allocates nothing.
 *   Arguments as kvc_compact, without the workspace.
 *   Returns KVC_EWORKSPACE when kvc_workspace_bytes(p) exceeds
 *   KVC_NOALLOC_SCRATCH_BYTES (64 MiB; e.g. one head of 4096 tokens with
 *   t = 256, or a few heads of 8192), KVC_EHIP if the array's device address
 *   cannot be obtained, else as kvc_compact.
 *   All calls on one device share its array, which keeps the last call's
 *   contents: calls that overlap in time on one device race (order them on one
 *   stream). */
#define KVC_NOALLOC_SCRATCH_BYTES (64ull << 20)
int kvc_compact_noalloc(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
                        void* out_K, float* out_bias, void* out_V, int32_t* out_idx,
                        int32_t* out_status, hipStream_t stream);

/* Bias and value fit for a caller-given kept set (steps 3-4 only).
 *   idx [B, t] int32, strictly ascending, in [0, T).  Other arguments as in
 *   kvc_compact.  Used to check the fits in isolation and to re-fit a cache
 *   whose keys were chosen elsewhere. */
int kvc_fit(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
            const int32_t* idx, float* out_bias, void* out_V, int32_t* out_status,
            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Ragged per-head budgets: head b keeps t_heads[b] keys, 1 <= t_heads[b] <=
 * p->t, so one call serves a non-uniform head/layer schedule (the per-head
 * retention ratios of the method's schedule; the per-segment budgets of the
 * thought-aware variant's budget rule).  Each head is compacted exactly as
 * kvc_compact would with t = t_heads[b].
 *   t_heads  [B] int32, DEVICE memory, 4-byte aligned; read on the stream, so
 *            the values may come from earlier work on it.  A value outside
 *            [1, p->t] is clamped and flags KVC_STATUS_BUDGET for that head.
 *   Outputs have kvc_compact's shapes with t = p->t (the largest budget).
 *   Head b's first t_heads[b] slots hold its compact cache; the remaining
 *   slots are padding that attention ignores: out_idx = -1, out_K and out_V
 *   rows of zeros, out_bias = -inf (a zero softmax weight).
 *   workspace  >= kvc_workspace_bytes(p) bytes.
 * Returns as kvc_compact. */
int kvc_compact_ragged(const kvc_params_t* p, const int32_t* t_heads, const void* Q_ref,
                       const void* K, const void* V, void* out_K, float* out_bias, void* out_V,
                       int32_t* out_idx, int32_t* out_status, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Greedy key selection by orthogonal matching pursuit (the summary's second
 * key-selection option: choose keys greedily to best satisfy the mass
 * matching, then fit weights by NNLS).  The dictionary is the whole-cache
 * softmax weights p_j = P[:, j] (over the reference queries) stored in
 * float32; the target is the relative mass y = 1.  For t steps: pick the key
 * not yet chosen with the largest p_j . r / ||p_j|| (float64; ties to the
 * lower index; keys whose column is all zero only when nothing else is
 * left), then set r to y minus its orthogonal projection on the chosen
 * columns.  The chosen set (ascending) then gets kvc_compact's bias and value
 * fits.  p->agg is ignored.
 * Cost: t passes over P (n * T * 4 bytes per head each); the workspace holds P
 * and an n x t basis per head: use kvc_workspace_bytes_omp.
 * Arguments and outputs as kvc_compact. */
size_t kvc_workspace_bytes_omp(const kvc_params_t* p);
int kvc_compact_omp(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
                    void* out_K, float* out_bias, void* out_V, int32_t* out_idx,
                    int32_t* out_status, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Protected keys ("Thought-Aware KV Cache Compaction for Reasoning via
 * Adaptive Attention Matching", section 2C: pivot tokens are kept exactly,
 * with zero bias, and the rest of the budget goes to the other tokens).
 * For head b let P be the marked keys (at most t - 1 of them, the first by
 * position; more sets KVC_STATUS_PROTECT) and R the others.  P is kept as is;
 * R is compacted to t - |P| keys exactly as kvc_compact compacts a cache,
 * with R's own log-sum-exp, output and importance (P's exact block carries
 * its own mass and output, so by the block decomposition of the main
 * objective the fitted part only has to match R).
 *   protect_mask [B, T] uint8, DEVICE memory: nonzero marks a protected key.
 *   Outputs have kvc_compact's shapes.  Head b's slots [0, t - |P|) hold the
 *   fitted part (indices ascending), slots [t - |P|, t) the protected keys
 *   (ascending): out_K and out_V their K and V rows (V converted to
 *   out_v_dtype), out_bias 0.
 *   workspace  >= kvc_workspace_bytes(p) bytes.
 * Returns as kvc_compact. */
int kvc_compact_protected(const kvc_params_t* p, const uint8_t* protect_mask, const void* Q_ref,
                          const void* K, const void* V, void* out_K, float* out_bias,
                          void* out_V, int32_t* out_idx, int32_t* out_status, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Chunked compaction ("Compaction par blocs" of the same summary): each head's
 * cache is cut into n_chunks contiguous chunks of T / n_chunks keys, every
 * chunk is compacted on its own to t entries against the head's full Q_ref
 * (lse, output, importance and both fits are taken over the chunk alone), and
 * the results are concatenated in chunk order.  Attention over concatenated
 * blocks splits into per-block (output, mass) pairs (the block-concatenation
 * decomposition of the main objective), so the concatenated (C_k, beta, C_v)
 * matches the whole cache's attention as each chunk matches its own; no bias
 * is re-fit after the merge.
 *   p          sizes of the whole problem: B heads of T keys, t kept keys PER
 *              CHUNK; T must be a multiple of n_chunks and t <= T / n_chunks
 *   n_chunks   >= 1; 1 gives exactly kvc_compact
 *   Q_ref      [B, n, d]             in_dtype
 *   K, V       [B, T, d]             in_dtype
 *   out_K      [B, n_chunks * t, d]  in_dtype   kept keys, chunk-major
 *   out_bias   [B, n_chunks * t]     float32
 *   out_V      [B, n_chunks * t, d]  out_v_dtype
 *   out_idx    [B, n_chunks * t]     int32      positions in the head's cache
 *                                               (ascending); may be NULL
 *   out_status [B, n_chunks]         int32      KVC_STATUS_* per chunk; may be NULL
 *   workspace  >= kvc_workspace_bytes_chunked(p, n_chunks) bytes
 * Returns as kvc_compact; KVC_EINVAL also when T % n_chunks != 0. */
size_t kvc_workspace_bytes_chunked(const kvc_params_t* p, int64_t n_chunks);
int kvc_compact_chunked(const kvc_params_t* p, int64_t n_chunks, const void* Q_ref,
                        const void* K, const void* V, void* out_K, float* out_bias, void* out_V,
                        int32_t* out_idx, int32_t* out_status, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Attention over a cache followed by an appended fixed block, for queries Q
 * (the keys are split across workgroups; workspace: at least
 * kvc_attend_workspace_bytes(p) bytes, may be NULL when that is 0):
 *   out_i = softmax_j(q_i . k_j + bias_j) v_j over the t1 keys of block 1
 *   (with bias1; e.g. a compact cache C_k, beta, C_v) and then the t2 keys of
 *   block 2 (bias 0; e.g. the fixed or future tokens appended after it),
 *   out_lse_i = log sum_j exp(q_i . k_j + bias_j).
 * This is the consumer's side of the main objective ("for any query and any
 * fixed block appended after the compact cache"): with the original cache as
 * block 1 it gives the reference, with the compact cache the compacted
 * attention, on the GPU.  float32 arithmetic, online softmax.
 *   Q      [B, m, d]   in_dtype
 *   K1     [B, t1, d]  in_dtype;  bias1 [B, t1] float32 or NULL (zeros; -inf
 *                      gives a key zero weight);  V1 [B, t1, d] float32 when
 *                      v1_f32 = 1 (fitted values), else in_dtype
 *   K2, V2 [B, t2, d]  in_dtype; may be NULL when t2 = 0
 *   out    [B, m, d]   float32;  out_lse [B, m] float64 or NULL
 * t1 >= 0, t2 >= 0, t1 + t2 >= 1.  Returns KVC_OK once enqueued. */
typedef struct {
  int64_t B, m, d, t1, t2;
  int32_t in_dtype;  /* kvc_dtype_t of Q, K1, K2, V2 (and V1 unless v1_f32) */
  int32_t v1_f32;    /* 1: V1 is float32; 0: V1 has in_dtype */
  int32_t reserved;  /* must be 0 */
  int32_t reserved2; /* must be 0 */
} kvc_attend_params_t;
size_t kvc_attend_workspace_bytes(const kvc_attend_params_t* p);
int kvc_attend(const kvc_attend_params_t* p, const void* Q, const void* K1, const float* bias1,
               const void* V1, const void* K2, const void* V2, float* out, double* out_lse,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Where the intermediates of the last call live inside its workspace (byte
 * offsets), for inspection after the stream completes:
 *   lse [B, n] f64; O [B, n, d] f32 (full-cache output); imp [B, T] f32 holding
 *   sum_i p_ij^2 (RMS) or sum_i p_ij (mean) -- the ranking key before the
 *   monotone sqrt(./n) or ./n; w [B, t] f64 the NNLS multipliers;
 *   fit_flops [B, 2] f64 the floating-point operations the NNLS rounds
 *   (factorizations and solves) and the value solve performed for each head. */
typedef struct {
  size_t lse, O, imp, w, fit_flops;
  size_t omp_order; /* [B, t] int32: after kvc_compact_omp, the keys in the
                       order the pursuit chose them (workspace of
                       kvc_workspace_bytes_omp) */
  size_t value_C;   /* f64: the value fit's solution before its float32 (or
                       bf16) output, head b's passive variable a (the a-th
                       kept slot with w > 0) at row a of a [value_ld]-strided
                       matrix starting value_C + 8 b value_ld^2, columns 0..d-1 */
  size_t value_ld;  /* that row stride, in doubles */
} kvc_ws_layout_t;
int kvc_workspace_layout(const kvc_params_t* p, kvc_ws_layout_t* out);

/* Instrumentation for benchmarks (not thread-safe; leave off in production).
 * While the stage mask is non-zero, every kvc_compact / kvc_fit call records a
 * HIP event pair on its stream around each selected stage; events are created
 * on first use and reused.  kvc_profile_enable() resets the counters, and a
 * zero mask also destroys the events; kvc_profile_read() waits for the
 * recorded events of one stage and returns the summed elapsed time and the
 * number of recorded launches. */
#define KVC_STAGE_SCORE_LSE   0  /* scores + online log-sum-exp kernel           */
#define KVC_STAGE_EXPWEIGHT   1  /* p = exp(s - lse), P V, importance kernel      */
#define KVC_STAGE_SELECT      2  /* top-t select and gather (or the greedy pass) */
#define KVC_STAGE_PS          3  /* kept-key softmax weights P_S (fp64)           */
#define KVC_STAGE_GRAM        4  /* mass Gram P_S^T P_S (fp64 MFMA)               */
#define KVC_STAGE_NNLS        5  /* pivoting rounds incl. their Cholesky solves   */
#define KVC_STAGE_VALUE       6  /* value fit: Gram, right-hand side, solve       */
#define KVC_STAGE_TOTAL       7  /* the whole call                                */
#define KVC_STAGE_IMP_REDUCE  8  /* importance partials summed per key            */
#define KVC_STAGE_TOPT        9  /* the top-t select kernel alone                 */
#define KVC_STAGE_GATHER     10  /* kept-key row gather alone                     */
#define KVC_STAGE_VALUE_GRAM 11  /* value Gram and right-hand side X_F^T [X_F O]
                                      in one launch (fp64 MFMA)                  */
#define KVC_STAGE_VALUE_SWEEP 12 /* value system solve alone                      */
#define KVC_NUM_STAGES       13
int kvc_profile_enable(uint32_t stage_mask);
int kvc_profile_read(int stage, double* total_ms, int64_t* launches);

/* Upper bound on each wait of a fit team (in ticks of the 100 MHz constant
 * clock; default 2e9, i.e. 20 s).  A wait that runs out turns the later waits
 * of that launch into no-ops, so every kernel still ends, and flags
 * KVC_STATUS_SYNC_TIMEOUT on the launch's heads, whose fits are then
 * incomplete.  0 restores the default.  Applies to calls enqueued after it;
 * process-wide and not thread-safe: meant for exercising the time-out path. */
int kvc_set_wait_limit(uint64_t ticks);

/* Static text for a KVC_* return code. */
const char* kvc_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H_ */
