/*
 * libspecverify: batched rejection-sampling verification for speculative
 * decoding on AMD Instinct MI355X (gfx950).
 *
 * The operation.  For each request b, a draft model proposed draft_len[b]
 * tokens x_0 .. x_{n-1}; the target model produced logits for the n+1
 * positions that follow the committed prefix.  Target row k verifies draft
 * token k, and target row n supplies a bonus token when every draft survives
 * (nickwang.xyz, "推测解码：草稿、验证与实际加速", section "候选已知，验证才能并行").
 * p_k and q_k are the target and draft distributions after temperature and
 * the optional top-k / top-p filters, applied the same way to both rows
 * (same page, section "接受与拒绝怎样保住分布").  Scanning k = 0, 1, ..., the
 * call accepts x_k when u[b][k] < alpha_k = min(1, p_k(x_k) / q_k(x_k))
 * (eq. a(x) there; tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告", formula 1
 * and section "4. 实现逻辑"), stops at the first rejection j and replaces
 * x_j by a draw from max(p_j - q_j, 0) renormalised (eq. r(x); bowenzhou.top
 * "投机采样", section "深入推导"), or, when all n drafts are accepted, draws
 * a bonus token from p_n.  Both draws are inverse-CDF draws at u_final[b] over
 * token ids in ascending order (nickwang.xyz, section "算完三个 token 的全部概率",
 * function sample()).  The library draws no random numbers: the caller
 * supplies every uniform, so results are reproducible.
 *
 * Conventions for every entry point below.
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no pointer after it returns.
 *  - The call is asynchronous on `stream`; outputs are valid once the caller
 *    has synchronised that stream.  The library is stateless and reentrant;
 *    calls that share a workspace must not overlap.
 *  - Host-checkable argument errors return a status and enqueue nothing.
 *  - Per-request precondition violations found on the device (draft_len
 *    outside [0, K], a draft token outside [0, V), q(x) == 0, a uniform
 *    outside [0, 1), a needed row with no finite logit) set n_emitted[b] = -1
 *    and out_tokens[b][*] = -1; other requests are not affected.
 *  - Logits must be finite or -inf (-inf masks a token out).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define SPECV_API __attribute__((visibility("default")))
#else
#define SPECV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPECV_OK = 0,
  SPECV_EINVAL = 1,       /* bad argument (null/misaligned pointer, bad size or parameter) */
  SPECV_EWORKSPACE = 2,   /* workspace missing, misaligned (16 B) or smaller than specv_workspace_bytes() */
  SPECV_EHIP = 3,         /* a HIP launch failed */
  SPECV_EUNSUPPORTED = 4, /* valid request the library does not implement (see specv_verify) */
  SPECV_ESCRATCH = 5      /* specv_verify_noalloc: sizes beyond its fixed scratch */
} specv_status_t;

typedef enum {
  SPECV_F32 = 0,          /* IEEE float32 logits */
  SPECV_BF16 = 1          /* bfloat16 logits (upper half of a float32) */
} specv_dtype_t;

/* Largest draft length K the call accepts. */
#define SPECV_MAX_K 64
/* Largest vocabulary the call accepts (larger V returns SPECV_EUNSUPPORTED). */
#define SPECV_MAX_V 4194304
/* Bytes of the fixed device scratch array behind specv_verify_noalloc. */
#define SPECV_NOALLOC_SCRATCH_BYTES (16u << 20)
/* Largest hidden size the fused LM-head call accepts. */
#define SPECV_MAX_D 65536

/*
 * Bytes of device workspace specv_verify needs for these sizes.  Returns 0
 * for sizes specv_verify would reject.  The workspace holds per-row
 * statistics, per-request decisions and fp64 chunk partials; its contents
 * need no initialisation and are meaningless to the caller after the call.
 * (On path 3 it also keeps a per-request call counter from one call to the
 * next, which the library reads whatever it holds.  There a request whose
 * internal wait ran out -- n_emitted = -1 for valid inputs, after some 2^18
 * polls of a word another workgroup had not yet written -- may leave words
 * that a replay of the same captured graph would accept: zero the workspace
 * before replaying after such an error.)  Two calls that overlap on one
 * workspace race.  The size depends on the path the call takes
 * (specv_path_kind), so query it after any specv_set_small_batch_limit.
 */
SPECV_API size_t specv_workspace_bytes(int B, int K, int V, specv_dtype_t dtype, int top_k, float top_p);

/*
 * One batched verification step: target logits, draft logits, draft tokens,
 * draft lengths and uniforms in; emitted tokens and their count out.
 *
 *  target_logits  [B][K+1][V] of `dtype`, row-major, contiguous; element-aligned
 *                 (16-byte alignment of rows enables vector loads).
 *  draft_logits   [B][K][V] of `dtype`; may be NULL when K == 0.
 *  draft_tokens   [B][K] int32; entry k is read only when k < draft_len[b].
 *  draft_len      [B] int32, each in [0, K].
 *  u              [B][K] float32 in [0, 1): the accept test of position k.
 *  u_final        [B] float32 in [0, 1): the one correction or bonus draw.
 *  B >= 1, 0 <= K <= SPECV_MAX_K, 1 <= V <= SPECV_MAX_V (B * (K+1) * V below 2^62).
 *  temperature    > 0 and finite; logits are divided by it before filtering.
 *  top_k          0 = off; otherwise keep logits >= the top_k-th largest (ties
 *                 kept).  top_k >= V is the same as off.
 *  top_p          1 = off; otherwise in (0, 1): keep the shortest prefix of
 *                 the top-k renormalised distribution, by logit descending,
 *                 whose mass reaches top_p (crossing token and its ties kept).
 *                 Every combination is supported, for any kept-set size.  A
 *                 small active top-k (0 < top_k <= 128 whose per-chunk
 *                 candidate slots fit on chip: (ceil(V / 8192) - 1) * c
 *                 + max(c, 256) <= 4096 with c = 8 * ceil((1.5 * top_k + 40) / 8);
 *                 top_k = 50 at V = 152064 uses 2416) takes a candidate
 *                 select; every other setting (top-p alone, larger top_k) a
 *                 radix select: a one-read histogram select for bf16 rows, a
 *                 select that reads each needed row once per key digit for
 *                 float32 rows (specv_path_kind tells which).
 *  eos_id         -1 = off; else in [0, V): the round stops right after the
 *                 first emitted EOS (accepted draft or drawn token).
 *  out_tokens     [B][K+1] int32 output: emitted tokens, -1 beyond n_emitted.
 *  n_emitted      [B] int32 output: 1 .. draft_len[b] + 1, or -1 on a
 *                 per-request error.
 *  workspace      device buffer of at least specv_workspace_bytes(...) bytes,
 *                 16-byte aligned.
 */
SPECV_API specv_status_t specv_verify(const void *target_logits, const void *draft_logits,
                            specv_dtype_t dtype, const int32_t *draft_tokens,
                            const int32_t *draft_len, const float *u, const float *u_final,
                            int B, int K, int V, float temperature, int top_k, float top_p,
                            int eos_id, int32_t *out_tokens, int32_t *n_emitted,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * specv_verify for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, outputs and kernels as
 * specv_verify without the workspace; the call allocates nothing (no
 * hipMalloc, no allocating library routine).  Its scratch is one fixed
 * device array of SPECV_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held until
 * the process ends; its address is looked up once per device.  Sizes whose
 * workspace (specv_workspace_bytes) exceeds it return SPECV_ESCRATCH before
 * any device work.  It covers B=64, K=4, V=128256 (3.3 MB of workspace) and
 * B=64, K=8, V=129280 (3.4 MB); top-k 50 / top-p 0.9 at K=8, V=152064 needs
 * about 0.4 MB per request (B <= 40 fits).
 * Every call on one GPU shares that GPU's array, so calls that overlap on
 * one GPU (on different streams or host threads) race; calls in one stream
 * order are safe.  The scratch needs no initialisation.
 */
SPECV_API specv_status_t specv_verify_noalloc(const void *target_logits, const void *draft_logits,
                                    specv_dtype_t dtype, const int32_t *draft_tokens,
                                    const int32_t *draft_len, const float *u, const float *u_final,
                                    int B, int K, int V, float temperature, int top_k, float top_p,
                                    int eos_id, int32_t *out_tokens, int32_t *n_emitted,
                                    hipStream_t stream);

/*
 * specv_verify plus diagnostic outputs, each nullable:
 *  accept_prob    [B][K] float32: alpha_k for k < draft_len[b], -1 otherwise
 *                 (and -1 for error requests).
 *  residual_mass  [B] float64: sum_v max(p_j - q_j, 0) on the rejection path
 *                 (nickwang.xyz, section "算完三个 token 的全部概率": it equals one
 *                 minus the acceptance rate), 0 on other paths.
 *  stop_pos       [B] int32: the rejected position, the EOS position, or
 *                 draft_len[b] when every draft was accepted; -1 on error.
 *  path           [B] int32: 0 rejection + correction, 1 bonus, 2 EOS, -1 error.
 */
SPECV_API specv_status_t specv_verify_debug(const void *target_logits, const void *draft_logits,
                                  specv_dtype_t dtype, const int32_t *draft_tokens,
                                  const int32_t *draft_len, const float *u,
                                  const float *u_final, int B, int K, int V,
                                  float temperature, int top_k, float top_p, int eos_id,
                                  int32_t *out_tokens, int32_t *n_emitted, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream,
                                  float *accept_prob, double *residual_mass,
                                  int32_t *stop_pos, int32_t *path);

/*
 * Batched draws from processed distributions: for each row r of
 * logits[R][V], out_tokens[r] is the token at u[r] of the inverse CDF of
 * F(logits[r]), F being the temperature / top-k / top-p processing that
 * specv_verify applies, with token ids in ascending order and a strict
 * comparison (nickwang.xyz, "推测解码：草稿、验证与实际加速", section
 * "算完三个 token 的全部概率", function sample()).  Its main use is the draft
 * model's own step: a drafted token x_k is a draw from q_k (same page,
 * section "接受与拒绝怎样保住分布"), so tokens drawn here from the draft
 * logits, with their own uniforms, are the draft_tokens that specv_verify
 * then checks.
 *
 *  logits      [R][V] dtype, row-major, device; rows 16-B aligned take the vector path
 *  u           [R] float32 in [0, 1), device
 *  out_tokens  [R] int32, device: the drawn ids; -1 for a row with no finite
 *              logit or u outside [0, 1) (other rows unaffected)
 *  workspace   device, 16-B aligned, at least specv_workspace_bytes(R, 0, V,
 *              dtype, top_k, top_p) bytes
 *
 * Same conventions, limits and status codes as specv_verify (it is that call
 * with K = 0 and draft_len = 0 for every row); 1 <= R.  Asynchronous on
 * `stream`.
 */
SPECV_API specv_status_t specv_sample(const void *logits, specv_dtype_t dtype, const float *u,
                                      int R, int V, float temperature, int top_k, float top_p,
                                      int32_t *out_tokens, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * Per-position acceptance rates, a diagnostic: beta[b][k] =
 * sum_x min(p_k(x), q_k(x)) for every drafted position k < draft_len[b], the
 * probability that a token drawn from q_k is accepted at that position
 * (nickwang.xyz, "推测解码：草稿、验证与实际加速", section "好草稿也要算得便宜").
 * p_k, q_k are the same processed distributions as in specv_verify.  It
 * reads both rows of every drafted position (a second pass over them when
 * run next to specv_verify); draft tokens and uniforms are not needed.
 *
 *  target_logits, draft_logits, draft_len: as for specv_verify
 *  beta        [B][K] float32, device: the rates; -1 where k >= draft_len[b],
 *              draft_len[b] is outside [0, K] or a row has no finite logit
 *              (or, with filters, exceeds the kept-list capacity)
 *  workspace   at least specv_workspace_bytes(B, K, V, dtype, top_k, top_p)
 *
 * Float32 without filters (relative error ~1e-7), float64 with them.  Same
 * conventions, limits and status codes as specv_verify.  Asynchronous.
 */
SPECV_API specv_status_t specv_acceptance_rates(const void *target_logits,
                                                const void *draft_logits, specv_dtype_t dtype,
                                                const int32_t *draft_len, int B, int K, int V,
                                                float temperature, int top_k, float top_p,
                                                float *beta, void *workspace,
                                                size_t workspace_bytes, hipStream_t stream);

/*
 * Statistics of one verified round (nickwang.xyz, "推测解码：草稿、验证与实际加速",
 * section "好草稿也要算得便宜": count the tokens a round really commits; its
 * measurement table under "在相同负载和质量下比较" keeps the draft acceptance
 * apart from the useful output).  The inputs are one specv_verify call's
 * inputs and outputs, unchanged.
 *
 *  draft_tokens, draft_len   [B][K], [B] int32, device: as passed to specv_verify
 *                            (draft_tokens may be NULL when K == 0)
 *  out_tokens, n_emitted     [B][K+1], [B] int32, device: as specv_verify wrote them
 *  beta        [B][K] float32, device, or NULL: rates from specv_acceptance_rates
 *  accepted    [B] int32, device, or NULL: accepted drafts of each request, i.e.
 *              the emitted tokens that are drafts the verifier accepted (all
 *              but the last, or all when an accepted EOS stopped the round);
 *              -1 for a failed round (n_emitted < 1 or inconsistent with
 *              draft_len).  When the verifier had to fall back from an empty
 *              residual (a flagged case, impossible in exact arithmetic) and
 *              redrew the rejected token, that round reads as an EOS stop.
 *  expected    [B] float32, device, or NULL (needs beta): E[N] of the
 *              request's round if its drafted positions accepted independently
 *              with rates beta[b][0..draft_len-1]: 1 + b0 + b0 b1 + ...;
 *              -1 when draft_len is outside [0, K] or a rate is negative
 *  totals      [SPECV_NUM_TOTALS] int64, device, or NULL: batch sums indexed by
 *              specv_total_t (failed rounds count only as errors)
 *
 * B >= 1, 0 <= K <= SPECV_MAX_K; arrays element-aligned.  SPECV_EINVAL for
 * bad sizes, NULL required pointers or expected without beta.
 * Asynchronous on `stream`; allocates nothing.
 */
typedef enum {
  SPECV_TOTAL_REQUESTS = 0,     /* rounds that verified */
  SPECV_TOTAL_ERRORS = 1,       /* failed rounds */
  SPECV_TOTAL_DRAFTED = 2,      /* sum of draft_len */
  SPECV_TOTAL_ACCEPTED = 3,     /* sum of accepted drafts */
  SPECV_TOTAL_EMITTED = 4,      /* sum of n_emitted */
  SPECV_TOTAL_EOS_STOPS = 5,    /* rounds stopped by an accepted EOS */
  SPECV_TOTAL_FULL_ACCEPTS = 6, /* rounds that accepted every draft (a bonus was drawn) */
  SPECV_TOTAL_REJECTIONS = 7,   /* rounds that ended on a rejection (a correction) */
  SPECV_NUM_TOTALS = 8
} specv_total_t;

SPECV_API specv_status_t specv_round_stats(const int32_t *draft_tokens, const int32_t *draft_len,
                                           const int32_t *out_tokens, const int32_t *n_emitted,
                                           const float *beta, int B, int K, int32_t *accepted,
                                           float *expected, int64_t *totals, hipStream_t stream);

/* Largest monitor window, in rounds. */
#define SPECV_MAX_WINDOW 4096

/*
 * Adaptive draft length (tbxsx.cn, "推测解码采样验证优化策略 —— 深度调研报告",
 * section "4. 实现逻辑": an acceptance-rate monitor over a window of rounds, and
 * a draft length that moves one step up when the rate is above 0.85, at most
 * to the maximum draft length, and one step down when it is below 0.60, at
 * least to 1).  Every request has its own window in `state`: the ratio of its
 * accepted drafts (as specv_round_stats counts them) to its drafted positions
 * over its last `window` verified rounds.  The thresholds are applied exactly
 * as 17/20 and 3/5, strictly.
 *
 * specv_monitor_state_bytes(B, window): bytes of state for B requests (0 when
 *   B < 1 or window is outside [1, SPECV_MAX_WINDOW]).  The caller owns it:
 *   device memory, 16-byte aligned.
 * specv_monitor_reset: empties every window; needed before the first update
 *   and when window changes.  A fill kernel, so it may be captured in a graph.
 * specv_monitor_update, after a specv_verify call with the same B and K:
 *   draft_tokens, draft_len, out_tokens, n_emitted  as for specv_round_stats
 *   next_draft_len [B] int32, device: the draft length of each request's next
 *                 round, in [1, max_k]: draft_len[b] moved by the rule (kept
 *                 as it is while the window has no drafted position).  It may
 *                 be the draft_len array itself (updated in place).
 *   rate          [B] float64, device, or NULL: the window's rate after this
 *                 round, the correctly rounded quotient; -1 when undefined
 *   1 <= max_k <= SPECV_MAX_K.  A failed round adds nothing to its window.
 *   A state header that no reset wrote restarts that request's window.
 * Both asynchronous on `stream`; they allocate nothing.  Updates of one state
 * must not overlap (use one stream).
 */
SPECV_API size_t specv_monitor_state_bytes(int B, int window);
SPECV_API specv_status_t specv_monitor_reset(void *state, int B, int window, hipStream_t stream);
SPECV_API specv_status_t specv_monitor_update(const int32_t *draft_tokens,
                                              const int32_t *draft_len,
                                              const int32_t *out_tokens,
                                              const int32_t *n_emitted, int B, int K, int max_k,
                                              int window, void *state, int32_t *next_draft_len,
                                              double *rate, hipStream_t stream);

/*
 * LM-head weights in the order the fused call reads them.  The weights are a
 * model constant: pack them once, when the model is loaded, and pass the
 * packed copy to every specv_verify_lm_head call.
 *
 * The packed matrix is [ceil(V/128)][D/64][4][4][64] 16-byte pieces of bf16;
 * piece (t, kb, w, s, l) holds lm_head_weight[128 t + 32 w + l % 32][64 kb +
 * 32 (l / 32) + 8 s .. + 7], and zeros for vocabulary ids >= V.  Each load
 * instruction of the LM-head kernel then reads 1 KB of consecutive bytes and
 * each workgroup streams one contiguous range, instead of 128 rows D * 2
 * bytes apart.
 *
 * specv_lm_head_packed_weight_bytes: ceil(V/128) * 128 * D * 2, or 0 for
 * invalid sizes (V outside [1, SPECV_MAX_V], D not a positive multiple of 64
 * or above SPECV_MAX_D).
 *
 * specv_lm_head_pack_weight:
 *  lm_head_weight  [V][D] bf16 row-major, device, 16-byte aligned (read only).
 *  packed_weight   device output of specv_lm_head_packed_weight_bytes(V, D)
 *                  bytes, 16-byte aligned, not overlapping lm_head_weight.
 * SPECV_EINVAL for invalid sizes, null, misaligned or overlapping pointers;
 * SPECV_EHIP if the launch fails.  Asynchronous on `stream`; allocates
 * nothing.
 */
SPECV_API size_t specv_lm_head_packed_weight_bytes(int V, int D);
SPECV_API specv_status_t specv_lm_head_pack_weight(const void *lm_head_weight,
                                                   void *packed_weight, int V, int D,
                                                   hipStream_t stream);

/*
 * The verification step fused with the target model's LM head (tbxsx.cn,
 * "推测解码采样验证优化策略 —— 深度调研报告", section "6. 扩展性与安全性": fuse the
 * verification-stage forward pass of the target model with the sampling
 * step).  The target logits are computed on the matrix cores from the target
 * model's final hidden states, logits[b][k][v] = sum_d hidden[b][k][d] *
 * weight[v][d] (bf16 products, float32 accumulation, rounded to bf16
 * nearest-even).  Without top-k / top-p the softmax statistics of each target
 * row are taken in the same kernel, from the rounded values, before the
 * logits leave the chip, and the rest is specv_verify on those logits; with
 * top-k / top-p (whose select needs the whole rows) the filtered
 * specv_verify path runs on the logits the LM head wrote.
 *
 *  hidden          [B][K+1][D] bf16, device, 16-byte aligned: the hidden state
 *                  that produces target row k of request b.
 *  packed_weight   the LM-head weight [V][D] bf16 as specv_lm_head_pack_weight
 *                  writes it for this V and D; device, 16-byte aligned.
 *  D               > 0, a multiple of 64, <= SPECV_MAX_D.
 *  target_logits   [B][K+1][V] bf16, device output: the LM head's logits
 *                  (every row, whatever draft_len is); the draws read it.
 *  draft_logits, draft_tokens, draft_len, u, u_final, B, K, V, temperature,
 *  top_k, top_p, eos_id, out_tokens, n_emitted: as for specv_verify (bf16
 *                  draft logits).
 *  workspace       at least specv_lm_head_workspace_bytes(B, K, V, D, top_k,
 *                  top_p) bytes, 16-byte aligned; no initialisation needed.
 *  accept_prob, residual_mass, stop_pos, path: nullable diagnostics, as for
 *                  specv_verify_debug.
 *
 * Status codes as specv_verify; SPECV_EINVAL also for D not a multiple of
 * 64 or misaligned hidden / packed weight.  Per-request errors as specv_verify.
 * Asynchronous on `stream`; allocates nothing.
 */
SPECV_API size_t specv_lm_head_workspace_bytes(int B, int K, int V, int D, int top_k,
                                               float top_p);
SPECV_API specv_status_t specv_verify_lm_head(const void *hidden, const void *packed_weight,
                                              const void *draft_logits,
                                              const int32_t *draft_tokens,
                                              const int32_t *draft_len, const float *u,
                                              const float *u_final, int B, int K, int V, int D,
                                              float temperature, int top_k, float top_p,
                                              int eos_id, void *target_logits,
                                              int32_t *out_tokens, int32_t *n_emitted,
                                              void *workspace, size_t workspace_bytes,
                                              hipStream_t stream, float *accept_prob,
                                              double *residual_mass, int32_t *stop_pos,
                                              int32_t *path);

/*
 * Timing variant of specv_verify, for benchmarks: identical work, plus
 * hipEventRecord on `stream` of events[0] before the first kernel launch and
 * of events[i+1] after kernel stage i.  `events` holds specv_num_stages(p) + 1
 * caller-created HIP events, p = specv_path_kind(B, K, V, top_k, top_p) (SPECV_EINVAL
 * if NULL or any of those entries is NULL); the caller reads stage durations
 * with hipEventElapsedTime after synchronising.  The stages differ by path
 * (specv_stage_name).
 */
SPECV_API specv_status_t specv_verify_timed(const void *target_logits, const void *draft_logits,
                                            specv_dtype_t dtype, const int32_t *draft_tokens,
                                            const int32_t *draft_len, const float *u,
                                            const float *u_final, int B, int K, int V,
                                            float temperature, int top_k, float top_p,
                                            int eos_id, int32_t *out_tokens, int32_t *n_emitted,
                                            void *workspace, size_t workspace_bytes,
                                            hipStream_t stream, hipEvent_t *events);

/* Which kernel path a call with these sizes and settings takes: 0 without
 * filters (row statistics, accept scan, float64 chunk pass, draw: four
 * kernels), 1 top-k / top-p through the candidate select, 2 top-k / top-p
 * through the radix select, 3 without filters at small sizes (one kernel:
 * the row statistics, the chunk pass of every row pair the request could
 * draw from, and the accept scan with the draw from the pair it picks, each
 * stage reading the previous one's results through tagged words in the
 * workspace as soon as they land; tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告",
 * section "6. 扩展性与安全性", operator fusion against launch overhead).
 * Paths 0 and 3 give the same tokens but for a draw within float64 rounding
 * of a CDF edge (their draws sum over other chunk sizes, so residual masses
 * agree to rounding). */
SPECV_API int specv_path_kind(int B, int K, int V, int top_k, float top_p);
/* Sets the size up to which unfiltered calls take path 3: calls with
 * B * (K+1) * ceil(V / 2048) <= limit do (default 384; 0 turns the path
 * off, a huge value forces it).  Process-wide, for all devices; returns the
 * previous limit.  A call made while another thread changes the limit may
 * take either path; workspace sizes follow the limit in force. */
SPECV_API long long specv_set_small_batch_limit(long long limit);
/* Number of kernel stages a call on path `kind` launches (0 for an unknown
 * kind), and the static name of stage i (NULL when out of range). */
SPECV_API int specv_num_stages(int kind);
SPECV_API const char *specv_stage_name(int kind, int i);

/* Static, human-readable name of a status code. */
SPECV_API const char *specv_status_string(specv_status_t status);

/* Library version, 100 * major + minor. */
SPECV_API int specv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
