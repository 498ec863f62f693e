/*
 * libspecverify self-test and benchmark hooks (not part of the verification
 * API).
 *
 * These expose internal device routines so tests can check them directly
 * against a float64 reference, and let a benchmark time one kernel alone.
 */
#ifndef SPECVERIFY_SELFTEST_H
#define SPECVERIFY_SELFTEST_H

#include "specverify.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * y[i] = the sampler's float64 exp(x[i]) for i < n (Tang's table-driven
 * method, ACM TOMS 15(2), 1989), computed on the GPU on `stream`.  x and y
 * are device arrays of n doubles owned by the caller.  Valid for x <= 709;
 * x below about -745.1 gives 0.  Returns SPECV_EINVAL for n < 0 or null
 * arrays with n > 0, SPECV_EHIP if the launch fails.  Asynchronous.
 */
SPECV_API specv_status_t specv_selftest_exp64(const double *x, double *y, int n,
                                              hipStream_t stream);

/*
 * The row-statistics kernel alone (the first kernel of an unfiltered
 * specv_verify call), `reps` times back to back on `stream`, cycling through
 * `nsets` input sets, with `start` recorded before the first launch and
 * `stop` after the last, so (stop - start) / reps is the kernel's mean
 * duration (plus the short gap between consecutive launches).  Set i is
 * targets[i], drafts[i], draft_tokens[i], draft_lens[i]: device arrays laid
 * out as for specv_verify, all with the same dtype, B, K and V; the arrays of
 * pointers themselves are host arrays of nsets entries.  The workspace is
 * one valid for specv_verify with these sizes and no filters; its contents
 * are overwritten.  Returns SPECV_EINVAL for bad sizes, counts, temperature,
 * null or misaligned pointers or null events, SPECV_EWORKSPACE for a short
 * workspace, SPECV_EHIP if a launch or event record fails.  Asynchronous.
 */
SPECV_API specv_status_t specv_bench_row_stats(const void *const *targets,
                                               const void *const *drafts,
                                               const int32_t *const *draft_tokens,
                                               const int32_t *const *draft_lens, int nsets,
                                               specv_dtype_t dtype, int B, int K, int V,
                                               float temperature, void *workspace,
                                               size_t workspace_bytes, int reps,
                                               hipStream_t stream, hipEvent_t start,
                                               hipEvent_t stop);

/*
 * Benchmark hook: the LM-head kernel of specv_verify_lm_head alone (logits
 * and their per-256-id tile statistics), `reps` launches on `stream` between
 * hipEventRecord(start) and hipEventRecord(stop), for the roofline.
 *
 *  hidden [M][D] bf16, packed_weight as specv_lm_head_pack_weight writes it for
 *  this V and D (device, 16-byte aligned),
 *  logits [M][V] bf16 device output; D a multiple of 64, <= SPECV_MAX_D.
 *  workspace  at least M * ceil(V / 256) * 8 bytes, 16-byte aligned (the
 *             tile statistics are written there).
 *
 * SPECV_EINVAL for bad sizes, temperature, reps, null or misaligned pointers
 * or null events; SPECV_EWORKSPACE for a short workspace; SPECV_EHIP if a
 * launch or event record fails.  Asynchronous.
 */
SPECV_API specv_status_t specv_bench_lm_head(const void *hidden, const void *packed_weight,
                                             int M, int D, int V, float temperature,
                                             void *logits, void *workspace,
                                             size_t workspace_bytes, int reps,
                                             hipStream_t stream, hipEvent_t start,
                                             hipEvent_t stop);

/*
 * Failure-handling hook: the number of times each internal wait of the
 * one-kernel small-batch path (path kind 3) polls a word before it gives up
 * and makes its request an error (n_emitted = -1, every output -1).  limit < 1
 * restores the default (2^18).  Applies to launches made after the call, from
 * any thread; returns the previous limit.  A small limit makes waits run out
 * with every kernel still ending normally, so tests can exercise that path.
 */
SPECV_API int specv_selftest_set_small_poll_limit(int limit);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_SELFTEST_H */
