/*
 * libspecverify self-test hooks (not part of the verification API).
 *
 * These expose internal device routines so tests can check them directly
 * against a float64 reference.
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

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_SELFTEST_H */
