// Table-driven float64 exp for the sampler (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989), with N = 256 table entries.
//
//   x = (k / N) ln2 + r,  k = rint(x N / ln2),  |r| <= ln2 / (2N) ~ 1.35e-3
//   exp(x) = 2^(k >> 8) * 2^((k & 255) / 256) * (1 + p(r)),
//   p(r) = r + r^2/2 + r^3/6 + r^4/24   (truncation < r^5/120 < 4e-17)
//
// ln2/N is split into a 32-bit head (k * head is exact for |k| < 2^21) and a
// tail, so r carries full float64 accuracy.  Error: about 1 ulp over the
// whole range.  Valid for x <= 709; x below about -745.1 (including -inf)
// returns 0.  The constants come from gen_exp64_table.py.
#pragma once

#include <hip/hip_runtime.h>

#include "exp64_table.h"

namespace specv {

static __device__ const double kExp64Table[SPECV_EXP64_N] = SPECV_EXP64_TABLE;

// Stage the 2 KB table in LDS; every thread of the block must call this,
// followed by __syncthreads() before the first exp64.
__device__ __forceinline__ void exp64_stage_table(double* lds) {
  for (int i = threadIdx.x; i < SPECV_EXP64_N; i += blockDim.x) lds[i] = kExp64Table[i];
}

__device__ __forceinline__ double exp64(double x, const double* __restrict__ tbl) {
  x = fmax(x, -746.0);                              // -inf and deep underflow -> 0 below
  const double kd = rint(x * SPECV_EXP64_INV_L);
  double r = fma(-kd, SPECV_EXP64_L_HI, x);
  r = fma(-kd, SPECV_EXP64_L_LO, r);
  const int k = (int)kd;
  double q = fma(r, SPECV_EXP64_C4, SPECV_EXP64_C3);
  q = fma(r, q, 0.5);
  q = fma(r, q, 1.0);
  const double p = r * q;                           // exp(r) - 1
  const double t = tbl[k & (SPECV_EXP64_N - 1)];
  return ldexp(fma(t, p, t), k >> 8);               // k >> 8 is floor(k / 256)
}

}  // namespace specv
