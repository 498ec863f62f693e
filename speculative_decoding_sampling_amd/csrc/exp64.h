// Table-driven float64 exp for the sampler (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989), with N = 512 table entries.
//
//   x = (k / N) ln2 + r,  k = rint(x N / ln2),  |r| <= ln2 / (2N) ~ 6.8e-4
//   (k comes from adding 1.5 * 2^52, which rounds to an integer in one FMA)
//   exp(x) = 2^(k >> 9) * 2^((k & 511) / 512) * (1 + p(r)),
//   p(r) = r + r^2/2 + r^3/6   (truncation r^4/24 < 8.8e-15)
//
// r = x - k * (ln2/N) is one FMA with ln2/N rounded to float64, which adds a
// relative error of at most |x| * 2^-53.  Relative error in total: below
// 1e-14 + |x| * 1.2e-16 (below 1.5e-14 where x >= -40, the only range whose
// weights reach a sum's last bits), four orders of magnitude inside what the
// sampler needs (its draws are resolved to 1e-10 of the total mass).
// Valid for x <= 709; x below about -745.1 (including -inf) returns 0.  The
// constants come from gen_exp64_table.py.
#pragma once

#include <hip/hip_runtime.h>

#include "exp64_table.h"

namespace specv {

static __device__ const double kExp64Table[SPECV_EXP64_N] = SPECV_EXP64_TABLE;

// The 4 KB table staged in LDS by a block of NT threads, in two steps so a
// kernel can request its entries together with its other independent loads
// and write them to LDS once those are in flight: fetch() issues this
// thread's global loads (no wait in between), store() writes them.  Every
// thread of the block calls both, then __syncthreads() before the first exp64.
template <int NT>
struct Exp64Stage {
  static_assert(SPECV_EXP64_N % NT == 0, "block size must divide the table");
  static constexpr int kPer = SPECV_EXP64_N / NT;
  double v[kPer];
  __device__ __forceinline__ void fetch() {
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = kExp64Table[threadIdx.x + i * NT];
  }
  __device__ __forceinline__ void store(double* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) lds[threadIdx.x + i * NT] = v[i];
  }
};

// Both steps at once, for a block of NT threads.
template <int NT>
__device__ __forceinline__ void exp64_stage_table(double* lds) {
  Exp64Stage<NT> st;
  st.fetch();
  st.store(lds);
}

__device__ __forceinline__ double exp64(double x, const double* __restrict__ tbl) {
  x = fmax(x, -746.0);                              // -inf and deep underflow -> 0 below
  // t = 1.5 * 2^52 + rint(x * N / ln2): its low 32 bits are k as an integer.
  const double t = fma(x, SPECV_EXP64_INV_L, SPECV_EXP64_SHIFT);
  const double kd = t - SPECV_EXP64_SHIFT;
  const int k = (int)(unsigned)__double_as_longlong(t);
  const double r = fma(-kd, SPECV_EXP64_L, x);
  double q = fma(r, SPECV_EXP64_C3, 0.5);
  q = fma(r, q, 1.0);
  const double p = r * q;                           // exp(r) - 1
  const double tj = tbl[k & (SPECV_EXP64_N - 1)];
  return ldexp(fma(tj, p, tj), k >> SPECV_EXP64_LOG2N);   // floor(k / N)
}

// exp((z - m) / T) for a logit z, with mi = m / T precomputed: the argument
// is z / T - m / T formed with one rounding.
__device__ __forceinline__ double exp64_logit(float z, double invT, double mi,
                                              const double* __restrict__ tbl) {
  return exp64(fma((double)z, invT, -mi), tbl);
}

}  // namespace specv
