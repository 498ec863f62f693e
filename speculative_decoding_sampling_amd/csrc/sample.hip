// Residual / bonus sampler, float64 end to end, for the one row pair (after a
// rejection) or the one target row (after full acceptance) of each request.
//
// After a rejection at position j the correction token is drawn from
// r(v) = max(p_j(v) - q_j(v), 0) renormalised (nickwang.xyz
// "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布", eq. r(x);
// tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告", formula 4; bowenzhou.top
// "投机采样", section "深入推导").  After full acceptance the bonus token is
// drawn from p_n (nickwang.xyz, section "候选已知，验证才能并行").  Either draw
// is an inverse-CDF draw at u_final over token ids in ascending order with a
// strict comparison (same page, section "算完三个 token 的全部概率", sample()).
// When p == q every draft is accepted, so the residual is never formed.
//
// Precision.  Over a 128k vocabulary one token's CDF interval is ~1e-5 wide,
// so a float32 pipeline moves the drawn token in a large fraction of draws.
// Everything here -- exp, both normalisers, the residual and the prefix
// sums -- is float64, recomputed from the logits (the float32 row statistics
// are used only for the exact row maxima).
//
// Three launches: (a) per chunk, float64 sums of exp((z - M) / T) over the
// target and draft rows; (b) per chunk, the residual mass with the full
// normalisers; (c) per request, a blocked prefix over chunk masses finds the
// chunk holding t = u_final * total, and an in-chunk blocked scan finds the
// token.  All sums run in a fixed order, so the draw is deterministic.
#include <climits>

#include "common.h"

namespace specv {

template <typename T>
__device__ __forceinline__ void load8(const T* __restrict__ row, long e0, int V, bool aligned,
                                      float* out) {
  constexpr int N = Elem<T>::kPerVec;
#pragma unroll
  for (int j = 0; j < kSampPerThread / N; ++j) load_vec(row, e0 + j * N, V, aligned, out + j * N);
}

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Sum of one double per thread over the block, in a fixed order.
__device__ __forceinline__ double block_sum(double v, double* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kSampThreads / kWave; ++w) s += lds[w];
  return s;
}

// Exclusive prefix of one double per thread over the block (thread order),
// and the block total.  Fixed order, so every call with the same inputs gives
// the same bits.
__device__ __forceinline__ double block_exclusive_scan(double v, double* lds, double& total) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  double x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  double excl = __shfl_up(x, 1, kWave);
  if (lane == 0) excl = 0.0;
  __syncthreads();
  if (lane == kWave - 1) lds[wid] = x;
  __syncthreads();
  double off = 0.0;
  total = 0.0;
#pragma unroll
  for (int w = 0; w < kSampThreads / kWave; ++w) {
    if (w < wid) off += lds[w];
    total += lds[w];
  }
  return off + excl;
}

__device__ __forceinline__ int block_min(int v, int* lds) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  int r = lds[0];
#pragma unroll
  for (int w = 1; w < kSampThreads / kWave; ++w) r = min(r, lds[w]);
  return r;
}

__device__ __forceinline__ int block_max(int v, int* lds) { return -block_min(-v, lds); }

// Row normalisers from the per-chunk partials, summed by one wave in a fixed
// order (lane-strided, then butterfly).  Called by every thread of wave 0.
__device__ __forceinline__ double2 chunk_totals(const double2* __restrict__ p, int n) {
  double a = 0.0, d = 0.0;
  for (int i = threadIdx.x % kWave; i < n; i += kWave) {
    a += p[i].x;
    d += p[i].y;
  }
  return make_double2(wave_sum(a), wave_sum(d));
}

// (a) float64 chunk sums of exp((z - M) / T) for the sampled rows.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_norm_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, int K, int V, int nch, double invT,
    const Plan* __restrict__ plan, double2* __restrict__ norm_part) {
  __shared__ double lds[kSampThreads / kWave];
  const int c = blockIdx.x % nch, b = blockIdx.x / nch;
  const Plan pl = plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;
  const long e0 = (long)c * kSampChunk + (long)threadIdx.x * kSampPerThread;
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  float z[kSampPerThread];
  load8(trow, e0, V, aligned16(trow), z);
  const double mt = pl.mt;
  double st = 0.0;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) st += exp(((double)z[i] - mt) * invT);
  double sd = 0.0;
  if (pl.path == kPathReject) {
    const T* drow = dft + draft_row_off(b, pl.drow, K, V);
    load8(drow, e0, V, aligned16(drow), z);
    const double md = pl.md;
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) sd += exp(((double)z[i] - md) * invT);
  }
  st = block_sum(st, lds);
  sd = block_sum(sd, lds);
  if (threadIdx.x == 0) norm_part[(size_t)b * nch + c] = make_double2(st, sd);
}

// Residual weights of this thread's 8 elements: max(et/St - ed/Sd, 0).
template <typename T>
__device__ __forceinline__ void residual8(const T* trow, const T* drow, long e0, int V,
                                          double mt, double md, double invT, double St,
                                          double Sd, double* w) {
  float zt[kSampPerThread], zd[kSampPerThread];
  load8(trow, e0, V, aligned16(trow), zt);
  load8(drow, e0, V, aligned16(drow), zd);
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) {
    const double p = exp(((double)zt[i] - mt) * invT) / St;
    const double q = exp(((double)zd[i] - md) * invT) / Sd;
    const double r = p - q;
    w[i] = r > 0.0 ? r : 0.0;
  }
}

template <typename T>
__device__ __forceinline__ void target8(const T* trow, long e0, int V, double mt, double invT,
                                        double* w) {
  float zt[kSampPerThread];
  load8(trow, e0, V, aligned16(trow), zt);
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) w[i] = exp(((double)zt[i] - mt) * invT);
}

// (b) per-chunk residual mass after a rejection.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_resid_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, int K, int V, int nch, double invT,
    const Plan* __restrict__ plan, const double2* __restrict__ norm_part,
    double* __restrict__ resid_part) {
  __shared__ double lds[kSampThreads / kWave];
  __shared__ double2 tot;
  const int c = blockIdx.x % nch, b = blockIdx.x / nch;
  const Plan pl = plan[b];
  if (pl.path != kPathReject) return;
  if (threadIdx.x < kWave) {
    const double2 t = chunk_totals(norm_part + (size_t)b * nch, nch);
    if (threadIdx.x == 0) tot = t;
  }
  __syncthreads();
  const long e0 = (long)c * kSampChunk + (long)threadIdx.x * kSampPerThread;
  double w[kSampPerThread];
  residual8(tgt + target_row_off(b, pl.trow, K, V), dft + draft_row_off(b, pl.drow, K, V), e0, V,
            (double)pl.mt, (double)pl.md, invT, tot.x, tot.y, w);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) s += w[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) resid_part[(size_t)b * nch + c] = s;
}

// (c) the draw itself: one workgroup per request.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_draw_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const float* __restrict__ u_final,
    int K, int V, int nch, double invT, const Plan* __restrict__ plan,
    const double2* __restrict__ norm_part, const double* __restrict__ resid_part,
    int* __restrict__ out_tokens, double* __restrict__ rmass_out) {
  __shared__ double lds[kSampThreads / kWave];
  __shared__ int ilds[kSampThreads / kWave];
  __shared__ double2 tot;
  const int b = blockIdx.x;
  const Plan pl = plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;
  const double2* np = norm_part + (size_t)b * nch;
  if (threadIdx.x < kWave) {
    const double2 t = chunk_totals(np, nch);
    if (threadIdx.x == 0) tot = t;
  }
  __syncthreads();
  const double St = tot.x, Sd = tot.y;

  // Chunk weights: residual masses after a rejection, target masses for the
  // bonus.  A rejection whose residual rounds to zero everywhere (not
  // reachable in exact arithmetic) falls back to p_j.
  bool use_resid = pl.path == kPathReject;
  const int q = (nch + kSampThreads - 1) / kSampThreads;
  const int c_lo = min(nch, (int)threadIdx.x * q), c_hi = min(nch, c_lo + q);
  double total = 0.0;
  double mine = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    mine = 0.0;
    for (int cc = c_lo; cc < c_hi; ++cc) mine += use_resid ? resid_part[(size_t)b * nch + cc] : np[cc].x;
    const double s = block_sum(mine, lds);
    total = s;
    if (!(use_resid && s == 0.0)) break;
    use_resid = false;
  }
  const double rmass = pl.path == kPathReject ? (use_resid ? total : 0.0) : 0.0;

  const double t = (double)u_final[b] * total;
  double tot2;
  const double excl = block_exclusive_scan(mine, lds, tot2);
  // First chunk whose inclusive prefix exceeds t.
  int cand = INT_MAX, last_pos = -1;
  {
    double run = excl;
    for (int cc = c_lo; cc < c_hi; ++cc) {
      const double wc = use_resid ? resid_part[(size_t)b * nch + cc] : np[cc].x;
      run += wc;
      if (cand == INT_MAX && t < run) cand = cc;
      if (wc > 0.0) last_pos = cc;
    }
  }
  int cstar = block_min(cand, ilds);
  double tprime;
  if (cstar == INT_MAX) {                         // rounding fall-through: last chunk with mass
    cstar = block_max(last_pos, ilds);
    tprime = INFINITY;
    if (cstar < 0) {                              // no positive mass at all (non-finite input)
      if (threadIdx.x == 0) {
        out_tokens[(size_t)b * (K + 1) + pl.stop] = -1;
        if (rmass_out) rmass_out[b] = rmass;
      }
      return;
    }
  } else {
    // exclusive prefix of chunk cstar, recomputed by its owner thread
    __shared__ double cpre;
    if (cstar >= c_lo && cstar < c_hi) {
      double run = excl;
      for (int cc = c_lo; cc < cstar; ++cc) run += use_resid ? resid_part[(size_t)b * nch + cc] : np[cc].x;
      cpre = run;
    }
    __syncthreads();
    tprime = t - cpre;
  }

  const long e0 = (long)cstar * kSampChunk + (long)threadIdx.x * kSampPerThread;
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  double w[kSampPerThread];
  if (use_resid)
    residual8(trow, dft + draft_row_off(b, pl.drow, K, V), e0, V, (double)pl.mt, (double)pl.md,
              invT, St, Sd, w);
  else
    target8(trow, e0, V, (double)pl.mt, invT, w);
  double mysum = 0.0;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) mysum += w[i];
  double ctot;
  const double ex = block_exclusive_scan(mysum, lds, ctot);
  int vc = INT_MAX, vlast = -1;
  double run = ex;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) {
    run += w[i];
    if (vc == INT_MAX && tprime < run) vc = (int)(e0 + i);
    if (w[i] > 0.0) vlast = (int)(e0 + i);
  }
  int y = block_min(vc, ilds);
  if (y == INT_MAX) y = block_max(vlast, ilds);   // rounding fall-through inside the chunk
  if (threadIdx.x == 0) {
    out_tokens[(size_t)b * (K + 1) + pl.stop] = y;
    if (rmass_out) rmass_out[b] = rmass;
  }
}

template <typename T>
static hipError_t sample_norm_t(const void* tgt, const void* dft, int B, int K, int V, int nch,
                                double invT, const Plan* plan, double2* norm_part,
                                hipStream_t stream) {
  const size_t blocks = (size_t)B * nch;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  sample_norm_kernel<T><<<dim3((unsigned)blocks), dim3(kSampThreads), 0, stream>>>(
      static_cast<const T*>(tgt), static_cast<const T*>(dft), K, V, nch, invT, plan, norm_part);
  return hipGetLastError();
}

template <typename T>
static hipError_t sample_resid_t(const void* tgt, const void* dft, int B, int K, int V, int nch,
                                 double invT, const Plan* plan, const double2* norm_part,
                                 double* resid_part, hipStream_t stream) {
  const size_t blocks = (size_t)B * nch;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  sample_resid_kernel<T><<<dim3((unsigned)blocks), dim3(kSampThreads), 0, stream>>>(
      static_cast<const T*>(tgt), static_cast<const T*>(dft), K, V, nch, invT, plan, norm_part,
      resid_part);
  return hipGetLastError();
}

template <typename T>
static hipError_t sample_draw_t(const void* tgt, const void* dft, const float* u_final, int B,
                                int K, int V, int nch, double invT, const Plan* plan,
                                const double2* norm_part, const double* resid_part,
                                int* out_tokens, double* rmass_out, hipStream_t stream) {
  sample_draw_kernel<T><<<dim3(B), dim3(kSampThreads), 0, stream>>>(
      static_cast<const T*>(tgt), static_cast<const T*>(dft), u_final, K, V, nch, invT, plan,
      norm_part, resid_part, out_tokens, rmass_out);
  return hipGetLastError();
}

hipError_t launch_sample_norm(bool bf16, const void* tgt, const void* dft, int B, int K, int V,
                              int nch, double invT, const Plan* plan, double2* norm_part,
                              hipStream_t stream) {
  return bf16 ? sample_norm_t<bf16_t>(tgt, dft, B, K, V, nch, invT, plan, norm_part, stream)
              : sample_norm_t<float>(tgt, dft, B, K, V, nch, invT, plan, norm_part, stream);
}

hipError_t launch_sample_resid(bool bf16, const void* tgt, const void* dft, int B, int K, int V,
                               int nch, double invT, const Plan* plan, const double2* norm_part,
                               double* resid_part, hipStream_t stream) {
  return bf16 ? sample_resid_t<bf16_t>(tgt, dft, B, K, V, nch, invT, plan, norm_part, resid_part,
                                       stream)
              : sample_resid_t<float>(tgt, dft, B, K, V, nch, invT, plan, norm_part, resid_part,
                                      stream);
}

hipError_t launch_sample_draw(bool bf16, const void* tgt, const void* dft, const float* u_final,
                              int B, int K, int V, int nch, double invT, const Plan* plan,
                              const double2* norm_part, const double* resid_part,
                              int* out_tokens, double* rmass_out, hipStream_t stream) {
  return bf16 ? sample_draw_t<bf16_t>(tgt, dft, u_final, B, K, V, nch, invT, plan, norm_part,
                                      resid_part, out_tokens, rmass_out, stream)
              : sample_draw_t<float>(tgt, dft, u_final, B, K, V, nch, invT, plan, norm_part,
                                     resid_part, out_tokens, rmass_out, stream);
}

}  // namespace specv
