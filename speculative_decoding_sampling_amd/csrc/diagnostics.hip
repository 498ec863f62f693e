// Acceptance diagnostics: the per-position acceptance rate
// beta_k = sum_x min(p_k(x), q_k(x)) (nickwang.xyz "推测解码：草稿、验证与实际加速",
// section "好草稿也要算得便宜": the acceptance rate of a fixed prefix), for every
// drafted position of a batch.
//
// Without filters it needs a second pass over both rows of every drafted
// position (p and q normalised): beta_pass streams each (request, position,
// chunk) with the row-statistics kernel's layout, rebuilds the two rows'
// float32 (max, normaliser) from the chunk partials, and sums min(p, q) over
// the chunk in float32; beta_finish adds the chunk sums in chunk order.  A
// diagnostic needs no more than float32: the sum's relative error is ~1e-7.
// With top-k / top-p, p is zero off the target row's kept list, so
// beta_list walks that list (float64, as the filtered sampler does).
#include "common.h"
#include "exp64.h"

namespace specv {

// (max, normaliser) of one row from its chunk partials, by one wave: lane l
// combines partials l, l + 64, ... in order, then the wave combines lanes.
__device__ __forceinline__ void wave_row_stats(const float2* __restrict__ p, int n, float c,
                                               float& M, float& S) {
  const int lane = threadIdx.x % kWave;
  float m = -INFINITY, s = 0.f;
  for (int i = lane; i < n; i += kWave) {
    const float2 v = p[i];
    if (v.x == -INFINITY) continue;
    if (v.x > m) {
      if (m != -INFINITY) s *= __builtin_amdgcn_exp2f(__fmul_rn(m, c) - __fmul_rn(v.x, c));
      m = v.x;
      s += v.y;
    } else {
      s += v.y * __builtin_amdgcn_exp2f(__fmul_rn(v.x, c) - __fmul_rn(m, c));
    }
  }
  M = wave_max(m);
  const float scaled = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(__fmul_rn(m, c) - __fmul_rn(M, c));
  S = wave_sum(scaled);
}

// The same from one partial per lane (lanes past the row hold (-inf, 0)): what
// the loop above computes when n <= kWave, so a caller can issue the loads
// of several rows before the first wait.
__device__ __forceinline__ void wave_row_stats1(float2 v, float c, float& M, float& S) {
  const float m = v.x;
  const float s = m == -INFINITY ? 0.f : v.y;
  M = wave_max(m);
  const float scaled = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(__fmul_rn(m, c) - __fmul_rn(M, c));
  S = wave_sum(scaled);
}

template <typename T, int VECS>
__global__ __launch_bounds__(kRowThreads) void beta_pass_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    int K, int V, int nchunk, float c, const float2* __restrict__ part,
    float* __restrict__ beta_part) {
  constexpr int N = Elem<T>::kPerVec;
  constexpr int kChunk = kRowThreads * VECS * N;
  const int chunk = blockIdx.x % nchunk;
  const int bk = blockIdx.x / nchunk;
  const int k = bk % K, b = bk / K;
  const int nb = draft_len[b];
  if (nb < 0 || nb > K || k >= nb) return;            // the finish writes -1
  const int R = 2 * K + 1;
  const T* trow = tgt + target_row_off(b, k, K, V);
  const T* drow = dft + draft_row_off(b, k, K, V);

  // This chunk's logits of both rows, requested first; each wave rebuilds
  // the two rows' statistics from the partials meanwhile.
  uint4 wt[VECS], wd[VECS];
  const long e_base = (long)chunk * kChunk;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const long e_wave = e_base + (long)wid * VECS * kWave * N + (long)lane * N;
  const bool aligned = aligned16(trow) && aligned16(drow);
  if (aligned && e_base + kChunk <= V) {
#pragma unroll
    for (int j = 0; j < VECS; ++j) {
      wt[j] = load_raw_stream(trow, e_wave + (long)j * kWave * N);
      wd[j] = load_raw_stream(drow, e_wave + (long)j * kWave * N);
    }
  } else {
#pragma unroll
    for (int j = 0; j < VECS; ++j) {
      wt[j] = load_raw_checked(trow, e_wave + (long)j * kWave * N, V, aligned);
      wd[j] = load_raw_checked(drow, e_wave + (long)j * kWave * N, V, aligned);
    }
  }
  float Mt, St, Md, Sd;
  const float2* pt = part + ((size_t)b * R + k) * nchunk;
  const float2* pd = part + ((size_t)b * R + K + 1 + k) * nchunk;
  if (nchunk <= kWave) {
    // both rows' partials requested together: one wait covers them and the logits
    const float2 none = make_float2(-INFINITY, 0.f);
    const float2 vt = lane < nchunk ? pt[lane] : none;
    const float2 vd = lane < nchunk ? pd[lane] : none;
    wave_row_stats1(vt, c, Mt, St);
    wave_row_stats1(vd, c, Md, Sd);
  } else {
    wave_row_stats(pt, nchunk, c, Mt, St);
    wave_row_stats(pd, nchunk, c, Md, Sd);
  }
  const bool ok = Mt != -INFINITY && Md != -INFINITY;
  const float mtc = __fmul_rn(Mt, c), mdc = __fmul_rn(Md, c);
  const float rt = 1.f / St, rd = 1.f / Sd;
  float s = 0.f;
  if (ok) {
#pragma unroll
    for (int j = 0; j < VECS; ++j) {
      float zt[N], zd[N];
      unpack(wt[j], zt, T{});
      unpack(wd[j], zd, T{});
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(zt[i], c, -mtc)) * rt;
        const float q = __builtin_amdgcn_exp2f(fmaf(zd[i], c, -mdc)) * rd;
        s += fminf(p, q);
      }
    }
  }
  s = wave_sum(s);
  __shared__ float red[kRowThreads / kWave];
  if (lane == 0) red[wid] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kRowThreads / kWave; ++w) t += red[w];
    beta_part[(size_t)bk * nchunk + chunk] = ok ? t : NAN;
  }
}

// beta[b][k]: chunk sums added in chunk order; -1 where the position was not
// drafted, draft_len is out of range, or a row has no finite logit.
__global__ void beta_finish_kernel(const int* __restrict__ draft_len, int B, int K, int nchunk,
                                   const float* __restrict__ beta_part, float* __restrict__ beta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * K) return;
  const int b = i / K, k = i % K;
  const int nb = draft_len[b];
  float out = -1.f;
  if (nb >= 0 && nb <= K && k < nb) {
    double t = 0.0;
    for (int c = 0; c < nchunk; ++c) t += (double)beta_part[(size_t)i * nchunk + c];
    out = t == t ? (float)t : -1.f;                  // NaN: a row with no finite logit
  }
  beta[i] = out;
}

// Filtered path: one workgroup per (request, position); p is zero off the
// target row's kept list, so beta = sum over that list of min(p, q), q read
// from the draft row at the same id (zero unless kept there).  A target row
// whose kept set has no list (more than kKeptCap tokens) is streamed whole.
template <typename T>
__global__ __launch_bounds__(kFiltThreads) void beta_list_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    int K, int V, double invT, const FiltRow* __restrict__ rows, const Kept* __restrict__ kept,
    float* __restrict__ beta) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double red[kFiltThreads / kWave];
  const int bk = blockIdx.x;
  const int k = bk % K, b = bk / K;
  const int nb = draft_len[b];
  exp64_stage_table<kFiltThreads>(tbl);
  const int R = 2 * K + 1;
  const bool drafted = nb >= 0 && nb <= K && k < nb;
  FiltRow tr, dr;
  if (drafted) {
    tr = rows[(size_t)b * R + k];
    dr = rows[(size_t)b * R + K + 1 + k];
  }
  __syncthreads();
  if (!drafted || tr.status != 0 || dr.status != 0) {   // uniform per block
    if (threadIdx.x == 0) beta[bk] = -1.f;
    return;
  }
  const Kept* list = kept + ((size_t)b * R + k) * kKeptCap;
  const T* drow = dft + draft_row_off(b, k, K, V);
  auto q_at = [&](float zd) -> double {
    if (!(zd >= dr.tau) || zd == -INFINITY) return 0.0;
    return exp64(((double)zd - (double)dr.m) * invT, tbl) / dr.S;
  };
  double s = 0.0;
  if (tr.count <= kKeptCap) {
    for (int i = threadIdx.x; i < tr.count; i += kFiltThreads) {
      const Kept e = list[i];
      const double p = exp64(((double)e.z - (double)tr.m) * invT, tbl) / tr.S;
      const double q = q_at(to_f32(drow[e.id]));
      s += p < q ? p : q;
    }
  } else {
    const T* trow = tgt + target_row_off(b, k, K, V);
    for (long e = threadIdx.x; e < V; e += kFiltThreads) {
      const float zt = to_f32(trow[e]);
      if (!(zt >= tr.tau) || zt == -INFINITY) continue;
      const double p = exp64(((double)zt - (double)tr.m) * invT, tbl) / tr.S;
      const double q = q_at(to_f32(drow[e]));
      s += p < q ? p : q;
    }
  }
  s = wave_sum(s);
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  if (lane == 0) red[wid] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kFiltThreads / kWave; ++w) t += red[w];
    beta[bk] = (float)t;
  }
}

hipError_t launch_beta(bool bf16, bool filt, const void* tgt, const void* dft,
                       const int* draft_len, int B, int K, int V, int nch_row, float c,
                       double invT, const float2* part, const FiltRow* frows, const Kept* kept,
                       float* beta_part, float* beta, hipStream_t stream) {
  if (K == 0) return hipSuccess;
  if (filt) {
    const size_t blocks = (size_t)B * K;
    if (bf16)
      beta_list_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kFiltThreads), 0, stream>>>(
          static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), draft_len, K, V, invT,
          frows, kept, beta);
    else
      beta_list_kernel<float><<<dim3((unsigned)blocks), dim3(kFiltThreads), 0, stream>>>(
          static_cast<const float*>(tgt), static_cast<const float*>(dft), draft_len, K, V, invT,
          frows, kept, beta);
    return hipGetLastError();
  }
  const size_t blocks = (size_t)B * K * nch_row;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (bf16)
    beta_pass_kernel<bf16_t, kRowVecs><<<dim3((unsigned)blocks), dim3(kRowThreads), 0, stream>>>(
        static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), draft_len, K, V,
        nch_row, c, part, beta_part);
  else
    beta_pass_kernel<float, kRowVecs><<<dim3((unsigned)blocks), dim3(kRowThreads), 0, stream>>>(
        static_cast<const float*>(tgt), static_cast<const float*>(dft), draft_len, K, V, nch_row,
        c, part, beta_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = B * K;
  beta_finish_kernel<<<dim3((n + 255) / 256), dim3(256), 0, stream>>>(draft_len, B, K, nch_row,
                                                                     beta_part, beta);
  return hipGetLastError();
}

}  // namespace specv
