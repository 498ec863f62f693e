// Gather-and-accept scan: one wave64 per request, lane k owns draft position k.
//
// Lane k combines the chunk partials of target row k and draft row k into
// the exact row maxima and the normalisers, gathers p_k(x_k) and q_k(x_k) in
// float64, forms alpha_k = min(1, p/q) and tests u[b][k] < alpha_k
// (nickwang.xyz "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布",
// eq. a(x); the strict comparison of that page's replay code).  A ballot
// finds the first rejection: every earlier draft is emitted and every later
// one discarded (section "候选已知，验证才能并行"; tbxsx.cn
// "推测解码采样验证优化策略 —— 深度调研报告", section "4. 实现逻辑").  A second
// ballot finds the first accepted EOS, which ends the round early.  The lane
// at the stop position records what the sampler must draw: a correction from
// max(p_j - q_j, 0) after a rejection, or a bonus from target row draft_len
// when all drafts pass.
//
// Latency: the kernel is a short dependency chain per request, so every load
// that does not depend on another (draft_len, u_final, tokens, uniforms and
// the partials of all K+1 target and K draft rows) is issued up front; rows
// beyond draft_len are loaded but never used.
#include "common.h"

namespace specv {

constexpr int kCombineBatch = 16;

// Combine one row's chunk partials, in chunk order.  A chunk partial s with
// maximum m is relative to 2^fl(m*c); the result S is relative to 2^fl(M*c)
// with M the row maximum.  The partials are float32 sums, so float32 scale
// factors add no meaningful error.
__device__ __forceinline__ void combine_row(const float2* __restrict__ p, int n, float c,
                                            float& M, float& S) {
  float m = -INFINITY, s = 0.f;
  for (int base = 0; base < n; base += kCombineBatch) {
    float2 v[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j)
      v[j] = base + j < n ? p[base + j] : make_float2(-INFINITY, 0.f);
    float mb = m;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) mb = fmaxf(mb, v[j].x);
    if (mb != -INFINITY) {
      const float mbc = __fmul_rn(mb, c);
      if (m != -INFINITY) s *= __builtin_amdgcn_exp2f(__fmul_rn(m, c) - mbc);
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j)
        if (v[j].x != -INFINITY) s += v[j].y * __builtin_amdgcn_exp2f(__fmul_rn(v[j].x, c) - mbc);
    }
    m = mb;
  }
  M = m;
  S = s;
}

// Probability of token x in a filtered row: exp((z - m)/T) / S if z is kept.
__device__ __forceinline__ double filt_prob(float z, const FiltRow& fr, double invT) {
  if (!(z >= fr.tau) || z == -INFINITY) return 0.0;
  return exp(((double)z - (double)fr.m) * invT) / fr.S;
}

// FILT selects the row statistics: chunk partials of the unfiltered path, or
// the per-row (max, threshold, float64 normaliser) of the top-k / top-p path.
template <typename T, bool FILT>
__global__ __launch_bounds__(kWave) void accept_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ tokens,
    const int* __restrict__ draft_len, const float* __restrict__ u,
    const float* __restrict__ u_final, int K, int V, int nchunk, float c, double invT,
    int eos_id, const float2* __restrict__ part, const FiltRow* __restrict__ frows,
    Plan* __restrict__ plan, int* __restrict__ out_tokens, int* __restrict__ n_emitted,
    float* __restrict__ alpha_out, double* __restrict__ rmass_out, int* __restrict__ stop_out,
    int* __restrict__ path_out) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int R = 2 * K + 1;
  const int nb_raw = draft_len[b];
  const float uf = u_final[b];
  int x = -1;
  float uk = 0.f;
  if (lane < K) {
    x = tokens[(size_t)b * K + lane];
    uk = u[(size_t)b * K + lane];
  }
  float Mt = -INFINITY, Md = -INFINITY, St = 0.f, Sd = 0.f;
  FiltRow ft, fd;
  if constexpr (FILT) {
    if (lane <= K) ft = frows[(size_t)b * R + lane];
    if (lane < K) fd = frows[(size_t)b * R + K + 1 + lane];
  } else {
    const float2* prow = part + (size_t)b * R * nchunk;
    if (lane <= K) combine_row(prow + (size_t)lane * nchunk, nchunk, c, Mt, St);
    if (lane < K) combine_row(prow + (size_t)(K + 1 + lane) * nchunk, nchunk, c, Md, Sd);
  }

  bool bad = nb_raw < 0 || nb_raw > K || !(uf >= 0.f && uf < 1.f);
  const int nb = bad ? 0 : nb_raw;
  bool ok = true, accept = false;
  double alpha = -1.0;
  if (!bad && lane <= nb) {                                  // target row usable
    if constexpr (FILT) ok = ft.status == 0;
    else ok = Mt != -INFINITY;
  }
  if (!bad && lane < nb) {
    if constexpr (FILT) ok = ok && fd.status == 0;
    else ok = ok && Md != -INFINITY;
    ok = ok && x >= 0 && x < V && uk >= 0.f && uk < 1.f;
    if (ok) {
      const float zt = to_f32(tgt[target_row_off(b, lane, K, V) + x]);
      const float zd = to_f32(dft[draft_row_off(b, lane, K, V) + x]);
      double pt, qd;
      if constexpr (FILT) {
        pt = filt_prob(zt, ft, invT);
        qd = filt_prob(zd, fd, invT);
      } else {
        pt = exp2((double)zt * c - (double)__fmul_rn(Mt, c)) / (double)St;
        qd = exp2((double)zd * c - (double)__fmul_rn(Md, c)) / (double)Sd;
      }
      ok = qd > 0.0;                                         // x was drawn from q: q(x) > 0
      const double ratio = pt / qd;
      alpha = ratio < 1.0 ? ratio : 1.0;
      accept = (double)uk < alpha;
    }
  }
  bad = bad || (__ballot(!ok) != 0);

  const int row = b * (K + 1);
  if (bad) {
    for (int k = lane; k <= K; k += kWave) out_tokens[row + k] = -1;
    if (alpha_out)
      for (int k = lane; k < K; k += kWave) alpha_out[(size_t)b * K + k] = -1.f;
    if (lane == 0) {
      n_emitted[b] = -1;
      plan[b].path = kPathError;
      if (rmass_out) rmass_out[b] = 0.0;
      if (stop_out) stop_out[b] = -1;
      if (path_out) path_out[b] = kPathError;
    }
    return;
  }

  const uint64_t rej = __ballot(lane < nb && !accept);
  int stop = rej ? __ffsll((unsigned long long)rej) - 1 : nb;
  int path = rej ? kPathReject : kPathBonus;
  const uint64_t eos = __ballot(lane < nb && accept && x == eos_id);
  if (eos) {
    const int e = __ffsll((unsigned long long)eos) - 1;
    if (e < stop) { stop = e; path = kPathEos; }
  }

  if (lane <= K)
    out_tokens[row + lane] = (lane < stop || (lane == stop && path == kPathEos)) ? x : -1;
  if (alpha_out && lane < K) alpha_out[(size_t)b * K + lane] = lane < nb ? (float)alpha : -1.f;
  if (lane == stop) {
    Plan pl;
    pl.path = path;
    pl.stop = stop;
    pl.trow = stop;
    pl.drow = path == kPathReject ? stop : -1;
    pl.mt = Mt;
    pl.md = Md;
    pl.pad0 = pl.pad1 = 0;
    // S_t / S_d in natural-exp units: each base-2 normaliser is relative to
    // 2^fl(M*c); undo that offset exactly (M*c is exact in float64).
    pl.g = 0.0;
    if (!FILT && path == kPathReject) {
      const double off_t = (double)__fmul_rn(Mt, c) - (double)Mt * (double)c;
      const double off_d = (double)__fmul_rn(Md, c) - (double)Md * (double)c;
      pl.g = ((double)St / (double)Sd) * exp2(off_t - off_d);
    }
    pl.pad2 = 0.0;
    plan[b] = pl;
    n_emitted[b] = stop + 1;
    if (rmass_out) rmass_out[b] = 0.0;
    if (stop_out) stop_out[b] = stop;
    if (path_out) path_out[b] = path;
  }
}

hipError_t launch_accept(bool bf16, bool filt, const void* tgt, const void* dft, const int* tokens,
                         const int* draft_len, const float* u, const float* u_final, int B,
                         int K, int V, int nchunk, float c, double invT, int eos_id,
                         const float2* part, const FiltRow* frows, Plan* plan, int* out_tokens,
                         int* n_emitted, float* alpha_out, double* rmass_out, int* stop_out,
                         int* path_out, hipStream_t stream) {
#define SPECV_ACCEPT(TT, FF)                                                                     \
  accept_kernel<TT, FF><<<dim3(B), dim3(kWave), 0, stream>>>(                                    \
      static_cast<const TT*>(tgt), static_cast<const TT*>(dft), tokens, draft_len, u, u_final, K, \
      V, nchunk, c, invT, eos_id, part, frows, plan, out_tokens, n_emitted, alpha_out, rmass_out, \
      stop_out, path_out)
  if (bf16) {
    if (filt) SPECV_ACCEPT(bf16_t, true); else SPECV_ACCEPT(bf16_t, false);
  } else {
    if (filt) SPECV_ACCEPT(float, true); else SPECV_ACCEPT(float, false);
  }
#undef SPECV_ACCEPT
  return hipGetLastError();
}

}  // namespace specv
