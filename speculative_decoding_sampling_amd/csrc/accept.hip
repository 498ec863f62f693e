// Gather-and-accept scan: one wave64 per request, lane k owns draft position k.
//
// Lane k combines the chunk partials of target row k and draft row k into
// exact row maxima and float64 normalisers, gathers p_k(x_k) and q_k(x_k),
// forms alpha_k = min(1, p/q) and tests u[b][k] < alpha_k (nickwang.xyz
// "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布", eq. a(x); the
// strict comparison of that page's replay code).  A ballot finds the first
// rejection: every earlier draft is emitted and every later one discarded
// (section "候选已知，验证才能并行"; tbxsx.cn "推测解码采样验证优化策略 ——
// 深度调研报告", section "4. 实现逻辑").  A second ballot finds the first
// accepted EOS, which ends the round early.  The lane at the stop position
// records what the sampler must draw: a correction from max(p_j - q_j, 0)
// after a rejection, or a bonus from target row draft_len when all drafts
// pass.
#include "common.h"

namespace specv {

// Combine one row's chunk partials in chunk order.  The partial s of a chunk
// with maximum m is relative to 2^fl(m*c); the row normaliser is returned
// relative to 2^fl(M*c) with M the row maximum, in float64.
__device__ __forceinline__ void combine_row(const float2* __restrict__ p, int n, float c,
                                            float& M, double& S) {
  float m = -INFINITY;
  for (int i = 0; i < n; ++i) m = fmaxf(m, p[i].x);
  double s = 0.0;
  if (m != -INFINITY) {
    const double Mc = (double)__fmul_rn(m, c);
    for (int i = 0; i < n; ++i)
      if (p[i].x != -INFINITY) s += (double)p[i].y * exp2((double)__fmul_rn(p[i].x, c) - Mc);
  }
  M = m;
  S = s;
}

template <typename T>
__global__ __launch_bounds__(kWave) void accept_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ tokens,
    const int* __restrict__ draft_len, const float* __restrict__ u,
    const float* __restrict__ u_final, int K, int V, int nchunk, float c, int eos_id,
    const float2* __restrict__ part, Plan* __restrict__ plan, int* __restrict__ out_tokens,
    int* __restrict__ n_emitted, float* __restrict__ alpha_out, double* __restrict__ rmass_out,
    int* __restrict__ stop_out, int* __restrict__ path_out) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int R = 2 * K + 1;
  const int nb_raw = draft_len[b];
  const float uf = u_final[b];
  bool bad = nb_raw < 0 || nb_raw > K || !(uf >= 0.f && uf < 1.f);
  const int nb = bad ? 0 : nb_raw;

  float Mt = -INFINITY, Md = -INFINITY;
  double St = 0.0, Sd = 0.0;
  const float2* prow = part + (size_t)b * R * nchunk;
  if (!bad && lane <= nb) combine_row(prow + (size_t)lane * nchunk, nchunk, c, Mt, St);
  if (!bad && lane < nb) combine_row(prow + (size_t)(K + 1 + lane) * nchunk, nchunk, c, Md, Sd);

  bool ok = true, accept = false;
  double alpha = -1.0;
  int x = -1;
  if (!bad && lane <= nb) ok = Mt != -INFINITY;            // target row has a finite logit
  if (!bad && lane < nb) {
    x = tokens[(size_t)b * K + lane];
    const float uk = u[(size_t)b * K + lane];
    ok = ok && Md != -INFINITY && x >= 0 && x < V && uk >= 0.f && uk < 1.f;
    if (ok) {
      const float zt = to_f32(tgt[target_row_off(b, lane, K, V) + x]);
      const float zd = to_f32(dft[draft_row_off(b, lane, K, V) + x]);
      const double pt = exp2((double)zt * c - (double)__fmul_rn(Mt, c)) / St;
      const double qd = exp2((double)zd * c - (double)__fmul_rn(Md, c)) / Sd;
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
    plan[b] = pl;
    n_emitted[b] = stop + 1;
    if (rmass_out) rmass_out[b] = 0.0;
    if (stop_out) stop_out[b] = stop;
    if (path_out) path_out[b] = path;
  }
}

hipError_t launch_accept(bool bf16, const void* tgt, const void* dft, const int* tokens,
                         const int* draft_len, const float* u, const float* u_final, int B,
                         int K, int V, int nchunk, float c, int eos_id, const float2* part,
                         Plan* plan, int* out_tokens, int* n_emitted, float* alpha_out,
                         double* rmass_out, int* stop_out, int* path_out, hipStream_t stream) {
  if (bf16)
    accept_kernel<bf16_t><<<dim3(B), dim3(kWave), 0, stream>>>(
        static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), tokens, draft_len, u,
        u_final, K, V, nchunk, c, eos_id, part, plan, out_tokens, n_emitted, alpha_out,
        rmass_out, stop_out, path_out);
  else
    accept_kernel<float><<<dim3(B), dim3(kWave), 0, stream>>>(
        static_cast<const float*>(tgt), static_cast<const float*>(dft), tokens, draft_len, u,
        u_final, K, V, nchunk, c, eos_id, part, plan, out_tokens, n_emitted, alpha_out,
        rmass_out, stop_out, path_out);
  return hipGetLastError();
}

}  // namespace specv
