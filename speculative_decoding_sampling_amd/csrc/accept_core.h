// Accept scan of one request, run by one wave64: lane k owns draft position k.
//
// Lane k has the statistics of target row k and draft row k and the two
// logits at the drafted token x_k.  It forms p_k(x_k) and q_k(x_k) in
// float64, alpha_k = min(1, p/q), and tests u[b][k] < alpha_k
// (nickwang.xyz "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布",
// eq. a(x); the strict comparison of that page's replay code).  A ballot
// finds the first rejection: every earlier draft is emitted and every later
// one discarded (section "候选已知，验证才能并行"; tbxsx.cn
// "推测解码采样验证优化策略 —— 深度调研报告", section "4. 实现逻辑").  A second
// ballot finds the first accepted EOS, which ends the round early.  The lane
// at the stop position forms the request's plan: a correction from
// max(p_j - q_j, 0) after a rejection, or a bonus from target row draft_len
// when all drafts pass.
#pragma once

#include "common.h"

namespace specv {

constexpr int kCombineBatch = 16;

// Combine the chunk partials of this lane's target row (if has_t) and draft
// row (if has_d), each in chunk order.  A chunk partial s with maximum m is
// relative to 2^fl(m*c); a combined S is relative to 2^fl(M*c) with M the row
// maximum.  The partials are float32 sums, so float32 scale factors add no
// meaningful error.  Both rows' loads of a batch are issued together.
__device__ __forceinline__ void combine_batch(const float2* v, float c, float& m, float& s) {
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
__device__ __forceinline__ void combine_rows(const float2* __restrict__ pt,
                                             const float2* __restrict__ pd, int n, float c,
                                             bool has_t, bool has_d, float& Mt, float& St,
                                             float& Md, float& Sd) {
  float mt = -INFINITY, st = 0.f, md = -INFINITY, sd = 0.f;
  for (int base = 0; base < n; base += kCombineBatch) {
    float2 vt[kCombineBatch], vd[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const bool in = base + j < n;
      vt[j] = has_t && in ? pt[base + j] : make_float2(-INFINITY, 0.f);
      vd[j] = has_d && in ? pd[base + j] : make_float2(-INFINITY, 0.f);
    }
    combine_batch(vt, c, mt, st);
    combine_batch(vd, c, md, sd);
  }
  Mt = mt;
  St = st;
  Md = md;
  Sd = sd;
}

// S_t / S_d in natural-exp units from the two rows' combined float32
// statistics: each base-2 normaliser is relative to 2^fl(M*c); undo that
// offset exactly (M*c is exact in float64).
__device__ __forceinline__ double normaliser_ratio(float Mt, float St, float Md, float Sd,
                                                   float c) {
  const double off_t = (double)__fmul_rn(Mt, c) - (double)Mt * (double)c;
  const double off_d = (double)__fmul_rn(Md, c) - (double)Md * (double)c;
  return ((double)St / (double)Sd) * exp2(off_t - off_d);
}

// Probability of token x in a filtered row: exp((z - m)/T) / S if z is kept.
__device__ __forceinline__ double filt_prob(float z, const FiltRow& fr, double invT) {
  if (!(z >= fr.tau) || z == -INFINITY) return 0.0;
  return exp(((double)z - (double)fr.m) * invT) / fr.S;
}

// Statistics of lane k's rows: target row k (lane <= K) and draft row k
// (lane < K).  Unfiltered rows carry the combined float32 (max, normaliser),
// filtered rows their FiltRow.  With K = 64 target row 64 (the bonus row of
// a request that drafted 64 tokens) has no lane of its own: every lane then
// also holds its statistics in Mk, Sk / fk.
struct LaneRows {
  float Mt = -INFINITY, St = 0.f, Md = -INFINITY, Sd = 0.f;
  FiltRow ft, fd;
  float Mk = -INFINITY, Sk = 0.f;
  FiltRow fk;
};

// Outputs of the scan; pointers may be null where the caller wants none.
struct AcceptOut {
  Plan* plan;          // [B] the plan, for the sampler kernels
  int* out_tokens;     // [B][K+1]
  int* n_emitted;      // [B], or null (sampling calls)
  float* alpha_out;    // [B][K] or null
  double* rmass_out;   // [B] or null (written 0 here; the sampler sets it)
  int* stop_out;       // [B] or null
  int* path_out;       // [B] or null
};

// The scan for request b.  nb_raw = draft_len[b], uf = u_final[b] (both
// wave-uniform); per lane: x and uk (lane < K), xin = (lane < K and x in
// [0, V)), zt / zd the logits at x (read only where lane < draft_len and
// xin).  Writes the request's outputs and its plan.
template <bool FILT>
__device__ __forceinline__ void accept_scan(int b, int lane, int K, float c, double invT,
                                            int eos_id, int nb_raw, float uf, int x, float uk,
                                            bool xin, float zt, float zd, const LaneRows& rs,
                                            const AcceptOut& out) {
  bool bad = nb_raw < 0 || nb_raw > K || !(uf >= 0.f && uf < 1.f);
  const int nb = bad ? 0 : nb_raw;
  bool ok = true, accept = false;
  double alpha = -1.0;
  if (!bad && lane <= nb) {                                  // target row usable
    if constexpr (FILT) ok = rs.ft.status == 0;
    else ok = rs.Mt != -INFINITY;
  }
  if (!bad && nb == kWave) {                                 // the bonus row past the lanes
    if constexpr (FILT) bad = rs.fk.status != 0;
    else bad = rs.Mk == -INFINITY;
  }
  if (!bad && lane < nb) {
    if constexpr (FILT) ok = ok && rs.fd.status == 0;
    else ok = ok && rs.Md != -INFINITY;
    ok = ok && xin && uk >= 0.f && uk < 1.f;
    if (ok) {
      double pt, qd;
      if constexpr (FILT) {
        pt = filt_prob(zt, rs.ft, invT);
        qd = filt_prob(zd, rs.fd, invT);
      } else {
        pt = exp2((double)zt * c - (double)__fmul_rn(rs.Mt, c)) / (double)rs.St;
        qd = exp2((double)zd * c - (double)__fmul_rn(rs.Md, c)) / (double)rs.Sd;
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
    for (int k = lane; k <= K; k += kWave) out.out_tokens[row + k] = -1;
    if (out.alpha_out)
      for (int k = lane; k < K; k += kWave) out.alpha_out[(size_t)b * K + k] = -1.f;
    if (lane == 0) {
      Plan pl = {};
      pl.path = kPathError;
      pl.stop = -1;
      out.plan[b] = pl;
      if (out.n_emitted) out.n_emitted[b] = -1;
      if (out.rmass_out) out.rmass_out[b] = 0.0;
      if (out.stop_out) out.stop_out[b] = -1;
      if (out.path_out) out.path_out[b] = kPathError;
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
    out.out_tokens[row + lane] = (lane < stop || (lane == stop && path == kPathEos)) ? x : -1;
  if (K == kWave && lane == 0) out.out_tokens[row + K] = -1;   // the draw fills it if stop = 64
  if (out.alpha_out && lane < K)
    out.alpha_out[(size_t)b * K + lane] = lane < nb ? (float)alpha : -1.f;
  // the lane at the stop position writes the plan; a stop at 64 (every one
  // of 64 drafts accepted) is written by lane 0 from the bonus row's Mk
  if (lane == (stop < kWave ? stop : 0)) {
    Plan pl;
    pl.path = path;
    pl.stop = stop;
    pl.trow = stop;
    pl.drow = path == kPathReject ? stop : -1;
    pl.mt = FILT ? 0.f : (stop < kWave ? rs.Mt : rs.Mk);
    pl.md = FILT ? 0.f : rs.Md;
    pl.pad0 = pl.pad1 = 0;
    // S_t / S_d in natural-exp units, for the sampler's classification
    pl.g = (!FILT && path == kPathReject) ? normaliser_ratio(rs.Mt, rs.St, rs.Md, rs.Sd, c) : 0.0;
    pl.pad2 = 0.0;
    out.plan[b] = pl;
    if (out.n_emitted) out.n_emitted[b] = stop + 1;
    if (out.rmass_out) out.rmass_out[b] = 0.0;
    if (out.stop_out) out.stop_out[b] = stop;
    if (out.path_out) out.path_out[b] = path;
  }
}

// The scan of request b by one wave (lane 0..63), with its inputs gathered:
// the drafted tokens and uniforms, the logits at the drafted tokens and the
// statistics of all K+1 target and K draft rows, every load that does not
// depend on another issued up front (rows beyond draft_len are loaded but
// never used).  Without filters the row statistics are the chunk partials
// of the row-statistics pass and the logits at the drafted tokens the ones
// it recorded; with top-k / top-p they are the per-row FiltRow and two
// gathers from the logits.
template <typename T, bool FILT>
__device__ __forceinline__ void accept_request(
    int b, int lane, const T* __restrict__ tgt, const T* __restrict__ dft,
    const int* __restrict__ tokens, const int* __restrict__ draft_len, const float* __restrict__ u,
    const float* __restrict__ u_final, int K, int V, int nch_row, float c, double invT,
    int eos_id, const float2* __restrict__ part, const float* __restrict__ zx,
    const FiltRow* __restrict__ frows, const AcceptOut& out) {
  const int R = 2 * K + 1;
  const int nb_raw = draft_len ? draft_len[b] : 0;   // null: no drafts (sampling)
  const float uf = u_final[b];
  int x = -1;
  float uk = 0.f, zt = -INFINITY, zd = -INFINITY;
  if (lane < K) {
    x = tokens[(size_t)b * K + lane];
    uk = u[(size_t)b * K + lane];
    if constexpr (!FILT) {
      zt = zx[(size_t)b * 2 * K + lane];            // meaningful where the scan reads it
      zd = zx[(size_t)b * 2 * K + K + lane];
    }
  }
  const bool xin = lane < K && x >= 0 && x < V;
  LaneRows rs;
  if constexpr (FILT) {
    if (xin) {
      zt = to_f32(tgt[target_row_off(b, lane, K, V) + x]);
      zd = to_f32(dft[draft_row_off(b, lane, K, V) + x]);
    }
    if (lane <= K) rs.ft = frows[(size_t)b * R + lane];
    if (lane < K) rs.fd = frows[(size_t)b * R + K + 1 + lane];
    if (K == kWave) rs.fk = frows[(size_t)b * R + K];       // uniform: the bonus row of 64 drafts
  } else {
    const float2* prow = part + (size_t)b * R * nch_row;
    combine_rows(prow + (size_t)lane * nch_row, prow + (size_t)(K + 1 + lane) * nch_row, nch_row,
                 c, lane <= K, lane < K, rs.Mt, rs.St, rs.Md, rs.Sd);
    if (K == kWave) {                                        // uniform: the bonus row of 64 drafts
      float md, sd;
      combine_rows(prow + (size_t)K * nch_row, prow, nch_row, c, true, false, rs.Mk, rs.Sk, md, sd);
    }
  }
  accept_scan<FILT>(b, lane, K, c, invT, eos_id, nb_raw, uf, x, uk, xin, zt, zd, rs, out);
}

}  // namespace specv
