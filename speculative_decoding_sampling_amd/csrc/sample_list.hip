// The filtered path's draw: the residual after a rejection, or the bonus
// token after full acceptance, from the rows' kept sets (FiltRow and, when it
// fits, the kept list sorted by id).
//
// After a rejection at position j the token is drawn from
// max(p_j - q_j, 0) renormalised (nickwang.xyz "推测解码：草稿、验证与实际加速",
// section "接受与拒绝怎样保住分布", eq. r(x)); after full acceptance from p_n
// (section "候选已知，验证才能并行").  Both are inverse-CDF draws at u_final
// over token ids in ascending order with a strict comparison (section
// "算完三个 token 的全部概率", sample()), with p and q the filtered
// distributions.
#include <climits>

#include "common.h"
#include "exp64.h"
#include "filter_common.h"
#include "wave_scan.h"

namespace specv {

// ---------------------------------------------------------------------------
// The residual or bonus draw streamed over a whole filtered row pair, for a
// target row whose kept set has no list (more than kKeptCap tokens).  Chunks
// of 2048 tokens; in a chunk, lane l of a wave holds tokens c0 + 512 j + 8 l
// .. + 7 (j < 4), so the chunk's tokens in order are (j, lane, element).
// Weights in float64 from the rows' FiltRows: p = e_t / S_t on the target's
// kept tokens, and after a rejection max(p - q, 0) with q the same over the
// draft's kept tokens.  The chunk pass (one wave per chunk, the whole chip)
// writes each chunk's mass; the draw copies them to LDS, every wave finds the
// chunk holding t = u_final * total by a blocked prefix of its own, and the
// four waves scan inside that chunk, wave j its sub-block j.
constexpr int kStreamSub = kWave * 8;                  // 512 tokens per sub-block
constexpr int kStreamChunk = 4 * kStreamSub;           // 2048 tokens per chunk

template <typename T>
__device__ __forceinline__ void load8_checked(const T* __restrict__ row, long e0, int V, float* z) {
  constexpr int N = Elem<T>::kPerVec;
  const bool al = aligned16(row);
#pragma unroll
  for (int v = 0; v < 8 / N; ++v) load_vec_checked(row, e0 + v * N, V, al, z + v * N);
}

__device__ __forceinline__ double kept_prob(float z, const FiltRow& fr, double invT,
                                            const double* tbl) {
  if (!(z >= fr.tau) || z == -INFINITY) return 0.0;
  return exp64(((double)z - (double)fr.m) * invT, tbl) / fr.S;
}

// Element i (0..7) of eight registers, by a select tree (no indexed access).
__device__ __forceinline__ float pick8(const float* z, uint32_t i) {
  const float a = (i & 1u) ? z[1] : z[0], b = (i & 1u) ? z[3] : z[2];
  const float c = (i & 1u) ? z[5] : z[4], d = (i & 1u) ? z[7] : z[6];
  const float ab = (i & 2u) ? b : a, cd = (i & 2u) ? d : c;
  return (i & 4u) ? cd : ab;
}

// One chunk's masses, summed in a fixed order (per lane j then element, then
// the wave): .x the first attempt's (the residual after a rejection, else p),
// .y p alone (the fall-back when the residual has no mass).  A token outside
// the target's kept set adds exactly zero to both (p = 0, so p - q <= 0), so
// each lane visits only its kept tokens, in element order: the same sums,
// with far fewer exps when the kept set is a small share of the row.  (All
// four sub-blocks' loads issued before the first sum measured slower: 74
// against 58 VGPRs, and the chunk pass already overlaps loads across waves.)
template <typename T>
__device__ __forceinline__ double2 chunk_masses(const T* __restrict__ trow,
                                                const T* __restrict__ drow, int V, long c0,
                                                bool rej, const FiltRow& tr, const FiltRow& dr,
                                                double invT, const double* tbl) {
  const int lane = threadIdx.x % kWave;
  double acc_r = 0.0, acc_p = 0.0;
  for (int j = 0; j < 4; ++j) {
    const long e0 = c0 + j * kStreamSub + lane * 8;
    float zt[8], zd[8];
    load8_checked(trow, e0, V, zt);
    if (rej) load8_checked(drow, e0, V, zd);
    uint32_t km = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) km |= (zt[i] >= tr.tau && zt[i] != -INFINITY) ? 1u << i : 0u;
    while (km) {
      const uint32_t i = (uint32_t)__builtin_ctz(km);
      km &= km - 1u;
      const double p = kept_prob(pick8(zt, i), tr, invT, tbl);
      acc_p += p;
      if (rej) {
        const double x = p - kept_prob(pick8(zd, i), dr, invT, tbl);
        acc_r += x > 0.0 ? x : 0.0;
      }
    }
  }
  acc_p = wave_sum(acc_p);
  acc_r = rej ? wave_sum(acc_r) : acc_p;
  return make_double2(acc_r, acc_p);
}

// The chunk pass of the streamed draw: wave g of the grid takes chunk
// g % nch of request g / nch, when that request draws from a target row with
// no kept list.
template <typename T>
__global__ __launch_bounds__(kFiltThreads) void stream_chunks_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, int B, int K, int V, int nch,
    double invT, const Plan* __restrict__ plan, const FiltRow* __restrict__ rows,
    double2* __restrict__ cmass) {
  __shared__ double tbl[SPECV_EXP64_N];
  exp64_stage_table<kFiltThreads>(tbl);
  __syncthreads();
  const long g = (long)blockIdx.x * (kFiltThreads / kWave) + threadIdx.x / kWave;
  const int b = (int)(g / nch), c = (int)(g % nch);
  if (b >= B) return;
  const Plan pl = plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per wave
  const int R = 2 * K + 1;
  const FiltRow tr = rows[(size_t)b * R + pl.trow];
  if (tr.count <= kKeptCap) return;                  // the list draw serves it
  const bool rej = pl.path == kPathReject;
  FiltRow dr;
  dr.m = 0.f; dr.tau = 0.f; dr.S = 1.0; dr.count = 0; dr.status = 0; dr.pad = 0;
  if (rej) dr = rows[(size_t)b * R + K + 1 + pl.drow];
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  const T* drow = rej ? dft + draft_row_off(b, pl.drow, K, V) : trow;
  const double2 r = chunk_masses(trow, drow, V, (long)c * kStreamChunk, rej, tr, dr, invT, tbl);
  if (threadIdx.x % kWave == 0) cmass[(size_t)b * nch + c] = r;
}

template <typename T>
__device__ void stream_draw(const T* __restrict__ trow, const T* __restrict__ drow, int V,
                            bool rej, const FiltRow& tr, const FiltRow& dr, double invT,
                            const double* tbl, double uf, const double2* __restrict__ cm,
                            double* csum, double* dl, int* il, int& y_out, double& rmass_out) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nch = (V + kStreamChunk - 1) / kStreamChunk;
  auto weights = [&](long e0, bool resid, double* w) {
    float zt[8], zd[8];
    load8_checked(trow, e0, V, zt);
    if (resid) load8_checked(drow, e0, V, zd);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double x = kept_prob(zt[i], tr, invT, tbl);
      if (resid) {
        x -= kept_prob(zd[i], dr, invT, tbl);
        x = x > 0.0 ? x : 0.0;
      }
      w[i] = x;
    }
  };
  bool resid = rej;
  double total = 0.0, t = 0.0, pre = 0.0;
  int cstar = -1, clast = -1;
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (cm) {                                        // the chunk pass ran: copy its masses
      for (int c = threadIdx.x; c < nch; c += kFiltThreads) csum[c] = attempt == 0 ? cm[c].x : cm[c].y;
    } else {                                         // this block sums them, a wave per chunk
      for (int c = wid; c < nch; c += kFiltThreads / kWave) {
        const double2 r = chunk_masses(trow, drow ? drow : trow, V, (long)c * kStreamChunk, rej, tr,
                                       dr, invT, tbl);
        if (lane == 0) csum[c] = attempt == 0 ? r.x : r.y;
      }
    }
    __syncthreads();
    // every wave: blocked prefix over the chunk masses (lane l owns chunks
    // [l q, l q + q)), the same in every wave
    const int q = (nch + kWave - 1) / kWave;
    const int c_lo = min(nch, lane * q), c_hi = min(nch, c_lo + q);
    double mine = 0.0;
    for (int c = c_lo; c < c_hi; ++c) mine += csum[c];
    const double incl = wave_incl_scan(mine);
    total = lane_value(incl, kWave - 1);
    if (resid && !(total > 0.0)) {       // unreachable in exact arithmetic: draw from p_j
      resid = false;
      __syncthreads();                   // every wave has read csum
      continue;
    }
    t = uf * total;
    double run = wave_shr1(incl);
    int cand = -1, lastp = -1;
    double cpre = 0.0;
    for (int c = c_lo; c < c_hi; ++c) {
      const double before = run;
      run += csum[c];
      if (cand < 0 && t < run) {
        cand = c;
        cpre = before;
      }
      if (csum[c] > 0.0) lastp = c;
    }
    const uint64_t hit = __ballot(cand >= 0);
    if (hit) {
      const int L = __ffsll((unsigned long long)hit) - 1;
      cstar = lane_value(cand, L);
      pre = lane_value(cpre, L);
    } else {
      const uint64_t pos = __ballot(lastp >= 0);
      clast = pos ? lane_value(lastp, 63 - __clzll((long long)pos)) : -1;
    }
    break;
  }
  rmass_out = (rej && resid) ? total : 0.0;
  y_out = -1;
  const int cc = cstar >= 0 ? cstar : clast;         // uniform: every wave found the same
  if (cc < 0) return;                                // no positive mass at all
  // In-chunk scan by the four waves, wave w over sub-block w (lanes in
  // order): one round trip for the chunk's logits, the sub-block totals
  // combined in LDS in wave order.  After a rounding fall-through (no chunk
  // holds t) only the last positive token of the last chunk with mass counts.
  const long e0 = (long)cc * kStreamChunk + wid * kStreamSub + lane * 8;
  double w[8];
  weights(e0, resid, w);
  double mysum = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mysum += w[i];
  const double incl = wave_incl_scan(mysum);
  if (lane == kWave - 1) dl[wid] = incl;
  __syncthreads();
  double run = pre;
  for (int v = 0; v < wid; ++v) run += dl[v];
  run += wave_shr1(incl);
  int v = INT_MAX, vl = -1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    run += w[i];
    if (v == INT_MAX && t < run) v = (int)(e0 + i);
    if (w[i] > 0.0) vl = (int)(e0 + i);
  }
  // token order is wave order, then lane order: a wave's first hit is its
  // smallest, the first wave's hit the chunk's
  const uint64_t h1 = __ballot(v != INT_MAX), h2 = __ballot(vl >= 0);
  if (lane == 0) {
    il[wid] = h1 ? lane_value(v, __ffsll((unsigned long long)h1) - 1) : INT_MAX;
    il[kFiltThreads / kWave + wid] = h2 ? lane_value(vl, 63 - __clzll((long long)h2)) : -1;
  }
  __syncthreads();
  int y = INT_MAX, ylast = -1;
#pragma unroll
  for (int ww = 0; ww < kFiltThreads / kWave; ++ww) {
    y = min(y, il[ww]);
    ylast = max(ylast, il[kFiltThreads / kWave + ww]);
  }
  y_out = (cstar >= 0 && y != INT_MAX) ? y : ylast;  // rounding fall-through: last positive
}

// ---------------------------------------------------------------------------
// sample_list: per request, the residual or bonus draw over the target row's
// kept tokens in id order (streamed over the rows when the kept set has no
// list).
template <typename T>
__global__ __launch_bounds__(kFiltThreads) void sample_list_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const float* __restrict__ u_final,
    int K, int V, double invT, const Plan* __restrict__ plan, const FiltRow* __restrict__ rows,
    const Kept* __restrict__ kept, const double2* __restrict__ cmass, int* __restrict__ out_tokens,
    double* __restrict__ rmass_out) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double dl[kFiltThreads / kWave];
  __shared__ int il[2 * (kFiltThreads / kWave)];
  __shared__ double csum[kMaxSampChunks];
  const int b = blockIdx.x;
  exp64_stage_table<kFiltThreads>(tbl);
  const Plan pl = plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per block
  const int R = 2 * K + 1;
  const FiltRow tr = rows[(size_t)b * R + pl.trow];
  const bool rej = pl.path == kPathReject;
  FiltRow dr;
  dr.m = 0.f; dr.tau = 0.f; dr.S = 1.0; dr.count = 0; dr.status = 0; dr.pad = 0;
  if (rej) dr = rows[(size_t)b * R + K + 1 + pl.drow];
  const Kept* list = kept + ((size_t)b * R + pl.trow) * kKeptCap;
  const T* drow = rej ? dft + draft_row_off(b, pl.drow, K, V) : nullptr;
  __syncthreads();
  if (tr.count > kKeptCap) {                         // uniform: no list for this row
    int y;
    double rm;
    const int nch = (V + kStreamChunk - 1) / kStreamChunk;
    stream_draw(tgt + target_row_off(b, pl.trow, K, V), drow, V, rej, tr, dr, invT, tbl,
                (double)u_final[b], cmass ? cmass + (size_t)b * nch : nullptr, csum, dl, il, y,
                rm);
    if (threadIdx.x == 0) {
      out_tokens[(size_t)b * (K + 1) + pl.stop] = y;
      if (rmass_out) rmass_out[b] = rm;
    }
    return;
  }
  const int n = tr.count;
  const int q = (n + kFiltThreads - 1) / kFiltThreads;
  const int i_lo = min(n, (int)threadIdx.x * q), i_hi = min(n, i_lo + q);
  constexpr int kMaxPer = (kKeptCap + kFiltThreads - 1) / kFiltThreads;
  double w[kMaxPer];
  int ids[kMaxPer];
  double wp[kMaxPer];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    w[j] = wp[j] = 0.0;
    ids[j] = -1;
    const int i = i_lo + j;
    if (i < i_hi) {
      const Kept e = list[i];
      ids[j] = e.id;
      wp[j] = exp64(((double)e.z - (double)tr.m) * invT, tbl);
      w[j] = wp[j];
      if (rej) {
        const float zd = to_f32(drow[e.id]);
        double qv = 0.0;
        if (zd >= dr.tau && zd > -INFINITY) qv = exp64(((double)zd - (double)dr.m) * invT, tbl) / dr.S;
        const double r = wp[j] / tr.S - qv;
        w[j] = r > 0.0 ? r : 0.0;
      }
    }
  }
  double mine = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) mine += w[j];
  double total;
  double excl = block_scan_excl<double>(mine, dl, total);
  bool resid = rej;
  if (resid && !(total > 0.0)) {                     // unreachable in exact arithmetic: draw from p_j
    resid = false;
    mine = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      w[j] = wp[j];
      mine += w[j];
    }
    excl = block_scan_excl<double>(mine, dl, total);
  }
  const double t = (double)u_final[b] * total;
  int hit = INT_MAX, last = -1;
  double run = excl;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    if (ids[j] < 0) continue;
    run += w[j];
    if (hit == INT_MAX && t < run) hit = ids[j];
    if (w[j] > 0.0) last = ids[j];
  }
  int y = block_min_i(hit, il);
  if (y == INT_MAX) y = -block_min_i(-last, il);     // rounding fall-through: last positive
  if (threadIdx.x == 0) {
    out_tokens[(size_t)b * (K + 1) + pl.stop] = y;
    if (rmass_out) rmass_out[b] = (rej && resid) ? total : 0.0;
  }
}

int stream_chunks(int V) { return (V + kStreamChunk - 1) / kStreamChunk; }

// cmass: the chunk pass's output, or null to skip that pass (where kept sets
// above kKeptCap are rare: the draw then sums the chunk masses itself).
hipError_t launch_sample_list(bool bf16, const void* tgt, const void* dft, const float* u_final,
                              int B, int K, int V, double invT, const Plan* plan,
                              const FiltRow* rows, const Kept* kept, double2* cmass,
                              int* out_tokens, double* rmass_out, hipStream_t stream) {
  const int nch = stream_chunks(V);
  if (nch > kMaxSampChunks) return hipErrorInvalidConfiguration;
  constexpr int kWavesPer = kFiltThreads / kWave;
  const size_t blocks = ((size_t)B * nch + kWavesPer - 1) / kWavesPer;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (bf16) {
    if (cmass)
      stream_chunks_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kFiltThreads), 0, stream>>>(
          static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), B, K, V, nch, invT,
          plan, rows, cmass);
    sample_list_kernel<bf16_t><<<dim3(B), dim3(kFiltThreads), 0, stream>>>(
        static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), u_final, K, V, invT,
        plan, rows, kept, cmass, out_tokens, rmass_out);
  } else {
    if (cmass)
      stream_chunks_kernel<float><<<dim3((unsigned)blocks), dim3(kFiltThreads), 0, stream>>>(
          static_cast<const float*>(tgt), static_cast<const float*>(dft), B, K, V, nch, invT,
          plan, rows, cmass);
    sample_list_kernel<float><<<dim3(B), dim3(kFiltThreads), 0, stream>>>(
        static_cast<const float*>(tgt), static_cast<const float*>(dft), u_final, K, V, invT, plan,
        rows, kept, cmass, out_tokens, rmass_out);
  }
  return hipGetLastError();
}

}  // namespace specv
