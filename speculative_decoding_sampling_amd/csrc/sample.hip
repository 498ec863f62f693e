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
// sums -- is float64, recomputed from the logits; the float32 row statistics
// supply only the exact row maxima and an estimate g of S_t / S_d.
//
// One pass over the logits.  p_v > q_v  <=>  e_t(v) > e_d(v) * S_t / S_d.
// Each chunk workgroup of the pass kernel classifies its tokens against the
// estimate g: "certainly p > q" if e_t > e_d g (1 + w), "certainly not" if
// e_t < e_d g (1 - w), a near tie otherwise (w = 2^-14, well above g's
// float32 error).  It records the sums of e_t and e_d over the chunk and over
// the certain set, and the near ties themselves (in token order).  The finish
// kernel (one workgroup per request) forms the exact normalisers, checks
// |g / (S_t/S_d) - 1| <= w/4 so the certain set is certain, and builds each
// chunk's residual mass as A_t/S_t - A_d/S_d plus its near ties resolved
// exactly.  A chunk with more near ties than slots has its mass recomputed
// exactly from the logits; if the check fails, every chunk is (slow, rare).
// It then finds the chunk holding t = u_final * total with a blocked prefix
// and scans inside it.  All sums run in a fixed order, so the draw is
// deterministic.  The two kernels communicate only through the kernel
// boundary: on gfx950 a device-scope release inside a kernel writes back the
// XCD's L2, far too costly to do once per workgroup.
#include <climits>

#include "common.h"
#include "exp64.h"

namespace specv {

// This thread's 8 logits of the chunk starting at element c0 (thread t holds
// elements c0 + 8t .. c0 + 8t + 7).  The interior test is uniform per chunk.
template <typename T>
__device__ __forceinline__ void load8(const T* __restrict__ row, long c0, int V, float* out) {
  constexpr int N = Elem<T>::kPerVec;
  const long e0 = c0 + (long)threadIdx.x * kSampPerThread;
  const bool aligned = aligned16(row);
  if (aligned && c0 + kSampChunk <= V) {
#pragma unroll
    for (int j = 0; j < kSampPerThread / N; ++j) load_vec_fast(row, e0 + j * N, out + j * N);
  } else {
#pragma unroll
    for (int j = 0; j < kSampPerThread / N; ++j)
      load_vec_checked(row, e0 + j * N, V, aligned, out + j * N);
  }
}

constexpr int kSampWaves = kSampThreads / kWave;
constexpr int kPassChunks = 1;   // chunks per pass workgroup

// Sum of one double per thread over the block, in a fixed order (every
// thread gets the result).
__device__ __forceinline__ double block_sum(double v, double* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kSampWaves; ++w) s += lds[w];
  return s;
}

// Exclusive prefix of one value per thread over the block (thread order) and
// the block total.
template <typename V>
__device__ __forceinline__ V block_exclusive_scan(V v, V* lds, V& total) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  V x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const V y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  V excl = __shfl_up(x, 1, kWave);
  if (lane == 0) excl = V(0);
  __syncthreads();
  if (lane == kWave - 1) lds[wid] = x;
  __syncthreads();
  V off = V(0);
  total = V(0);
#pragma unroll
  for (int w = 0; w < kSampWaves; ++w) {
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
  for (int w = 1; w < kSampWaves; ++w) r = min(r, lds[w]);
  return r;
}

__device__ __forceinline__ int block_max(int v, int* lds) { return -block_min(-v, lds); }

// e = exp((z - m) / T), the unnormalised float64 weight of one logit.
__device__ __forceinline__ double weight_e(float z, double m, double invT, const double* tbl) {
  return exp64(((double)z - m) * invT, tbl);
}

// Residual weights max(e_t/S_t - e_d/S_d, 0) (resid) or target weights e_t of
// one thread's 8 tokens.
template <typename T>
__device__ __forceinline__ void chunk_weights(const T* trow, const T* drow, long c0, int V,
                                              bool resid, double mt, double md, double invT,
                                              double St, double Sd, const double* tbl,
                                              double* w) {
  float zt[kSampPerThread];
  load8(trow, c0, V, zt);
  if (resid) {
    float zd[kSampPerThread];
    load8(drow, c0, V, zd);
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) {
      const double r = weight_e(zt[i], mt, invT, tbl) / St - weight_e(zd[i], md, invT, tbl) / Sd;
      w[i] = r > 0.0 ? r : 0.0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) w[i] = weight_e(zt[i], mt, invT, tbl);
  }
}

// Sums and near ties of one 2048-token chunk whose logits this thread holds
// (8 per thread, token order = thread order), written to the chunk's record.
__device__ __forceinline__ void pass_chunk(const float* zt, const float* zd, bool rej, long e0,
                                           double mt, double md, double invT, double g,
                                           const double* tbl, double* dl, int* il,
                                           ChunkRec* __restrict__ rec, Tie* __restrict__ slot) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  double et[kSampPerThread], ed[kSampPerThread];
  double st = 0.0, sd = 0.0, at = 0.0, ad = 0.0;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) {
    et[i] = weight_e(zt[i], mt, invT, tbl);
    st += et[i];
  }
  unsigned tiemask = 0;
  if (rej) {
    const double ghi = g * (1.0 + kTieWindow), glo = g * (1.0 - kTieWindow);
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) {
      ed[i] = weight_e(zd[i], md, invT, tbl);
      sd += ed[i];
      if (et[i] > ed[i] * ghi) {
        at += et[i];
        ad += ed[i];
      } else if (et[i] > 0.0 && et[i] >= ed[i] * glo) {
        tiemask |= 1u << i;
      }
    }
  }
  st = wave_sum(st);
  sd = wave_sum(sd);
  at = wave_sum(at);
  ad = wave_sum(ad);
  __syncthreads();                                   // dl / il free from any earlier use
  if (lane == 0) {
    dl[wid * 4 + 0] = st;
    dl[wid * 4 + 1] = sd;
    dl[wid * 4 + 2] = at;
    dl[wid * 4 + 3] = ad;
  }
  int ntie_all = 0;
  if (rej) {
    // near ties go to the chunk's slots in token order (block prefix of counts)
    int off = block_exclusive_scan<int>(__popc(tiemask), il, ntie_all);
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) {
      if ((tiemask >> i) & 1u) {
        if (off < kTieCap) {
          Tie tv;
          tv.et = et[i];
          tv.ed = ed[i];
          tv.v = (int)(e0 + i);
          tv.pad = 0;
          slot[off] = tv;
        }
        ++off;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ChunkRec r;
    r.et = r.ed = r.at = r.ad = 0.0;
#pragma unroll
    for (int w = 0; w < kSampWaves; ++w) {
      r.et += dl[w * 4 + 0];
      r.ed += dl[w * 4 + 1];
      r.at += dl[w * 4 + 2];
      r.ad += dl[w * 4 + 3];
    }
    r.ntie = ntie_all;
#pragma unroll
    for (int i = 0; i < 7; ++i) r.pad[i] = 0;
    *rec = r;
  }
}

// (a) chunk pass: float64 sums and near ties, kPassChunks chunks per
// workgroup with every logit load issued before the first exp.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_pass_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, int K, int V, int nch, int ngrp,
    double invT, const Plan* __restrict__ plan, ChunkRec* __restrict__ recs,
    Tie* __restrict__ ties) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double dl[kSampWaves * 4];
  __shared__ int il[kSampWaves];

  const int grp = blockIdx.x % ngrp, b = blockIdx.x / ngrp;
  exp64_stage_table(tbl);                            // independent of the plan: overlaps it
  const Plan pl = plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per block
  const bool rej = pl.path == kPathReject;
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  const T* drow = rej ? dft + draft_row_off(b, pl.drow, K, V) : nullptr;
  const int c0 = grp * kPassChunks;
  const int nc = min(kPassChunks, nch - c0);
  float zt[kPassChunks][kSampPerThread], zd[kPassChunks][kSampPerThread];
#pragma unroll
  for (int s = 0; s < kPassChunks; ++s) {
    if (s < nc) {
      const long cs = (long)(c0 + s) * kSampChunk;
      load8(trow, cs, V, zt[s]);
      if (rej) load8(drow, cs, V, zd[s]);
    }
  }
  __syncthreads();                                   // table staged
#pragma unroll
  for (int s = 0; s < kPassChunks; ++s) {
    if (s < nc) {
      const int c = c0 + s;
      const long e0 = (long)c * kSampChunk + (long)threadIdx.x * kSampPerThread;
      pass_chunk(zt[s], zd[s], rej, e0, (double)pl.mt, (double)pl.md, invT, pl.g, tbl, dl, il,
                 recs + (size_t)b * nch + c, ties + ((size_t)b * nch + c) * kTieCap);
    }
  }
}

// (b) the draw: one workgroup per request, after every chunk record exists.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_finish_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const float* __restrict__ u_final,
    int K, int V, int nch, double invT, const Plan* __restrict__ plan,
    const ChunkRec* __restrict__ recs, const Tie* __restrict__ ties, int* __restrict__ out_tokens,
    double* __restrict__ rmass_out) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double dl[kSampWaves * 4];
  __shared__ int il[kSampWaves];
  __shared__ double wts[kMaxSampChunks];
  __shared__ int s_fb;
  __shared__ double s_St, s_Sd, s_cpre;

  const int b = blockIdx.x;
  exp64_stage_table(tbl);                            // independent of the plan: overlaps it
  const Plan pl = plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per block
  const bool rej = pl.path == kPathReject;
  __syncthreads();
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  const T* drow = rej ? dft + draft_row_off(b, pl.drow, K, V) : nullptr;
  const double mt = pl.mt, md = pl.md;
  const int lane = threadIdx.x % kWave;

  // ---------------- finish (one workgroup per request) ----------------
  const ChunkRec* rb = recs + (size_t)b * nch;
  if (threadIdx.x < kWave) {
    double a = 0.0, d = 0.0;
    int ovf = 0;
    for (int i = lane; i < nch; i += kWave) {
      a += rb[i].et;
      d += rb[i].ed;
      ovf |= rb[i].ntie > kTieCap;
    }
    a = wave_sum(a);
    d = wave_sum(d);
    const bool any_ovf = __ballot(ovf) != 0;
    if (lane == 0) {
      s_St = a;
      s_Sd = d;
      s_fb = any_ovf;
    }
  }
  __syncthreads();
  const double St = s_St, Sd = s_Sd;
  bool fb = s_fb != 0;
  if (rej && !fb) fb = !(fabs(pl.g * Sd / St - 1.0) <= 0.25 * kTieWindow);

  // chunk masses: A_t/S_t - A_d/S_d plus the chunk's near ties resolved exactly;
  // a chunk with more ties than slots (or every chunk, if the estimate check
  // failed) gets its mass recomputed exactly from the logits.
  __shared__ int s_nredo;
  __shared__ int redo[kMaxSampChunks];
  if (threadIdx.x == 0) s_nredo = 0;
  __syncthreads();
  if (rej) {
    for (int cc = threadIdx.x; cc < nch; cc += kSampThreads) {
      const ChunkRec r = rb[cc];
      if (fb || r.ntie > kTieCap) {
        redo[atomicAdd(&s_nredo, 1)] = cc;
        continue;
      }
      double w = r.at / St - r.ad / Sd;
      const Tie* ts = ties + ((size_t)b * nch + cc) * kTieCap;
      for (int i = 0; i < r.ntie; ++i) {
        const double x = ts[i].et / St - ts[i].ed / Sd;
        if (x > 0.0) w += x;
      }
      wts[cc] = w > 0.0 ? w : 0.0;
    }
  } else {
    for (int cc = threadIdx.x; cc < nch; cc += kSampThreads) wts[cc] = rb[cc].et;
  }
  __syncthreads();
  const int nredo = s_nredo;
  for (int i = 0; i < nredo; ++i) {                  // each chunk's mass is order-independent
    const int cc = redo[i];
    double w[kSampPerThread];
    chunk_weights(trow, drow, (long)cc * kSampChunk, V, true, mt, md, invT, St, Sd, tbl, w);
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < kSampPerThread; ++k) sum += w[k];
    sum = block_sum(sum, dl);
    if (threadIdx.x == 0) wts[cc] = sum;
  }
  __syncthreads();

  // blocked prefix over chunk masses: thread t owns chunks [c_lo, c_hi)
  const int q = (nch + kSampThreads - 1) / kSampThreads;
  const int c_lo = min(nch, (int)threadIdx.x * q), c_hi = min(nch, c_lo + q);
  bool resid = rej;
  double mine = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) mine += wts[cc];
  double total;
  double excl = block_exclusive_scan<double>(mine, dl, total);
  if (resid && !(total > 0.0)) {
    // residual rounded to zero everywhere (unreachable in exact arithmetic): draw from p_j
    resid = false;
    __syncthreads();
    for (int cc = threadIdx.x; cc < nch; cc += kSampThreads) wts[cc] = rb[cc].et;
    __syncthreads();
    mine = 0.0;
    for (int cc = c_lo; cc < c_hi; ++cc) mine += wts[cc];
    excl = block_exclusive_scan<double>(mine, dl, total);
  }
  const double rmass = (rej && resid) ? total : 0.0;
  const double t = (double)u_final[b] * total;
  int cand = INT_MAX, last_pos = -1;
  double run = excl;
  for (int cc = c_lo; cc < c_hi; ++cc) {
    run += wts[cc];
    if (cand == INT_MAX && t < run) cand = cc;
    if (wts[cc] > 0.0) last_pos = cc;
  }
  int cstar = block_min(cand, il);
  double tprime;
  if (cstar == INT_MAX) {            // rounding fall-through: last chunk with mass
    cstar = block_max(last_pos, il);
    tprime = INFINITY;
    if (cstar < 0) {                 // no positive mass at all (non-finite input)
      if (threadIdx.x == 0) {
        out_tokens[(size_t)b * (K + 1) + pl.stop] = -1;
        if (rmass_out) rmass_out[b] = rmass;
      }
      return;
    }
  } else {
    __syncthreads();
    if (cand == cstar) {             // the one thread owning chunk cstar
      double pre = excl;
      for (int cc = c_lo; cc < cstar; ++cc) pre += wts[cc];
      s_cpre = pre;
    }
    __syncthreads();
    tprime = t - s_cpre;
  }

  // in-chunk scan of chunk cstar
  const long e0 = (long)cstar * kSampChunk + (long)threadIdx.x * kSampPerThread;
  double w[kSampPerThread];
  chunk_weights(trow, drow, (long)cstar * kSampChunk, V, resid, mt, md, invT, St, Sd, tbl, w);
  double mysum = 0.0;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) mysum += w[i];
  double ctot;
  const double ex = block_exclusive_scan<double>(mysum, dl, ctot);
  int vc = INT_MAX, vlast = -1;
  run = ex;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) {
    run += w[i];
    if (vc == INT_MAX && tprime < run) vc = (int)(e0 + i);
    if (w[i] > 0.0) vlast = (int)(e0 + i);
  }
  int y = block_min(vc, il);
  if (y == INT_MAX) y = block_max(vlast, il);   // rounding fall-through inside the chunk
  if (threadIdx.x == 0) {
    out_tokens[(size_t)b * (K + 1) + pl.stop] = y;
    if (rmass_out) rmass_out[b] = rmass;
  }
}

template <typename T>
static hipError_t sample_pass_t(const void* tgt, const void* dft, int B, int K, int V, int nch,
                                double invT, const Plan* plan, ChunkRec* recs, Tie* ties,
                                hipStream_t stream) {
  const int ngrp = (nch + kPassChunks - 1) / kPassChunks;
  const size_t blocks = (size_t)B * ngrp;
  if (blocks > 0x7fffffffu || nch > kMaxSampChunks) return hipErrorInvalidConfiguration;
  sample_pass_kernel<T><<<dim3((unsigned)blocks), dim3(kSampThreads), 0, stream>>>(
      static_cast<const T*>(tgt), static_cast<const T*>(dft), K, V, nch, ngrp, invT, plan, recs,
      ties);
  return hipGetLastError();
}

template <typename T>
static hipError_t sample_finish_t(const void* tgt, const void* dft, const float* u_final, int B,
                                  int K, int V, int nch, double invT, const Plan* plan,
                                  const ChunkRec* recs, const Tie* ties, int* out_tokens,
                                  double* rmass_out, hipStream_t stream) {
  if (nch > kMaxSampChunks) return hipErrorInvalidConfiguration;
  sample_finish_kernel<T><<<dim3(B), dim3(kSampThreads), 0, stream>>>(
      static_cast<const T*>(tgt), static_cast<const T*>(dft), u_final, K, V, nch, invT, plan,
      recs, ties, out_tokens, rmass_out);
  return hipGetLastError();
}

hipError_t launch_sample_pass(bool bf16, const void* tgt, const void* dft, int B, int K, int V,
                              int nch, double invT, const Plan* plan, ChunkRec* recs, Tie* ties,
                              hipStream_t stream) {
  return bf16 ? sample_pass_t<bf16_t>(tgt, dft, B, K, V, nch, invT, plan, recs, ties, stream)
              : sample_pass_t<float>(tgt, dft, B, K, V, nch, invT, plan, recs, ties, stream);
}

hipError_t launch_sample_finish(bool bf16, const void* tgt, const void* dft, const float* u_final,
                                int B, int K, int V, int nch, double invT, const Plan* plan,
                                const ChunkRec* recs, const Tie* ties, int* out_tokens,
                                double* rmass_out, hipStream_t stream) {
  return bf16 ? sample_finish_t<bf16_t>(tgt, dft, u_final, B, K, V, nch, invT, plan, recs, ties,
                                        out_tokens, rmass_out, stream)
              : sample_finish_t<float>(tgt, dft, u_final, B, K, V, nch, invT, plan, recs, ties,
                                       out_tokens, rmass_out, stream);
}

// Test hook: y[i] = exp64(x[i]).
__global__ __launch_bounds__(256) void exp64_selftest_kernel(const double* __restrict__ x,
                                                             double* __restrict__ y, int n) {
  __shared__ double tbl[SPECV_EXP64_N];
  exp64_stage_table(tbl);
  __syncthreads();
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    y[i] = exp64(x[i], tbl);
}

hipError_t launch_exp64_selftest(const double* x, double* y, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const long want = ((long)n + 255) / 256;
  const int blocks = (int)(want < 1024 ? want : 1024);
  exp64_selftest_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace specv
