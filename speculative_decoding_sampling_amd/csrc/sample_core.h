// Device code shared by the float64 sampler kernels: logit loads, block and
// wave reductions, the chunk pass of one 2048-token chunk (sums over the
// chunk, near ties) and the draw of one request from its chunk records.  The
// method and its precision argument are described where the kernels are
// (sample.hip).
#pragma once

#include <climits>

#include "common.h"
#include "exp64.h"
#include "wave_scan.h"

namespace specv {

// The row maxima and ratio estimate one row pair's chunk pass used, kept for
// the draw (small-batch kernel, which runs the pass for every pair).
struct PairStat {
  float mt, md;
  double g;
};

// The sampler's chunks are kSampThreads * PT tokens, PT per thread: 8 on the
// general path, kSmallPerThread on the one-kernel small-batch path: 4 tokens
// per thread, 1024-token chunks.  Its chunk passes are few and each one's
// dependency chain sets the time, so shorter per-thread chains win (measured
// on MI355X against 2 and 8 tokens per thread: 12.0 against 12.6 and 13.0 us
// at B=8, K=4, V=4096 fp32; 12.9 against 13.7 and 13.3 us at B=1, K=5,
// V=32000 bf16).
constexpr int kSmallPerThread = 4;
constexpr int kSmallChunk = kSampThreads * kSmallPerThread;


// This thread's PT logits of the chunk starting at element c0 (thread t holds
// elements c0 + PT t .. c0 + PT t + PT - 1).  The interior test is uniform per
// chunk.  Fewer than a vector's worth per thread load element by element.
template <typename T, int PT = kSampPerThread>
__device__ __forceinline__ void load8(const T* __restrict__ row, long c0, int V, float* out) {
  constexpr int N = Elem<T>::kPerVec;
  const long e0 = c0 + (long)threadIdx.x * PT;
  if constexpr (PT % N == 0) {
    const bool aligned = aligned16(row);
    if (aligned && c0 + kSampThreads * PT <= V) {
#pragma unroll
      for (int j = 0; j < PT / N; ++j) load_vec_fast(row, e0 + j * N, out + j * N);
    } else {
#pragma unroll
      for (int j = 0; j < PT / N; ++j)
        load_vec_checked(row, e0 + j * N, V, aligned, out + j * N);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i) out[i] = e0 + i < V ? to_f32(row[e0 + i]) : -INFINITY;
  }
}

constexpr int kSampWaves = kSampThreads / kWave;
constexpr int kTiePre = 2;       // near-tie slots per chunk the finish reads up front

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

// e = exp((z - m) / T), the unnormalised float64 weight of one logit, with
// mi = m / T of the row precomputed.
__device__ __forceinline__ double weight_e(float z, double mi, double invT, const double* tbl) {
  return exp64_logit(z, invT, mi, tbl);
}

// Residual weights max(e_t/S_t - e_d/S_d, 0) (resid) or target weights e_t of
// one thread's PT tokens; rSt = 1/S_t and rSd = 1/S_d.
template <typename T, int PT = kSampPerThread>
__device__ __forceinline__ void chunk_weights(const T* trow, const T* drow, long c0, int V,
                                              bool resid, double mti, double mdi, double invT,
                                              double rSt, double rSd, const double* tbl,
                                              double* w) {
  float zt[PT];
  load8<T, PT>(trow, c0, V, zt);
  if (resid) {
    float zd[PT];
    load8<T, PT>(drow, c0, V, zd);
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const double r = fma(weight_e(zt[i], mti, invT, tbl), rSt,
                           -weight_e(zd[i], mdi, invT, tbl) * rSd);
      w[i] = r > 0.0 ? r : 0.0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i) w[i] = weight_e(zt[i], mti, invT, tbl);
  }
}

// Raw logits of one thread's PT tokens, kept packed until used: 16-byte
// vectors, or element bit patterns when PT is below a vector.
template <typename T, int PT = kSampPerThread> struct Raw8 {
  static constexpr bool kVec = PT % Elem<T>::kPerVec == 0;
  uint4 w[kVec ? PT / Elem<T>::kPerVec : 1];
  uint32_t e[kVec ? 1 : PT];
};

// This thread's PT logits of the chunk starting at element c0, as raw words;
// elements at or past V read as -inf.  The interior test is uniform per chunk.
template <typename T, int PT = kSampPerThread>
__device__ __forceinline__ void load_raw8(const T* __restrict__ row, long c0, int V,
                                          Raw8<T, PT>& r) {
  constexpr int N = Elem<T>::kPerVec;
  const long e0 = c0 + (long)threadIdx.x * PT;
  if constexpr (Raw8<T, PT>::kVec) {
    constexpr int NV = PT / N;
    const bool aligned = aligned16(row);
    if (aligned && c0 + kSampThreads * PT <= V) {
#pragma unroll
      for (int j = 0; j < NV; ++j) r.w[j] = *reinterpret_cast<const uint4*>(row + e0 + j * N);
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) r.w[j] = load_raw_checked(row, e0 + j * N, V, aligned);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i) r.e[i] = e0 + i < V ? elem_bits(row, e0 + i) : neg_inf_bits(T{});
  }
}

template <typename T, int PT = kSampPerThread>
__device__ __forceinline__ void unpack8(const Raw8<T, PT>& r, float* z) {
  constexpr int N = Elem<T>::kPerVec;
  if constexpr (Raw8<T, PT>::kVec) {
#pragma unroll
    for (int j = 0; j < PT / N; ++j) unpack(r.w[j], z + j * N, T{});
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i)
      z[i] = sizeof(T) == 2 ? __uint_as_float(r.e[i] << 16) : __uint_as_float(r.e[i]);
  }
}

// Lane exchanges for the wave reductions, without per-lane index registers:
// DPP moves within a row of 16 lanes, a swizzle across the two rows of each
// half wave, and one permute across the halves.
template <int CTRL>
__device__ __forceinline__ double dpp_mov(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double swizzle_xor16(double v) {   // lane ^ 16 within 32 lanes
  const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(v), 0x401f);
  const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(v), 0x401f);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double permute_xor32(double v, int addr) {   // addr = (lane ^ 32) * 4
  const int lo = __builtin_amdgcn_ds_bpermute(addr, __double2loint(v));
  const int hi = __builtin_amdgcn_ds_bpermute(addr, __double2hiint(v));
  return __hiloint2double(hi, lo);
}

// Sums of four doubles over the wave.  The first two steps exchange halves
// of the set (lane ^ 32, then lane ^ 16), so each 16-lane row keeps one
// quantity; four DPP steps then sum within the row (quad swaps, then the
// half-row and row mirrors, which pair each lane with one in the other half
// once the halves are uniform).  Lane L ends with the full sum of quantity
// 2 * bit5(L) + bit4(L) of (a, b, c, d), summed in one fixed tree order.
__device__ __forceinline__ double wave_sum4(double a, double b, double c, double d) {
  const int lane = threadIdx.x % kWave;
  const bool h5 = lane & 32, h4 = lane & 16;
  const int addr32 = (lane ^ 32) << 2;
  double k0 = h5 ? c : a, k1 = h5 ? d : b;
  k0 += permute_xor32(h5 ? a : c, addr32);
  k1 += permute_xor32(h5 ? b : d, addr32);
  double k = h4 ? k1 : k0;
  k += swizzle_xor16(h4 ? k0 : k1);
  k += dpp_mov<0xb1>(k);     // quad_perm [1,0,3,2]: lane ^ 1
  k += dpp_mov<0x4e>(k);     // quad_perm [2,3,0,1]: lane ^ 2
  k += dpp_mov<0x141>(k);    // row_half_mirror
  k += dpp_mov<0x140>(k);    // row_mirror
  return k;
}

// Sums and near ties of one chunk whose logits this thread holds (PT per
// thread, token order = thread order), written to the chunk's record.
//
// With d = e_t - e_d g and band = e_d g w: d > band means p > q for certain,
// d < -band means p <= q for certain (the finish checks g against the exact
// ratio to a quarter of w), anything else is a near tie.  Tokens with
// e_t = 0 are never ties (their residual is 0).  The common path keeps only a
// per-lane "some near tie" flag; a wave that has one recomputes its weights
// and appends each near tie to an LDS list, stored in token order (rank by
// id) so that the stored slots do not depend on scheduling.  tcnt counts
// this chunk's ties; tcnt_next (the counter of a following chunk, if the
// caller loops) is cleared between the two barriers, after its last reader.
template <int PT = kSampPerThread>
__device__ __forceinline__ void pass_chunk(const float* zt, const float* zd, bool rej, long e0,
                                           double mti, double mdi, double invT, double g,
                                           const double* tbl, double* dl, Tie* tl, int* tcnt,
                                           int* tcnt_next, ChunkRec* __restrict__ rec,
                                           Tie* __restrict__ slot) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  double st = 0.0, sd = 0.0, at = 0.0, ad = 0.0;
  const double gw = g * kTieWindow;
  bool anytie = false;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const double et = weight_e(zt[i], mti, invT, tbl);
    st += et;
    if (rej) {
      const double ed = weight_e(zd[i], mdi, invT, tbl);
      sd += ed;
      const double dlt = fma(-ed, g, et);
      const double band = ed * gw;
      const bool sure = dlt > band;
      const double s01 = sure ? 1.0 : 0.0;           // weights are finite: fma adds or keeps
      at = fma(et, s01, at);
      ad = fma(ed, s01, ad);
      anytie |= !sure && dlt >= -band && et > 0.0;
    }
  }
  if (__ballot(anytie) != 0) {                       // rare: this wave has near ties
    // Recompute the weights (the same arithmetic, so the same classification)
    // and append each near tie to the chunk's list.
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const double et = weight_e(zt[i], mti, invT, tbl);
      const double ed = weight_e(zd[i], mdi, invT, tbl);
      const double dlt = fma(-ed, g, et);
      const double band = ed * gw;
      if (!(dlt > band) && dlt >= -band && et > 0.0) {
        const int s = atomicAdd(tcnt, 1);
        if (s < kTieCap) {
          Tie tv;
          tv.et = et;
          tv.ed = ed;
          tv.v = (int)(e0 + i);
          tv.pad = 0;
          tl[s] = tv;
        }
      }
    }
  }
  const double red = wave_sum4(st, sd, at, ad);
  __syncthreads();                                   // ties recorded; dl free from the last chunk
  if ((lane & 15) == 0) dl[wid * 4 + (lane >> 4)] = red;
  if (threadIdx.x == 0) *tcnt_next = 0;              // its last reader ran before the barrier
  __syncthreads();
  const int ntie = *tcnt;
  const int nst = min(ntie, kTieCap);
  if ((int)threadIdx.x < nst) {                      // store in token order
    const Tie tv = tl[threadIdx.x];
    int rank = 0;
    for (int j = 0; j < nst; ++j) rank += tl[j].v < tv.v;
    slot[rank] = tv;
  }
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
    r.ntie = ntie;
#pragma unroll
    for (int i = 0; i < 7; ++i) r.pad[i] = 0;
    *rec = r;
  }
}

// LDS of one draw.
struct DrawLds {
  double tbl[SPECV_EXP64_N];
  double dl[kSampWaves * 4];
  int il[kSampWaves * 2];
  double wts[kMaxSampChunks];
  int nredo;
  int redo[kMaxSampChunks];
};

// What a draw reads before its plan is needed: thread t < nch holds chunk
// t's record and that chunk's first kTiePre near-tie slots (read whether
// used or not; the slots exist).
struct DrawPre {
  bool have0;
  ChunkRec r0;
  Tie t0[kTiePre];
};

__device__ __forceinline__ void draw_prefetch(const ChunkRec* __restrict__ rb,
                                              const Tie* __restrict__ tb, int nch, DrawPre& p) {
  const int tid = threadIdx.x;
  p.have0 = tid < nch;
  if (p.have0) {
    p.r0 = rb[tid];
#pragma unroll
    for (int i = 0; i < kTiePre; ++i) p.t0[i] = tb[(size_t)tid * kTieCap + i];
  }
}

// The draw of request b from its chunk records rb[nch] and near ties tb, by
// the whole block: exact normalisers, chunk masses, the chunk holding
// t = uf * total and the scan inside it.  pl names the rows, the row maxima
// and the ratio estimate the chunk pass used; its path is a rejection or a
// bonus.  xs holds this thread's exp-table entries (fetched, not stored).
// Barriers are few: the chunk holding t is found by every wave on its own
// (a wave-wide blocked prefix over the chunk masses), and only the in-chunk
// scan combines the four waves.
template <typename T, int PT = kSampPerThread>
__device__ __forceinline__ void draw_request(const T* __restrict__ tgt, const T* __restrict__ dft,
                                             float uf, int b, int K, int V, int nch, double invT,
                                             const Plan& pl, const ChunkRec* __restrict__ rb,
                                             const Tie* __restrict__ tb, const DrawPre& pre,
                                             const Exp64Stage<kSampThreads>& xs, DrawLds& s,
                                             int* __restrict__ out_tokens,
                                             double* __restrict__ rmass_out) {
  const int tid = threadIdx.x, lane = tid % kWave, wid = tid / kWave;
  const bool rej = pl.path == kPathReject;
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  const T* drow = rej ? dft + draft_row_off(b, pl.drow, K, V) : nullptr;
  const double mti = (double)pl.mt * invT, mdi = (double)pl.md * invT;   // m / T
  const bool have0 = pre.have0;

  // exact normalisers: chunk sums added in a fixed order (thread-strided,
  // then the wave tree, then the four waves), and whether any chunk
  // overflowed its tie slots
  double a = 0.0, d = 0.0;
  int ovf = 0;
  if (have0) {
    a = pre.r0.et;
    d = pre.r0.ed;
    ovf = pre.r0.ntie > kTieCap;
  }
  for (int cc = tid + kSampThreads; cc < nch; cc += kSampThreads) {
    const ChunkRec r = rb[cc];
    a += r.et;
    d += r.ed;
    ovf |= r.ntie > kTieCap;
  }
  const double red = wave_sum4(a, d, 0.0, 0.0);
  const bool wovf = __ballot(ovf) != 0;
  if (tid == 0) s.nredo = 0;
  if (lane == 0 || lane == 16) s.dl[wid * 2 + (lane >> 4)] = red;
  if (lane == 0) s.il[wid] = wovf;
  xs.store(s.tbl);
  __syncthreads();                                   // table staged; wave sums
  double St = 0.0, Sd = 0.0;
  bool fb = false;
#pragma unroll
  for (int w = 0; w < kSampWaves; ++w) {
    St += s.dl[w * 2];
    Sd += s.dl[w * 2 + 1];
    fb |= s.il[w] != 0;
  }
  if (rej && !fb) fb = !(fabs(pl.g * Sd / St - 1.0) <= 0.25 * kTieWindow);
  const double rSt = 1.0 / St, rSd = 1.0 / Sd;

  // chunk masses: A_t/S_t - A_d/S_d plus the chunk's near ties resolved exactly;
  // a chunk with more ties than slots (or every chunk, if the estimate check
  // failed) gets its mass recomputed exactly from the logits.
  if (rej) {
    for (int cc = tid; cc < nch; cc += kSampThreads) {
      const bool first = cc == tid;
      const ChunkRec r = first ? pre.r0 : rb[cc];
      if (fb || r.ntie > kTieCap) {
        s.redo[atomicAdd(&s.nredo, 1)] = cc;
        continue;
      }
      double w = fma(r.at, rSt, -r.ad * rSd);
      const Tie* ts = tb + (size_t)cc * kTieCap;
      for (int i = 0; i < r.ntie; ++i) {
        Tie tv;
        if (first && i < kTiePre) {
#pragma unroll
          for (int j = 0; j < kTiePre; ++j)
            if (j == i) tv = pre.t0[j];
        } else {
          tv = ts[i];
        }
        const double x = fma(tv.et, rSt, -tv.ed * rSd);
        if (x > 0.0) w += x;
      }
      s.wts[cc] = w > 0.0 ? w : 0.0;
    }
  } else {
    for (int cc = tid; cc < nch; cc += kSampThreads) s.wts[cc] = cc == tid ? pre.r0.et : rb[cc].et;
  }
  __syncthreads();                                   // wts, redo list
  const int nredo = s.nredo;
  for (int i = 0; i < nredo; ++i) {                  // each chunk's mass is order-independent
    const int cc = s.redo[i];
    double w[PT];
    chunk_weights<T, PT>(trow, drow, (long)cc * (kSampThreads * PT), V, true, mti, mdi, invT, rSt,
                         rSd, s.tbl, w);
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < PT; ++k) sum += w[k];
    sum = block_sum(sum, s.dl);
    if (tid == 0) s.wts[cc] = sum;
  }
  if (nredo > 0) __syncthreads();                    // uniform

  // Blocked prefix over the chunk masses, per wave: lane l owns chunks
  // [l q, l q + q).  If the residual rounded to zero everywhere (unreachable
  // in exact arithmetic) the draw is from p_j: the target sums instead.
  const int q = (nch + kWave - 1) / kWave;
  const int c_lo = min(nch, lane * q), c_hi = min(nch, c_lo + q);
  bool resid = rej;
  double mine = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) mine += s.wts[cc];
  double incl = wave_incl_scan(mine);
  double total = lane_value(incl, kWave - 1);
  if (resid && !(total > 0.0)) {
    resid = false;
    mine = 0.0;
    for (int cc = c_lo; cc < c_hi; ++cc) mine += rb[cc].et;
    incl = wave_incl_scan(mine);
    total = lane_value(incl, kWave - 1);
  }
  const double rmass = (rej && resid) ? total : 0.0;
  const double t = (double)uf * total;
  const double excl = wave_shr1(incl);
  int cand = -1, last_pos = -1;
  double run = excl, pre_t = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) {
    const double m = (rej && !resid) ? rb[cc].et : s.wts[cc];
    const double before = run;
    run += m;
    if (cand < 0 && t < run) {
      cand = cc;
      pre_t = before;
    }
    if (m > 0.0) last_pos = cc;
  }
  const uint64_t hit = __ballot(cand >= 0);
  int cstar;
  double tprime;
  if (hit) {
    const int L = __ffsll((unsigned long long)hit) - 1;
    cstar = lane_value(cand, L);
    tprime = t - lane_value(pre_t, L);
  } else {                           // rounding fall-through: last chunk with mass
    const uint64_t pos = __ballot(last_pos >= 0);
    if (!pos) {                      // no positive mass at all (non-finite input)
      if (tid == 0) {
        out_tokens[(size_t)b * (K + 1) + pl.stop] = -1;
        if (rmass_out) rmass_out[b] = rmass;
      }
      return;                        // uniform: every wave saw the same masses
    }
    cstar = lane_value(last_pos, 63 - __clzll((long long)pos));
    tprime = INFINITY;
  }

  // in-chunk scan of chunk cstar
  const long e0 = (long)cstar * (kSampThreads * PT) + (long)tid * PT;
  double w[PT];
  chunk_weights<T, PT>(trow, drow, (long)cstar * (kSampThreads * PT), V, resid, mti, mdi, invT,
                       rSt, rSd, s.tbl, w);
  double mysum = 0.0;
#pragma unroll
  for (int i = 0; i < PT; ++i) mysum += w[i];
  const double wincl = wave_incl_scan(mysum);
  const double wex = wave_shr1(wincl);
  if (lane == kWave - 1) s.dl[wid] = wincl;          // dl's last readers passed a barrier
  __syncthreads();
  double off = 0.0;
#pragma unroll
  for (int wv = 0; wv < kSampWaves; ++wv)
    if (wv < wid) off += s.dl[wv];
  int vc = INT_MAX, vlast = -1;
  run = off + wex;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    run += w[i];
    if (vc == INT_MAX && tprime < run) vc = (int)(e0 + i);
    if (w[i] > 0.0) vlast = (int)(e0 + i);
  }
  // token order is thread order: the wave's first hit is its smallest
  const uint64_t h1 = __ballot(vc != INT_MAX), h2 = __ballot(vlast >= 0);
  const int wvc = h1 ? lane_value(vc, __ffsll((unsigned long long)h1) - 1) : INT_MAX;
  const int wvl = h2 ? lane_value(vlast, 63 - __clzll((long long)h2)) : -1;
  if (lane == 0) {
    s.il[wid] = wvc;
    s.il[kSampWaves + wid] = wvl;
  }
  __syncthreads();
  if (tid == 0) {
    int y = INT_MAX, yl = -1;
#pragma unroll
    for (int wv = 0; wv < kSampWaves; ++wv) {
      y = min(y, s.il[wv]);
      yl = max(yl, s.il[kSampWaves + wv]);
    }
    if (y == INT_MAX) y = yl;        // rounding fall-through inside the chunk
    out_tokens[(size_t)b * (K + 1) + pl.stop] = y;
    if (rmass_out) rmass_out[b] = rmass;
  }
}

}  // namespace specv
