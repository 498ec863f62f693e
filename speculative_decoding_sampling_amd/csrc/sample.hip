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

// e = exp((z - m) / T), the unnormalised float64 weight of one logit, with
// mi = m / T of the row precomputed.
__device__ __forceinline__ double weight_e(float z, double mi, double invT, const double* tbl) {
  return exp64_logit(z, invT, mi, tbl);
}

// Residual weights max(e_t/S_t - e_d/S_d, 0) (resid) or target weights e_t of
// one thread's 8 tokens; rSt = 1/S_t and rSd = 1/S_d.
template <typename T>
__device__ __forceinline__ void chunk_weights(const T* trow, const T* drow, long c0, int V,
                                              bool resid, double mti, double mdi, double invT,
                                              double rSt, double rSd, const double* tbl,
                                              double* w) {
  float zt[kSampPerThread];
  load8(trow, c0, V, zt);
  if (resid) {
    float zd[kSampPerThread];
    load8(drow, c0, V, zd);
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) {
      const double r = fma(weight_e(zt[i], mti, invT, tbl), rSt,
                           -weight_e(zd[i], mdi, invT, tbl) * rSd);
      w[i] = r > 0.0 ? r : 0.0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSampPerThread; ++i) w[i] = weight_e(zt[i], mti, invT, tbl);
  }
}

// Inclusive prefix sum over the wave, in lane order.
__device__ __forceinline__ double wave_incl_scan(double x) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

// Raw logits of one thread's 8 tokens, kept packed until used.
template <typename T> struct Raw8 {
  uint4 w[kSampPerThread / Elem<T>::kPerVec];
};

// This thread's 8 logits of the chunk starting at element c0, as raw words;
// elements at or past V read as -inf.  The interior test is uniform per chunk.
template <typename T>
__device__ __forceinline__ void load_raw8(const T* __restrict__ row, long c0, int V,
                                          Raw8<T>& r) {
  constexpr int N = Elem<T>::kPerVec, NV = kSampPerThread / N;
  const long e0 = c0 + (long)threadIdx.x * kSampPerThread;
  const bool aligned = aligned16(row);
  if (aligned && c0 + kSampChunk <= V) {
#pragma unroll
    for (int j = 0; j < NV; ++j) r.w[j] = *reinterpret_cast<const uint4*>(row + e0 + j * N);
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) r.w[j] = load_raw_checked(row, e0 + j * N, V, aligned);
  }
}

template <typename T>
__device__ __forceinline__ void unpack8(const Raw8<T>& r, float* z) {
  constexpr int N = Elem<T>::kPerVec;
#pragma unroll
  for (int j = 0; j < kSampPerThread / N; ++j) unpack(r.w[j], z + j * N, T{});
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

// Sums and near ties of one 2048-token chunk whose logits this thread holds
// (8 per thread, token order = thread order), written to the chunk's record.
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
  for (int i = 0; i < kSampPerThread; ++i) {
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
    for (int i = 0; i < kSampPerThread; ++i) {
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

// (a) chunk pass: one workgroup per (request, chunk).  The plan load and the
// exp table staging overlap; every logit load is issued before the first
// exp.  Many small workgroups keep the chip busy while others wait on memory.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_pass_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, int K, int V, int nch,
    double invT, const Plan* __restrict__ plan, ChunkRec* __restrict__ recs,
    Tie* __restrict__ ties) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double dl[kSampWaves * 4];
  __shared__ Tie tl[kTieCap];
  __shared__ int tcnt[2];

  const int c = blockIdx.x % nch, b = blockIdx.x / nch;
  // One round trip before the logits: the plan and this thread's exp-table
  // entries are requested together, the logit loads as soon as the plan
  // names the rows, and the table reaches LDS while those are in flight.  A
  // request with no draw (EOS, error) loads from target row 0, which every
  // request has, and leaves before using it.
  const Plan pl = plan[b];
  Exp64Stage<kSampThreads> xs;
  xs.fetch();
  const bool live = pl.path == kPathReject || pl.path == kPathBonus;
  const bool rej = pl.path == kPathReject;
  // Row indices are selected, not branched on, so the plan arrives in one
  // round trip; the draft row is dereferenced only after a rejection.
  const T* trow = tgt + target_row_off(b, live ? pl.trow : 0, K, V);
  const T* drow = dft + draft_row_off(b, rej ? pl.drow : 0, K, V);

  Raw8<T> rt, rd;
  load_raw8(trow, (long)c * kSampChunk, V, rt);
  if (rej) load_raw8(drow, (long)c * kSampChunk, V, rd);
  if (!live) return;                                 // uniform per block
  const double mti = (double)pl.mt * invT, mdi = (double)pl.md * invT;   // m / T
  xs.store(tbl);
  if (threadIdx.x == 0) tcnt[0] = 0;
  __syncthreads();                                   // table staged, tie counter clear
  float zt[kSampPerThread], zd[kSampPerThread];
  unpack8(rt, zt);
  if (rej) unpack8(rd, zd);
  const long e0 = (long)c * kSampChunk + (long)threadIdx.x * kSampPerThread;
  pass_chunk(zt, zd, rej, e0, mti, mdi, invT, pl.g, tbl, dl, tl, &tcnt[0], &tcnt[1],
             recs + (size_t)b * nch + c, ties + ((size_t)b * nch + c) * kTieCap);
}

// (b) the draw: one workgroup per request, after every chunk record exists.
// Barriers are few: the chunk holding t is found by every wave on its own
// (a wave-wide blocked prefix over the chunk masses), and only the in-chunk
// scan combines the four waves.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_finish_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const float* __restrict__ u_final,
    int K, int V, int nch, double invT, const Plan* __restrict__ plan,
    const ChunkRec* __restrict__ recs, const Tie* __restrict__ ties, int* __restrict__ out_tokens,
    double* __restrict__ rmass_out) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double dl[kSampWaves * 4];
  __shared__ int il[kSampWaves * 2];
  __shared__ double wts[kMaxSampChunks];
  __shared__ int s_nredo;
  __shared__ int redo[kMaxSampChunks];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wid = tid / kWave;
  // Everything that does not depend on the plan is requested with it: the
  // exp table, this thread's first chunk record and that chunk's first
  // kTiePre near-tie slots (read whether used or not; the slots exist).  The
  // table reaches LDS just before the first barrier.
  Exp64Stage<kSampThreads> xs;
  xs.fetch();
  const Plan pl = plan[b];
  const ChunkRec* rb = recs + (size_t)b * nch;
  const Tie* tb = ties + (size_t)b * nch * kTieCap;
  const bool have0 = tid < nch;
  ChunkRec r0;
  Tie t0[kTiePre];
  if (have0) {
    r0 = rb[tid];
#pragma unroll
    for (int i = 0; i < kTiePre; ++i) t0[i] = tb[(size_t)tid * kTieCap + i];
  }
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per block
  const bool rej = pl.path == kPathReject;
  const T* trow = tgt + target_row_off(b, pl.trow, K, V);
  const T* drow = rej ? dft + draft_row_off(b, pl.drow, K, V) : nullptr;
  const double mti = (double)pl.mt * invT, mdi = (double)pl.md * invT;   // m / T

  // exact normalisers: chunk sums added in a fixed order (thread-strided,
  // then the wave tree, then the four waves), and whether any chunk
  // overflowed its tie slots
  double a = 0.0, d = 0.0;
  int ovf = 0;
  if (have0) {
    a = r0.et;
    d = r0.ed;
    ovf = r0.ntie > kTieCap;
  }
  for (int cc = tid + kSampThreads; cc < nch; cc += kSampThreads) {
    const ChunkRec r = rb[cc];
    a += r.et;
    d += r.ed;
    ovf |= r.ntie > kTieCap;
  }
  const double red = wave_sum4(a, d, 0.0, 0.0);
  const bool wovf = __ballot(ovf) != 0;
  if (tid == 0) s_nredo = 0;
  if (lane == 0 || lane == 16) dl[wid * 2 + (lane >> 4)] = red;
  if (lane == 0) il[wid] = wovf;
  xs.store(tbl);
  __syncthreads();                                   // table staged; wave sums
  double St = 0.0, Sd = 0.0;
  bool fb = false;
#pragma unroll
  for (int w = 0; w < kSampWaves; ++w) {
    St += dl[w * 2];
    Sd += dl[w * 2 + 1];
    fb |= il[w] != 0;
  }
  if (rej && !fb) fb = !(fabs(pl.g * Sd / St - 1.0) <= 0.25 * kTieWindow);
  const double rSt = 1.0 / St, rSd = 1.0 / Sd;

  // chunk masses: A_t/S_t - A_d/S_d plus the chunk's near ties resolved exactly;
  // a chunk with more ties than slots (or every chunk, if the estimate check
  // failed) gets its mass recomputed exactly from the logits.
  if (rej) {
    for (int cc = tid; cc < nch; cc += kSampThreads) {
      const bool first = cc == tid;
      const ChunkRec r = first ? r0 : rb[cc];
      if (fb || r.ntie > kTieCap) {
        redo[atomicAdd(&s_nredo, 1)] = cc;
        continue;
      }
      double w = fma(r.at, rSt, -r.ad * rSd);
      const Tie* ts = tb + (size_t)cc * kTieCap;
      for (int i = 0; i < r.ntie; ++i) {
        Tie tv;
        if (first && i < kTiePre) {
#pragma unroll
          for (int j = 0; j < kTiePre; ++j)
            if (j == i) tv = t0[j];
        } else {
          tv = ts[i];
        }
        const double x = fma(tv.et, rSt, -tv.ed * rSd);
        if (x > 0.0) w += x;
      }
      wts[cc] = w > 0.0 ? w : 0.0;
    }
  } else {
    for (int cc = tid; cc < nch; cc += kSampThreads) wts[cc] = cc == tid ? r0.et : rb[cc].et;
  }
  __syncthreads();                                   // wts, redo list
  const int nredo = s_nredo;
  for (int i = 0; i < nredo; ++i) {                  // each chunk's mass is order-independent
    const int cc = redo[i];
    double w[kSampPerThread];
    chunk_weights(trow, drow, (long)cc * kSampChunk, V, true, mti, mdi, invT, rSt, rSd, tbl, w);
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < kSampPerThread; ++k) sum += w[k];
    sum = block_sum(sum, dl);
    if (tid == 0) wts[cc] = sum;
  }
  if (nredo > 0) __syncthreads();                    // uniform

  // Blocked prefix over the chunk masses, per wave: lane l owns chunks
  // [l q, l q + q).  If the residual rounded to zero everywhere (unreachable
  // in exact arithmetic) the draw is from p_j: the target sums instead.
  const int q = (nch + kWave - 1) / kWave;
  const int c_lo = min(nch, lane * q), c_hi = min(nch, c_lo + q);
  bool resid = rej;
  double mine = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) mine += wts[cc];
  double incl = wave_incl_scan(mine);
  double total = __shfl(incl, kWave - 1, kWave);
  if (resid && !(total > 0.0)) {
    resid = false;
    mine = 0.0;
    for (int cc = c_lo; cc < c_hi; ++cc) mine += rb[cc].et;
    incl = wave_incl_scan(mine);
    total = __shfl(incl, kWave - 1, kWave);
  }
  const double rmass = (rej && resid) ? total : 0.0;
  const double t = (double)u_final[b] * total;
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  int cand = -1, last_pos = -1;
  double run = excl, pre = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) {
    const double m = (rej && !resid) ? rb[cc].et : wts[cc];
    const double before = run;
    run += m;
    if (cand < 0 && t < run) {
      cand = cc;
      pre = before;
    }
    if (m > 0.0) last_pos = cc;
  }
  const uint64_t hit = __ballot(cand >= 0);
  int cstar;
  double tprime;
  if (hit) {
    const int L = __ffsll((unsigned long long)hit) - 1;
    cstar = __shfl(cand, L, kWave);
    tprime = t - __shfl(pre, L, kWave);
  } else {                           // rounding fall-through: last chunk with mass
    const uint64_t pos = __ballot(last_pos >= 0);
    if (!pos) {                      // no positive mass at all (non-finite input)
      if (tid == 0) {
        out_tokens[(size_t)b * (K + 1) + pl.stop] = -1;
        if (rmass_out) rmass_out[b] = rmass;
      }
      return;                        // uniform: every wave saw the same masses
    }
    cstar = __shfl(last_pos, 63 - __clzll((long long)pos), kWave);
    tprime = INFINITY;
  }

  // in-chunk scan of chunk cstar
  const long e0 = (long)cstar * kSampChunk + (long)tid * kSampPerThread;
  double w[kSampPerThread];
  chunk_weights(trow, drow, (long)cstar * kSampChunk, V, resid, mti, mdi, invT, rSt, rSd, tbl, w);
  double mysum = 0.0;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) mysum += w[i];
  const double wincl = wave_incl_scan(mysum);
  double wex = __shfl_up(wincl, 1, kWave);
  if (lane == 0) wex = 0.0;
  if (lane == kWave - 1) dl[wid] = wincl;            // dl's last readers passed a barrier
  __syncthreads();
  double off = 0.0;
#pragma unroll
  for (int wv = 0; wv < kSampWaves; ++wv)
    if (wv < wid) off += dl[wv];
  int vc = INT_MAX, vlast = -1;
  run = off + wex;
#pragma unroll
  for (int i = 0; i < kSampPerThread; ++i) {
    run += w[i];
    if (vc == INT_MAX && tprime < run) vc = (int)(e0 + i);
    if (w[i] > 0.0) vlast = (int)(e0 + i);
  }
  // token order is thread order: the wave's first hit is its smallest
  const uint64_t h1 = __ballot(vc != INT_MAX), h2 = __ballot(vlast >= 0);
  const int wvc = h1 ? __shfl(vc, __ffsll((unsigned long long)h1) - 1, kWave) : INT_MAX;
  const int wvl = h2 ? __shfl(vlast, 63 - __clzll((long long)h2), kWave) : -1;
  if (lane == 0) {
    il[wid] = wvc;
    il[kSampWaves + wid] = wvl;
  }
  __syncthreads();
  if (tid == 0) {
    int y = INT_MAX, yl = -1;
#pragma unroll
    for (int wv = 0; wv < kSampWaves; ++wv) {
      y = min(y, il[wv]);
      yl = max(yl, il[kSampWaves + wv]);
    }
    if (y == INT_MAX) y = yl;        // rounding fall-through inside the chunk
    out_tokens[(size_t)b * (K + 1) + pl.stop] = y;
    if (rmass_out) rmass_out[b] = rmass;
  }
}

template <typename T>
static hipError_t sample_pass_t(const void* tgt, const void* dft, int B, int K, int V, int nch,
                                double invT, const Plan* plan, ChunkRec* recs, Tie* ties,
                                hipStream_t stream) {
  const size_t blocks = (size_t)B * nch;
  if (blocks > 0x7fffffffu || nch > kMaxSampChunks) return hipErrorInvalidConfiguration;
  sample_pass_kernel<T><<<dim3((unsigned)blocks), dim3(kSampThreads), 0, stream>>>(
      static_cast<const T*>(tgt), static_cast<const T*>(dft), K, V, nch, invT, plan, recs,
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
  exp64_stage_table<256>(tbl);
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
