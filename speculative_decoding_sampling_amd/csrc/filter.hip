// Top-k / top-p filtering for a small top-k: the candidate select.
//
// p and q are the target's and the draft's distributions after temperature,
// top-k and top-p, each row filtered on its own (nickwang.xyz
// "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布": both already
// include those settings).  top-k keeps every logit >= the k-th largest;
// top-p then keeps the shortest prefix of the renormalised top-k
// distribution, ordered by logit (descending) then token id, whose mass
// reaches top_p, with the crossing token and its ties.
//
// One pass over HBM.  filter_cand streams each needed row in 8192-token
// chunks and keeps a superset of the chunk's top-k: every thread takes the
// max of its 32 logits and T_c is the k-th largest of the 256 thread maxima,
// so the chunk has >= k logits >= T_c; the chunk's k-th largest logit is
// >= T_c, and the row's k-th largest is at least the chunk's, so every logit
// the row keeps is a candidate.  The candidates (~60 per chunk, ~1.1 k per
// 152k-token row on random data) go to a per-chunk slot.  filter_merge
// selects tau_k, the k-th largest candidate, by radix select, sorts the
// candidates >= tau_k in LDS by (logit desc, id asc), runs top-p in float64
// over that sorted prefix, and writes the row
// maximum, the final threshold, the float64 normaliser over the kept set and
// the kept tokens sorted by id.  Nothing downstream reads the full rows
// again: acceptance needs two gathers per position, and the residual or
// bonus draw walks the target row's kept list (p is zero elsewhere).
#include <algorithm>
#include <cfloat>
#include <climits>

#include "common.h"
#include "exp64.h"

#include "filter_common.h"
#include "radix_select.h"

namespace specv {

static_assert(kFiltSortMax % kFiltThreads == 0, "the merge gather gives each thread whole steps");
static_assert(kFiltMaxChunks <= kWave, "one wave scans a row's chunk counts");
constexpr int kRadixBins = 2048;               // the merge's radix select: 11-bit digits
static_assert(kFiltSortMax / kFiltThreads <= 16, "a thread's block of the list stays small");

// The value of lane (lane ^ S).  S = 1, 2: one DPP quad permutation; S = 4:
// the half-row mirror (lane i of each 8 takes 7 - i) then the quad reversal,
// which together send i to i ^ 4; S = 8: the half-row mirror then the row
// mirror (i of each 16 takes 15 - i), together i ^ 8; S = 16: a swizzle in
// bit-mask mode (xor 16 within each 32 lanes); S = 32: a permute.  Only the
// last two go through the LDS unit.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (S == 1) return dpp_u32<0xb1>(v);                       // quad_perm [1,0,3,2]
  else if constexpr (S == 2) return dpp_u32<0x4e>(v);                  // quad_perm [2,3,0,1]
  else if constexpr (S == 4) return dpp_u32<0x1b>(dpp_u32<0x141>(v));  // half mirror, [3,2,1,0]
  else if constexpr (S == 8) return dpp_u32<0x140>(dpp_u32<0x141>(v)); // half mirror, mirror
  else if constexpr (S == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401f);
  else return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((threadIdx.x % kWave) ^ 32) << 2, (int)v);
}

template <int S>
__device__ __forceinline__ uint64_t lane_xor(uint64_t v) {
  const uint32_t lo = lane_xor<S>((uint32_t)v), hi = lane_xor<S>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange stage of the bitonic network at a fixed size and stride.
// Lane l keeps the larger key where ((l & SIZE) == 0) == ((l & STRIDE) == 0),
// the smaller elsewhere: a fixed set of lanes per stage, given to the select
// as a constant lane mask (scalar moves) instead of being derived from the
// lane id with vector instructions.
template <int SIZE, int STRIDE>
constexpr unsigned long long bitonic_max_lanes() {
  unsigned long long m = 0;
  for (int l = 0; l < 64; ++l)
    if (((l & SIZE) == 0) == ((l & STRIDE) == 0)) m |= 1ull << l;
  return m;
}
template <int SIZE, int STRIDE, typename K>
__device__ __forceinline__ K bitonic_stage(K key, int) {
  const K other = lane_xor<STRIDE>(key);
  const bool keep_max = __builtin_amdgcn_inverse_ballot_w64(bitonic_max_lanes<SIZE, STRIDE>());
  return keep_max ? (key > other ? key : other) : (key < other ? key : other);
}
template <int SIZE, int STRIDE, typename K>
__device__ __forceinline__ K bitonic_merge(K key, int lane) {
  key = bitonic_stage<SIZE, STRIDE>(key, lane);
  if constexpr (STRIDE > 1) key = bitonic_merge<SIZE, STRIDE / 2>(key, lane);
  return key;
}
template <int SIZE, typename K>
__device__ __forceinline__ K bitonic_sort(K key, int lane) {
  if constexpr (SIZE > 2) key = bitonic_sort<SIZE / 2>(key, lane);
  return bitonic_merge<SIZE, SIZE / 2>(key, lane);
}

// Descending sort of one key per lane across a wave (bitonic network), for
// 32- and 64-bit keys.
template <typename K>
__device__ __forceinline__ K wave_sort_desc(K key) {
  static_assert(kWave == 64, "the lane exchanges are written for wave64");
  return bitonic_sort<kWave>(key, (int)(threadIdx.x % kWave));
}

// ---------------------------------------------------------------------------
// filter_cand: per (request, needed row, 8192-token chunk).  In a full chunk
// of a 16-byte aligned row, thread t holds the 16-byte vectors j = 0..NV-1 at
// elements e_base + (256 j + t) N .. + N - 1 (N logits per vector): every
// load instruction of a wave reads 1 KB of consecutive bytes.  Any other
// chunk uses element loads, thread t holding tokens e_base + 256 j + t,
// j = 0..31, issued back-to-back (the address is clamped instead of branched
// on); a chunk with 256 or more valid tokens then gives every thread data, so
// every wave's threshold is a real logit.  Which 32 logits a thread holds
// does not matter to the threshold argument below, only that each thread's
// maximum is one of the chunk's logits.  A chunk with at most `slot` valid
// tokens (only a row's last chunk can have so few) keeps all of them.
template <typename T>
__global__ __launch_bounds__(kFiltThreads) void filter_cand_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    int K, int V, int nch, int top_k, int cap, int row_stride, uint64_t* __restrict__ cand,
    int* __restrict__ counts, int* __restrict__ redo_count) {
  __shared__ uint32_t tw[kFiltThreads / kWave];
  __shared__ uint32_t lists[kFiltThreads];
  __shared__ int il[kFiltThreads / kWave];
  const int R = 2 * K + 1;
  const int chunk = blockIdx.x % nch;
  const int rr = blockIdx.x / nch;
  // The block merge's row list starts empty (the merge kernels run after
  // this one, so the clear is ordered before their appends).
  if (blockIdx.x == 0 && threadIdx.x == 0) *redo_count = 0;
  const int r = rr % R, b = rr / R;
  const int nb = draft_len ? draft_len[b] : 0;      // null: no drafts (sampling)
  if (nb < 0 || nb > K) return;
  bool is_target;
  int k;
  if (!row_needed(r, K, nb, is_target, k)) return;
  const T* row = is_target ? tgt + target_row_off(b, k, K, V) : dft + draft_row_off(b, k, K, V);
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const long e_base = (long)chunk * kFiltChunk;
  const int n_valid = (int)min((long)kFiltChunk, (long)V - e_base);
  const int slot = chunk == nch - 1 ? row_stride - (nch - 1) * cap : cap;
  constexpr int N = Elem<T>::kPerVec;
  const bool vec = n_valid == kFiltChunk && aligned16(row);   // uniform per block
  // token id of v[j], formed where a candidate is stored (the empty asm keeps
  // the compiler from computing all 32 ahead and holding them)
  const uint32_t id_base = (uint32_t)(vec ? e_base + threadIdx.x * N : e_base + threadIdx.x);
  auto id_of = [&](int j) -> uint32_t {
    uint32_t ib = id_base;
    asm volatile("" : "+v"(ib));
    return ib + (vec ? (uint32_t)((j / N) * kFiltThreads * N + j % N) : (uint32_t)(j * kFiltThreads));
  };
  // Addressing keeps registers for the logits: each vector load adds this
  // lane's one offset to a per-vector base that is uniform (scalar
  // registers), and each element load's clamped offset is formed right
  // before its load (the empty asm pins it there) instead of all 32 first.
  const T* cb = row + e_base;
  float v[kFiltPerThread];
  if (vec) {
    const uint32_t lo = threadIdx.x * N;
#pragma unroll
    for (int j = 0; j < kFiltPerThread / N; ++j)
      load_vec_stream(cb + (size_t)j * kFiltThreads * N, lo, v + j * N);
  } else {
    // offsets past the row are clamped to its last token and read as -inf
    const uint32_t last = (uint32_t)(n_valid - 1);
#pragma unroll
    for (int j = 0; j < kFiltPerThread; ++j) {
      // a 32-bit byte offset from the uniform base: one address register
      uint32_t ob = min((uint32_t)(j * kFiltThreads) + threadIdx.x, last) * (uint32_t)sizeof(T);
      asm volatile("" : "+v"(ob));
      v[j] = to_f32(*reinterpret_cast<const T*>(reinterpret_cast<const char*>(cb) + ob));
    }
#pragma unroll
    for (int j = 0; j < kFiltPerThread; ++j)
      if ((uint32_t)(j * kFiltThreads) + threadIdx.x > last) v[j] = -INFINITY;
  }
  // The threshold search compares floats: for finite or -inf logits their
  // order is exactly the order of the keys (fkey gives -0 and +0 one key,
  // and float compares treat them as equal), so only the thread maxima and
  // the candidates are turned into keys.
  uint32_t tc = kNegInfKey;                          // keep every valid logit ...
  if (n_valid > slot) {                              // ... unless the chunk is larger than its slot
    // T_c = the top_k-th largest of the 256 thread maxima: top_k distinct
    // threads each hold a logit >= T_c.  Each wave sorts its maxima; every
    // thread ranks its own maximum against the four sorted lists.
    float fm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kFiltPerThread; ++j) fm = fmaxf(fm, v[j]);
    const uint32_t tmax = fkey(fm);
    lists[threadIdx.x] = wave_sort_desc(tmax);        // wave w's list at [64w, 64w + 64)
    __syncthreads();
    // rank = thread maxima >= tmax: in each descending list the count of
    // entries >= tmax, by binary lifting (pos only grows while its entry
    // is >= tmax), the four lists interleaved so their reads overlap
    constexpr int kLists = kFiltThreads / kWave;
    int pos[kLists];
#pragma unroll
    for (int w = 0; w < kLists; ++w) pos[w] = 0;
#pragma unroll
    for (int step = kWave / 2; step >= 1; step >>= 1)
#pragma unroll
      for (int w = 0; w < kLists; ++w)
        if (lists[w * kWave + pos[w] + step - 1] >= tmax) pos[w] += step;
    int rank = 0;                                    // pos <= 63: one last entry to test
#pragma unroll
    for (int w = 0; w < kLists; ++w) rank += pos[w] + (lists[w * kWave + pos[w]] >= tmax ? 1 : 0);
    uint32_t best = rank >= top_k ? tmax : 0u;
    best = max(best, lane_xor<32>(best));
    best = max(best, lane_xor<16>(best));
    best = max(best, lane_xor<8>(best));
    best = max(best, lane_xor<4>(best));
    best = max(best, lane_xor<2>(best));
    best = max(best, lane_xor<1>(best));
    if (lane == 0) tw[wid] = best;
    __syncthreads();
    tc = tw[0];
#pragma unroll
    for (int w = 1; w < kFiltThreads / kWave; ++w) tc = max(tc, tw[w]);
  }
  // candidates: finite logits with key >= tc, written in thread order, as
  // one float compare each (key >= tc with tc above -inf's key is
  // v >= unkey(tc); otherwise every finite logit, v >= -FLT_MAX).  They
  // are rare (~60 of 8192 on random data): each thread counts its own, and
  // the store loop repeats the compare, skipping a position no lane of the
  // wave has.
  const float thr = tc > kNegInfKey ? unkey(tc) : -FLT_MAX;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kFiltPerThread; ++j) mine += v[j] >= thr ? 1 : 0;
  // exclusive offset of this thread's candidates in the block: a DPP scan
  // per wave, the four wave totals through LDS (il is not used before here)
  const int incl = wave_incl_scan_i32(mine);
  if (lane == kWave - 1) il[wid] = incl;
  __syncthreads();
  int total = 0, off = incl - mine;
#pragma unroll
  for (int w = 0; w < kFiltThreads / kWave; ++w) {
    if (w < wid) off += il[w];
    total += il[w];
  }
  uint64_t* dst = cand + (size_t)rr * row_stride + (size_t)chunk * cap;
#pragma unroll
  for (int j = 0; j < kFiltPerThread; ++j) {
    const bool c = v[j] >= thr;
    if (__ballot(c) != 0ull) {
      if (c) {
        // the key, formed here for the 64-bit word (the empty asm keeps it a
        // fresh register rather than the high half of a pair)
        uint32_t hi = fkey(v[j]);
        asm volatile("" : "+v"(hi));
        if (off < slot) dst[off] = ((uint64_t)hi << 32) | (uint64_t)(0xffffffffu - id_of(j));
        ++off;
      }
    }
  }
  if (threadIdx.x == 0) counts[(size_t)rr * nch + chunk] = total;
}

// ---------------------------------------------------------------------------
// filter_merge: per (request, needed row).
__device__ __forceinline__ void lds_bitonic_desc(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < n / 2; idx += kFiltThreads) {
        const int lo = 2 * stride * (idx / stride) + (idx % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x < y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// filter_merge_wave: the merge of one row by one wave, four rows per
// workgroup, for the usual row: at most kWaveCand candidates (held in
// registers, kWaveCand / 64 per lane) and at most 64 of them >= tau_k (the
// top-k and its ties).  Nothing waits at a workgroup barrier.
//  - chunk offsets: one lane per chunk, a wave scan;
//  - gather: every load first, the chunk of flat index f by binary search
//    over the offsets (in this wave's LDS);
//  - tau_k = the largest 32-bit key v with #{keys >= v} >= k, bit by bit
//    from the top (up to 32 rounds of compare-and-count, counted with
//    ballots and scalar popcounts);
//  - the keys >= tau_k, one per lane, sorted descending in registers; top-p
//    in float64 by a lane-order scan and ballots; the kept list sorted by id
//    in registers.
// A row outside those bounds (a chunk over its slot, more candidates, more
// than 64 keys >= tau_k) is marked kStatusRedo and merged by
// filter_merge_kernel, which runs next and leaves every other row alone.
constexpr int kWaveCand = 2048;
constexpr int kWavePer = kWaveCand / kWave;           // candidates per lane
constexpr int kStatusRedo = 3;                        // internal: the block merge takes the row
constexpr int kMergeWaves = kFiltThreads / kWave;     // rows per workgroup

// Maximum of an int over the wave on DPP (quad swaps, half-row and row
// mirrors), then the four row maxima read as scalars: short latency, no LDS.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<0xb1>(v));
  v = max(v, dpp_i<0x4e>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<0xb1>((int)v));
  v = max(v, (uint32_t)dpp_i<0x4e>((int)v));
  v = max(v, (uint32_t)dpp_i<0x141>((int)v));
  v = max(v, (uint32_t)dpp_i<0x140>((int)v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

__global__ __launch_bounds__(kFiltThreads) void filter_merge_wave_kernel(
    const int* __restrict__ draft_len, int B, int K, int nch, int cap, int row_stride,
    int top_k, float top_p, double invT, const uint64_t* __restrict__ cand,
    const int* __restrict__ counts, FiltRow* __restrict__ rows, Kept* __restrict__ kept,
    int* __restrict__ redo_count, int* __restrict__ redo_rows) {
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ uint64_t s_buf[kMergeWaves][kWave];
  __shared__ uint32_t s_sel[kMergeWaves][4 * kWave];
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int R = 2 * K + 1;
  const int rr = blockIdx.x * kMergeWaves + wid;
  exp64_stage_table<kFiltThreads>(tbl);
  __syncthreads();                                   // the only barrier: the exp table
  if (rr >= B * R) return;
  const int r = rr % R, b = rr / R;
  // the row's chunk counts are requested with draft_len (lane c = chunk c)
  const int cnt = lane < nch ? counts[(size_t)rr * nch + lane] : 0;
  const int nb = draft_len ? draft_len[b] : 0;       // null: no drafts (sampling)
  if (nb < 0 || nb > K) return;
  bool is_target;
  int k;
  if (!row_needed(r, K, nb, is_target, k)) return;

  FiltRow out;
  out.pad = 0;
  // chunk offsets and the candidate total
  int n = 0, over = 0;
  if (lane < nch) {
    const int slot = lane == nch - 1 ? row_stride - (nch - 1) * cap : cap;
    over = cnt > slot;
    n = min(cnt, slot);
  }
  const int incl = wave_incl_scan_i32(n);
  const int n_all = __builtin_amdgcn_readlane(incl, kWave - 1);
  // lanes per chunk: lane l reads chunk l / q, its entries l % q, l % q + q, ...
  const int q = kWave / max(nch, 1);
  const int nmax = wave_max_i(n);
  if (__ballot(over) != 0 || nmax > q * kWavePer) {  // the block merge takes it
    if (lane == 0) {
      out.m = 0.f;
      out.tau = 0.f;
      out.S = 0.0;
      out.count = 0;
      out.status = kStatusRedo;
      rows[rr] = out;
      redo_rows[atomicAdd(redo_count, 1)] = rr;      // the block merge's list
    }
    return;
  }
  if (n_all == 0) {                                  // no finite logit in the row
    if (lane == 0) {
      out.m = -INFINITY;
      out.tau = INFINITY;
      out.S = 0.0;
      out.count = 0;
      out.status = 2;
      rows[rr] = out;
    }
    return;
  }
  // gather the key halves (a candidate is key << 32 | ~id): every address is
  // arithmetic, every load unconditional (clamped into the chunk's slot), so
  // the loads leave back to back; entries past the chunk's count read 0,
  // below every key
  const int c_me = min(lane / q, nch - 1), s_me = lane % q;
  const bool lane_on = lane < q * nch;
  const int n_me = lane_on ? __shfl(n, c_me, kWave) : 0;
  const uint64_t* rowc = cand + (size_t)rr * row_stride;
  const uint32_t* rowh = reinterpret_cast<const uint32_t*>(rowc);
  const int base = c_me * cap;
  uint32_t key[kWavePer];
#pragma unroll
  for (int i = 0; i < kWavePer; ++i)
    key[i] = rowh[2 * (base + min(s_me + q * i, max(n_me - 1, 0))) + 1];
#pragma unroll
  for (int i = 0; i < kWavePer; ++i)
    if (s_me + q * i >= n_me) key[i] = 0u;

  // tau_k, the largest key v with #{keys >= v} >= kk.  T0 = the kk-th
  // largest of the 64 lane maxima is a lower bound (kk lanes hold a key
  // >= T0); the keys >= T0 (usually a few more than kk) are compacted, at
  // most four per lane, and tau_k is found among them bit by bit from the
  // top.  With more than 256 such keys, among all of them.  (A bound from the
  // kk-th largest of four group maxima per lane is tighter, but its own walk
  // costs more than it saves.)
  const int kk = min(top_k, n_all);
  uint32_t lmax = 0u;
#pragma unroll
  for (int i = 0; i < kWavePer; ++i) lmax = max(lmax, key[i]);
  uint32_t t0 = 0u, kmax;
  if (kk <= kWave) {
    const uint32_t sm = wave_sort_desc(lmax);
    t0 = (uint32_t)__builtin_amdgcn_readlane((int)sm, kk - 1);
    kmax = (uint32_t)__builtin_amdgcn_readlane((int)sm, 0);
  } else {
    kmax = wave_max_u(lmax);
  }
  const int top = 32 - __clz((int)(t0 ^ kmax));     // bits left to decide
  const uint32_t known = top >= 32 ? 0u : kmax & (0xffffffffu << top);
  int c0 = 0;
#pragma unroll
  for (int i = 0; i < kWavePer; ++i) c0 += key[i] >= t0 && key[i] > 0u ? 1 : 0;
  const int incl0 = wave_incl_scan_i32(c0);
  const int nt = __builtin_amdgcn_readlane(incl0, kWave - 1);
  uint32_t tk = known;
  int L = nt;                                        // #{keys >= tk} (every key >= t0 here)
  if (nt <= 4 * kWave) {
    int qpos = incl0 - c0;
#pragma unroll
    for (int i = 0; i < kWavePer; ++i)
      if (key[i] >= t0 && key[i] > 0u) s_sel[wid][qpos++] = key[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t k4[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int e = lane + kWave * r4;
      k4[r4] = e < nt ? s_sel[wid][e] : 0u;
    }
    // each round counts with ballots and scalar popcounts: four VALU
    // compares instead of a wave reduction
#pragma unroll 1
    for (int bit = top - 1; bit >= 0; --bit) {
      const uint32_t tryv = tk | (1u << bit);
      int c = 0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) c += __popcll(__ballot(k4[r4] >= tryv));
      if (c >= kk) {
        tk = tryv;
        L = c;
      }
    }
  } else {
#pragma unroll 1
    for (int bit = top - 1; bit >= 0; --bit) {
      const uint32_t tryv = tk | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < kWavePer; ++i) c += __popcll(__ballot(key[i] >= tryv));
      if (c >= kk) {
        tk = tryv;
        L = c;
      }
    }
  }
  if (L > kWave) {                                   // the top-k and its ties exceed a wave
    if (lane == 0) {
      out.m = 0.f;
      out.tau = 0.f;
      out.S = 0.0;
      out.count = 0;
      out.status = kStatusRedo;
      rows[rr] = out;
      redo_rows[atomicAdd(redo_count, 1)] = rr;      // the block merge's list
    }
    return;
  }
  // the keys >= tau_k: their candidate words' indices compacted one per
  // lane, then each lane reads its whole word (one round trip); sorted
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kWavePer; ++i) mine += key[i] >= tk ? 1 : 0;
  const int pincl = wave_incl_scan_i32(mine);
  int pos = pincl - mine;
#pragma unroll
  for (int i = 0; i < kWavePer; ++i)
    if (key[i] >= tk) reinterpret_cast<int*>(s_buf[wid])[pos++] = base + s_me + q * i;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t x = 0ull;                                 // 0 sorts last
  if (lane < L) x = rowc[reinterpret_cast<int*>(s_buf[wid])[lane]];
  x = wave_sort_desc(x);

  // top-p over the sorted prefix, float64 (lane i holds entry i)
  const uint32_t k32 = lane < L ? (uint32_t)(x >> 32) : 0u;
  const float m = unkey((uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), 0));
  const double md = (double)m;
  const bool in = lane < L;
  const double wgt = in ? exp64(((double)unkey(k32) - md) * invT, tbl) : 0.0;
  const double run = wave_incl_scan(wgt);
  const double tot = lane_value(run, kWave - 1);
  uint32_t tau = tk;
  int Lk = L;
  if (top_p < 1.0f) {
    // M = first sorted index whose running mass reaches top_p of the total
    const uint64_t hit = __ballot(in && run / tot >= (double)top_p);
    const int M = hit ? __ffsll((unsigned long long)hit) - 1 : L - 1;
    tau = (uint32_t)__builtin_amdgcn_readlane((int)k32, M);
    const uint64_t below = __ballot(in && k32 < tau);
    Lk = below ? __ffsll((unsigned long long)below) - 1 : L;
  }
  const double keep_sum = wave_sum(lane < Lk ? wgt : 0.0);

  // the kept tokens by id ascending: key (~id << 32 | logit bits), descending
  uint64_t y = 0ull;
  if (lane < Lk) {
    const uint32_t id = 0xffffffffu - (uint32_t)x;
    y = ((uint64_t)(0xffffffffu - id) << 32) | (uint64_t)__float_as_uint(unkey(k32));
  }
  y = wave_sort_desc(y);
  if (lane < Lk) {
    Kept e;
    e.id = (int)(0xffffffffu - (uint32_t)(y >> 32));
    e.z = __uint_as_float((uint32_t)y);
    kept[(size_t)rr * kKeptCap + lane] = e;
  }
  if (lane == 0) {
    out.m = m;
    out.tau = unkey(tau);
    out.S = keep_sum;
    out.count = Lk;
    out.status = 0;
    rows[rr] = out;
  }
}

// The candidate list and the radix histogram share their LDS with the
// general select, which a row runs instead when a chunk had more candidates
// than its slot (massive ties at a chunk's threshold).
constexpr size_t kMergeListBytes = kFiltSortMax * sizeof(uint64_t) + kRadixBins * sizeof(int);
constexpr size_t kMergePoolBytes =
    sizeof(SelectLds) > kMergeListBytes ? sizeof(SelectLds) : kMergeListBytes;
constexpr size_t kMergeGrid = 512;                   // block-merge workgroups at most

// The block merge of row rr (a row its wave marked), by the whole block.
template <typename T>
__device__ __forceinline__ void merge_row(
    int rr, const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    int K, int V, int nch, int cap, int row_stride, int top_k, float top_p, double invT,
    const uint64_t* __restrict__ cand, const int* __restrict__ counts,
    FiltRow* __restrict__ rows, Kept* __restrict__ kept) {
  __shared__ __align__(16) unsigned char pool[kMergePoolBytes];
  __shared__ double tbl[SPECV_EXP64_N];
  __shared__ double dl[kFiltThreads / kWave];
  __shared__ int il[kFiltThreads / kWave];
  __shared__ int s_off[kFiltMaxChunks + 1];
  __shared__ int s_status;
  __shared__ int s_digit, s_need;
  uint64_t* const keys = reinterpret_cast<uint64_t*>(pool);
  int* const hist = reinterpret_cast<int*>(pool + kFiltSortMax * sizeof(uint64_t));
  const int R = 2 * K + 1;
  const int r = rr % R, b = rr / R;
  exp64_stage_table<kFiltThreads>(tbl);
  const int nb = draft_len ? draft_len[b] : 0;      // null: no drafts (sampling)
  if (nb < 0 || nb > K) return;
  bool is_target;
  int k;
  if (!row_needed(r, K, nb, is_target, k)) return;
  if (rows[rr].status != kStatusRedo) return;        // uniform: merged by its wave already

  // the chunks' candidate counts, clipped to their slots, and their offsets
  // in the row's list: one wave, lane c = chunk c (nch <= kFiltMaxChunks)
  if (threadIdx.x < kWave) {
    const int c = threadIdx.x;
    int n = 0, over = 0;
    if (c < nch) {
      const int cnt = counts[(size_t)rr * nch + c];
      const int slot = c == nch - 1 ? row_stride - (nch - 1) * cap : cap;
      over = cnt > slot;
      n = min(cnt, slot);
    }
    const int x = wave_incl_scan_i32(n);             // inclusive scan over the lanes
    if (c < nch) s_off[c + 1] = x;
    const bool any_over = __ballot(over) != 0;
    if (c == 0) {
      s_off[0] = 0;
      s_status = any_over ? 1 : 0;
    }
  }
  __syncthreads();
  if (s_status != 0) {                               // uniform: a chunk overflowed its slot
    const T* row = is_target ? tgt + target_row_off(b, k, K, V) : dft + draft_row_off(b, k, K, V);
    const FiltRow o = select_row<T, kFiltThreads>(row, V, sizeof(T) == 2, top_k, top_p, invT, tbl,
                                                  reinterpret_cast<SelectLds*>(pool),
                                                  kept + (size_t)rr * kKeptCap);
    if (threadIdx.x == 0) rows[rr] = o;
    return;
  }
  const int n_all = s_off[nch];
  // gather: every load of this thread first (flat index f, its chunk found
  // by binary search over the offsets), then the stores to LDS
  constexpr int kGather = kFiltSortMax / kFiltThreads;
  uint64_t gv[kGather];
#pragma unroll
  for (int j = 0; j < kGather; ++j) {
    const int f = (int)threadIdx.x + j * kFiltThreads;
    gv[j] = 0ull;
    if (f < n_all) {
      int lo = 0, hi = nch;                          // s_off[lo] <= f < s_off[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= f) lo = mid;
        else hi = mid;
      }
      gv[j] = cand[(size_t)rr * row_stride + (size_t)lo * cap + (f - s_off[lo])];
    }
  }
#pragma unroll
  for (int j = 0; j < kGather; ++j) {
    const int f = (int)threadIdx.x + j * kFiltThreads;
    if (f < n_all) keys[f] = gv[j];
  }
  __syncthreads();

  // tau_k = the kk-th largest candidate key, kk = min(top_k, n_all) (top_k <
  // V here; ties are kept), by radix select: three passes over 11-, 11- and
  // 10-bit digits, each a histogram in LDS of the keys that match the digits
  // chosen so far, then the bin where the count from the top reaches the
  // remaining rank.  Only the keys >= tau_k (the top-k and its ties) are
  // sorted afterwards; the other candidates never need an order.
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int kk = min(top_k, n_all);
  uint32_t tau_k = 0u;
  if (n_all > 0) {
    constexpr int kPer = kRadixBins / kFiltThreads;
    uint32_t prefix = 0u, pmask = 0u;
    int need = kk;
    for (int i = threadIdx.x; i < kRadixBins; i += kFiltThreads) hist[i] = 0;
    __syncthreads();
    // Three barriers a pass: (A) the histogram is complete; (B) the wave
    // totals of the bin scan are in il, every read of the histogram done,
    // so it is cleared for the next pass; (C) the chosen digit is visible
    // and the histogram clear.  s_digit and il are rewritten only after
    // the next (A), by which time every thread has read them.
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int bits = pass < 2 ? 11 : 10, shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nbins = 1 << bits;
      for (int f = threadIdx.x; f < n_all; f += kFiltThreads) {
        const uint32_t k32 = (uint32_t)(keys[f] >> 32);
        if ((k32 & pmask) == prefix) atomicAdd(&hist[(k32 >> shift) & (uint32_t)(nbins - 1)], 1);
      }
      __syncthreads();                               // (A)
      // thread t takes bins nbins-1-(kPer t + i), i < kPer: digits from the top
      int c[kPer], csum = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int d = nbins - 1 - (kPer * (int)threadIdx.x + i);
        c[i] = d >= 0 ? hist[d] : 0;
        csum += c[i];
      }
      const int incl = wave_incl_scan_i32(csum);
      if (lane == kWave - 1) il[wid] = incl;
      __syncthreads();                               // (B)
      for (int i = threadIdx.x; i < kRadixBins; i += kFiltThreads) hist[i] = 0;
      int above = incl - csum;                       // matching keys in higher bins
#pragma unroll
      for (int w = 0; w < kFiltThreads / kWave; ++w)
        if (w < wid) above += il[w];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (above < need && need <= above + c[i]) {      // exactly one bin of the block
          s_digit = nbins - 1 - (kPer * (int)threadIdx.x + i);
          s_need = need - above;
        }
        above += c[i];
      }
      __syncthreads();                               // (C)
      prefix |= (uint32_t)s_digit << shift;
      pmask |= (uint32_t)(nbins - 1) << shift;
      need = s_need;
    }
    tau_k = prefix;
  }
  // the keys >= tau_k, moved to the front of keys in their current order (L
  // of them; each thread takes a contiguous block of the list, so a key
  // never moves past a slot not yet read) and sorted descending
  const int qa = (n_all + kFiltThreads - 1) / kFiltThreads;
  const int a_lo = min(n_all, (int)threadIdx.x * qa), a_hi = min(n_all, a_lo + qa);
  int mine_n = 0;
  for (int f = a_lo; f < a_hi; ++f) mine_n += (uint32_t)(keys[f] >> 32) >= tau_k ? 1 : 0;
  const int incl_n = wave_incl_scan_i32(mine_n);
  if (lane == kWave - 1) il[wid] = incl_n;           // il's last readers passed (C)
  uint64_t kept_keys[kGather];
  int nk = 0;
#pragma unroll
  for (int j = 0; j < kGather; ++j) {
    const int f = a_lo + j;
    kept_keys[j] = f < a_hi ? keys[f] : 0ull;
  }
  __syncthreads();                                   // every read of the list is done
  int L = 0, pos = incl_n - mine_n;
#pragma unroll
  for (int w = 0; w < kFiltThreads / kWave; ++w) {
    if (w < wid) pos += il[w];
    L += il[w];
  }
#pragma unroll
  for (int j = 0; j < kGather; ++j) {
    if (a_lo + j < a_hi && (uint32_t)(kept_keys[j] >> 32) >= tau_k) keys[pos + nk++] = kept_keys[j];
  }
  if (L <= kWave) {
    // the usual case (top-k and a few ties): one wave sorts in registers
    __syncthreads();
    if (wid == 0) {
      uint64_t x = lane < L ? keys[lane] : 0ull;     // 0 sorts last
      x = wave_sort_desc(x);
      if (lane < L) keys[lane] = x;
    }
    __syncthreads();
  } else {
    int P = 2;
    while (P < L) P <<= 1;
    for (int i = L + (int)threadIdx.x; i < P; i += kFiltThreads) keys[i] = 0ull;   // sorts last
    lds_bitonic_desc(keys, P);
  }

  FiltRow out;
  out.status = s_status;
  if (n_all == 0) out.status = 2;                    // no finite logit in the row
  const float m = n_all > 0 ? unkey((uint32_t)(keys[0] >> 32)) : -INFINITY;
  const double md = (double)m;

  int Lk = L;                                        // kept prefix length
  uint32_t tau = tau_k;
  double keep_sum = 0.0;
  if (L <= kWave) {
    // The usual case: the whole sorted prefix is one wave, lane i holding
    // entry i; the running sums are one inclusive scan in lane order, the
    // crossing and the first entry below tau are ballots.  Every thread
    // keeps Lk = L <= 64 so all take the same branch below; wave 0 refines it.
    if (wid == 0) {
      const bool in = lane < L;
      const uint32_t k32 = in ? (uint32_t)(keys[lane] >> 32) : 0u;
      const double wgt = in ? exp64(((double)unkey(k32) - md) * invT, tbl) : 0.0;
      const double run = wave_incl_scan(wgt);
      const double tot = lane_value(run, kWave - 1);
      if (top_p < 1.0f && L > 0) {
        // M = first sorted index whose running mass reaches top_p of the total
        const uint64_t hit = __ballot(in && run / tot >= (double)top_p);
        const int M = hit ? __ffsll((unsigned long long)hit) - 1 : L - 1;
        tau = (uint32_t)lane_value((int)k32, M);
        const uint64_t below = __ballot(in && k32 < tau);
        Lk = below ? __ffsll((unsigned long long)below) - 1 : L;
      }
      keep_sum = wave_sum(lane < Lk ? wgt : 0.0);   // normaliser over the kept prefix
    }
  } else {
  // float64 weights of the sorted prefix, blocked scan in sorted order
  const int q = (L + kFiltThreads - 1) / kFiltThreads;
  const int i_lo = min(L, (int)threadIdx.x * q), i_hi = min(L, i_lo + q);
  double mine = 0.0;
  for (int i = i_lo; i < i_hi; ++i)
    mine += exp64(((double)unkey((uint32_t)(keys[i] >> 32)) - md) * invT, tbl);
  double tot;
  const double excl = block_scan_excl<double>(mine, dl, tot);
  if (top_p < 1.0f && L > 0) {
    // M = first sorted index whose running mass reaches top_p of the total
    int hit = INT_MAX;
    double run = excl;
    for (int i = i_lo; i < i_hi; ++i) {
      run += exp64(((double)unkey((uint32_t)(keys[i] >> 32)) - md) * invT, tbl);
      if (hit == INT_MAX && run / tot >= (double)top_p) hit = i;
    }
    int M = block_min_i(hit, il);
    if (M == INT_MAX) M = L - 1;
    tau = (uint32_t)(keys[M] >> 32);
    int first_below = INT_MAX;
    for (int i = threadIdx.x; i < L; i += kFiltThreads)
      if ((uint32_t)(keys[i] >> 32) < tau) first_below = min(first_below, i);
    Lk = block_min_i(first_below, il);
    if (Lk == INT_MAX) Lk = L;
  }
  // normaliser over the kept prefix, same blocked order
  {
    const int j_lo = min(Lk, (int)threadIdx.x * q), j_hi = min(Lk, j_lo + q);
    for (int i = j_lo; i < j_hi; ++i)
      keep_sum += exp64(((double)unkey((uint32_t)(keys[i] >> 32)) - md) * invT, tbl);
    double stot;
    (void)block_scan_excl<double>(keep_sum, dl, stot);
    keep_sum = stot;
  }
  }
  // a kept set above kKeptCap gets no list: its samplers stream the row

  // kept tokens re-sorted by id ascending: key (~id << 32 | logit bits), descending
  auto id_key = [&](uint64_t e) -> uint64_t {
    const uint32_t id = 0xffffffffu - (uint32_t)e;
    return ((uint64_t)(0xffffffffu - id) << 32) | (uint64_t)__float_as_uint(unkey((uint32_t)(e >> 32)));
  };
  if (Lk <= kWave) {
    // one wave in registers, straight to the kept list
    if (wid == 0) {
      uint64_t x = lane < Lk ? id_key(keys[lane]) : 0ull;
      x = wave_sort_desc(x);
      if (lane < Lk) {
        Kept e;
        e.id = (int)(0xffffffffu - (uint32_t)(x >> 32));
        e.z = __uint_as_float((uint32_t)x);
        kept[(size_t)rr * kKeptCap + lane] = e;
      }
    }
  } else if (Lk <= kKeptCap) {
    __syncthreads();
    int P2 = 2;
    while (P2 < Lk) P2 <<= 1;
    for (int i = threadIdx.x; i < P2; i += kFiltThreads) {
      keys[kFiltSortMax / 2 + i] = i < Lk ? id_key(keys[i]) : 0ull;
    }
    lds_bitonic_desc(keys + kFiltSortMax / 2, P2);
    Kept* dst = kept + (size_t)rr * kKeptCap;
    for (int i = threadIdx.x; i < Lk; i += kFiltThreads) {
      const uint64_t x = keys[kFiltSortMax / 2 + i];
      Kept e;
      e.id = (int)(0xffffffffu - (uint32_t)(x >> 32));
      e.z = __uint_as_float((uint32_t)x);
      dst[i] = e;
    }
  }
  if (threadIdx.x == 0) {
    out.m = m;
    out.tau = unkey(tau);
    out.S = keep_sum;
    out.count = Lk;
    out.pad = 0;
    rows[rr] = out;
  }
}

// The block merge over the rows the wave merge listed, a grid-stride loop
// so the grid needs no row count from the host: with the usual empty list
// every workgroup leaves after one load.
template <typename T>
__global__ __launch_bounds__(kFiltThreads) void filter_merge_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    int K, int V, int nch, int cap, int row_stride, int top_k, float top_p, double invT,
    const uint64_t* __restrict__ cand, const int* __restrict__ counts,
    FiltRow* __restrict__ rows, Kept* __restrict__ kept, const int* __restrict__ redo_count,
    const int* __restrict__ redo_rows) {
  const int n = *redo_count;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {  // uniform per block
    merge_row<T>(redo_rows[i], tgt, dft, draft_len, K, V, nch, cap, row_stride, top_k, top_p,
                 invT, cand, counts, rows, kept);
    __syncthreads();                                 // the next row reuses the LDS
  }
}

// ---------------------------------------------------------------------------
int filter_cap(int top_k) { return ((3 * top_k) / 2 + 40 + 7) / 8 * 8; }

// Candidate slots of one row: cap per chunk, at least 256 for the last one
// (it keeps every valid token when it has 256 or fewer).
int filter_row_stride(int nch, int top_k) {
  const int cap = filter_cap(top_k);
  return (nch - 1) * cap + (cap > 256 ? cap : 256);
}

hipError_t launch_filter(bool bf16, const void* tgt, const void* dft, const int* draft_len, int B,
                         int K, int V, int nch, int top_k, float top_p, double invT,
                         uint64_t* cand, int* counts, FiltRow* rows, Kept* kept, int* redo,
                         hipStream_t stream, hipEvent_t mid) {
  const int cap = filter_cap(top_k);
  const int stride = filter_row_stride(nch, top_k);
  const size_t blocks = (size_t)B * (2 * K + 1) * nch;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (bf16)
    filter_cand_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kFiltThreads), 0, stream>>>(
        static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), draft_len, K, V, nch,
        top_k, cap, stride, cand, counts, redo);
  else
    filter_cand_kernel<float><<<dim3((unsigned)blocks), dim3(kFiltThreads), 0, stream>>>(
        static_cast<const float*>(tgt), static_cast<const float*>(dft), draft_len, K, V, nch,
        top_k, cap, stride, cand, counts, redo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, stream)) != hipSuccess) return e;
  const size_t nrows = (size_t)B * (2 * K + 1);
  filter_merge_wave_kernel<<<dim3((unsigned)((nrows + kMergeWaves - 1) / kMergeWaves)),
                             dim3(kFiltThreads), 0, stream>>>(
      draft_len, B, K, nch, cap, stride, top_k, top_p, invT, cand, counts, rows, kept, redo,
      redo + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // as many workgroups as fit at once (two per CU at the merge's register
  // count), or one per row if fewer
  const dim3 grid((unsigned)std::min<size_t>(nrows, kMergeGrid));
  if (bf16)
    filter_merge_kernel<bf16_t><<<grid, dim3(kFiltThreads), 0, stream>>>(
        static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), draft_len, K, V, nch,
        cap, stride, top_k, top_p, invT, cand, counts, rows, kept, redo, redo + 1);
  else
    filter_merge_kernel<float><<<grid, dim3(kFiltThreads), 0, stream>>>(
        static_cast<const float*>(tgt), static_cast<const float*>(dft), draft_len, K, V, nch, cap,
        stride, top_k, top_p, invT, cand, counts, rows, kept, redo, redo + 1);
  return hipGetLastError();
}

}  // namespace specv
