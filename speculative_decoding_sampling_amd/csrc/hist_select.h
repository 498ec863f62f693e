// Top-k / top-p threshold of one bfloat16 row from one read of the row: a
// count histogram over all 65536 16-bit logit keys.
//
// The cuts are those of radix_select.h (nickwang.xyz "推测解码：草稿、验证与
// 实际加速", section "接受与拒绝怎样保住分布": p and q are both taken after
// temperature, top-k and top-p): the kept set is {z >= tau}, with
//   tau_k = the largest value v with #{z >= v} >= k,
//   tau_p = the largest value v >= tau_k with M(v) >= top_p * M(tau_k),
//   M(v)  = sum over z >= v of exp((z - m) / T).
//
// A bfloat16 logit has one of 65536 bit patterns, and its weight depends on
// nothing else, so a key's share of every count and mass is its count times
// the share of one logit.  One pass over the row counts the keys (two 16-bit
// counters per LDS word, 128 KB); a census then marks the populated keys of
// each 64-key range and counts those below it, and each cut is found from
// there: thread t sums one weight per key over its slice of the populated
// keys from the largest down (reached by a binary search over the ranges), a
// block scan finds the slice that holds the cut, and its thread walks it.  Masses are the same 2^-64 fixed-point sums as
// radix_select.h's (count times the same two parts of the same float64
// weight), so the cut, the count and the kept normaliser are bit-identical to
// that select's.  Keys whose weight is below 2^-64 (more than 45 T below the
// maximum) add nothing there and are skipped here.
//
// The row falls back to radix_select.h when a counter could have wrapped (a
// key held by 65536 or more logits: the decoded total then falls short of V),
// or when the row holds a NaN or +inf.
#pragma once

#include "radix_select.h"

namespace specv {

constexpr int kHistWords = 32768;                 // 65536 keys, two per word
constexpr int kBitmapBits = kHistWords * 32;      // kept-id bitmap over a row, in its place
constexpr uint32_t kKey16Lo = 0x0080u;            // smallest finite key (-max)
constexpr uint32_t kKey16Hi = 0xff7fu;            // largest finite key (+max)
constexpr uint32_t kKey16NegInf = 0x007fu;

constexpr int kRanges = 1024;                     // 64-key ranges of the key space

struct HistAux {
  unsigned long long pmask[kRanges];              // populated finite keys of each range
  uint32_t roff[kRanges + 1];                     // populated finite keys below each range
  uint32_t wc[kSelMaxWaves];                      // wave totals of the scans
  unsigned long long wh[kSelMaxWaves], wl[kSelMaxWaves];
  uint32_t wt[kSelMaxWaves], wm[kSelMaxWaves], wb[kSelMaxWaves];
  uint32_t key, ge_c;                             // the cut key, totals of the keys >= it
  unsigned long long ge_h, ge_l;
};

union HistPool {
  uint32_t w[kHistWords];                         // the histogram, then the kept-id bitmap
  SelectLds sel;                                  // or the fallback select
};

// 32-bit key (as fkey) of the bfloat16 logit with 16-bit key k: the low half
// is 0 for a positive logit and all ones for a negative one.
__device__ __forceinline__ uint32_t key32_of(uint32_t k) {
  return (k << 16) | ((k & 0x8000u) ? 0u : 0xffffu);
}

// 16-bit keys of the two bfloat16 logits of word u, as one word: the pattern
// with the sign bit flipped (positive) or every bit flipped (negative).  -0
// gets key 0x7fff, next to +0's 0x8000.
typedef short short2_v __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t key_pair(uint32_t u) {
  const short2_v sgn = __builtin_bit_cast(short2_v, u) >> (short)15;   // 0 or -1 per half
  return u ^ (__builtin_bit_cast(uint32_t, sgn) | 0x80008000u);
}

// Count both logits of word u: key k lives in half k & 1 of word k >> 1.
__device__ __forceinline__ void hist_add_pair(uint32_t* hw, uint32_t u) {
  const uint32_t k = key_pair(u);
  atomicAdd(&hw[(k & 0xffffu) >> 1], (k & 1u) * 0xffffu + 1u);
  atomicAdd(&hw[k >> 17], ((k >> 16) & 1u) * 0xffffu + 1u);
}
__device__ __forceinline__ void hist_add_one(uint32_t* hw, uint32_t h) {
  const uint32_t k = key_pair(h) & 0xffffu;
  atomicAdd(&hw[k >> 1], (k & 1u) * 0xffffu + 1u);
}

// c logits of key k: their two-part fixed-point mass (radix_select.h's
// weight and parts, times c).
__device__ __forceinline__ void key_mass(uint32_t k, uint32_t c, float m, double invT,
                                         const double* tbl, unsigned long long& h,
                                         unsigned long long& l) {
  h = l = 0ull;
  const double x = ((double)unkey(key32_of(k)) - (double)m) * invT;
  if (x < -45.0) return;                          // weight < 2^-64: both parts 0
  unsigned long long ph, pl;
  fixed_parts(exp64(x, tbl), ph, pl);
  h = ph * c;
  l = pl * c;
}


// Position of the k-th (from 0) set bit of m, counting from bit 0.
__device__ __forceinline__ uint32_t select_bit(unsigned long long m, uint32_t k) {
  uint32_t pos = 0u, c = (uint32_t)__popc((uint32_t)m);
  if (k >= c) {
    k -= c;
    m >>= 32;
    pos = 32u;
  }
  uint32_t x = (uint32_t)m;
#pragma unroll
  for (uint32_t w = 16u; w >= 1u; w >>= 1) {
    c = (uint32_t)__popc(x & ((1u << w) - 1u));
    if (k >= c) {
      k -= c;
      x >>= w;
      pos += w;
    }
  }
  return pos;
}

// The range holding the populated finite key of ascending index s: the last
// range r with roff[r] <= s (a non-empty one, as roff[r + 1] > s).
__device__ __forceinline__ int range_of(const HistAux* a, int s) {
  int lo = 0, hi = kRanges;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int mid = (lo + hi) >> 1;
    if ((int)a->roff[mid] <= s) lo = mid; else hi = mid;
  }
  return lo;
}

// The populated finite keys of ascending index s, s - 1, ... (at most nk of
// them), largest first, each given to f(key) until it returns false.
template <typename F>
__device__ __forceinline__ void walk_down(const HistAux* a, int s, int nk, F&& f) {
  int r = range_of(a, s);
  unsigned long long msk = a->pmask[r];
  const uint32_t pos = select_bit(msk, (uint32_t)(s - (int)a->roff[r]));
  msk &= pos == 63u ? ~0ull : ((2ull << pos) - 1ull);
  for (int j = 0; j < nk; ++j, --s) {
    if (msk == 0ull) {                            // the next lower non-empty range
      r = range_of(a, s);
      msk = a->pmask[r];
      if (msk == 0ull) break;                     // unreachable for 0 <= s < n
    }
    const uint32_t b = 63u - (uint32_t)__clzll((long long)msk);
    msk &= ~(1ull << b);
    if (!f(64u * (uint32_t)r + b)) break;
  }
}

// Count of key k in the histogram.
__device__ __forceinline__ uint32_t key_count(const uint32_t* hw, uint32_t k) {
  const uint32_t w = hw[k >> 1];
  return (k & 1u) ? (w >> 16) : (w & 0xffffu);
}

// The cut among the top ntop populated finite keys (those >= the floor): the
// largest key whose cumulative total from the top reaches the target --
// count >= k (count mode) or mass / W >= top_p, W the total mass of those
// keys -- left in a->key and a->ge_* (with find false, only the totals, in
// a->ge_*).  Thread t sums the keys of descending rank t q .. t q + q - 1
// (q = ceil(ntop / NT)); a block scan finds the thread whose keys hold the
// cut, and that thread walks them again.
template <int NT>
__device__ __forceinline__ void hist_cut(const uint32_t* hw, int n, int ntop, bool mass_mode,
                                         bool find, uint32_t k, float top_p, float m, double invT,
                                         const double* tbl, HistAux* a) {
  const int t = threadIdx.x;
  const int q = (ntop + NT - 1) / NT;
  const int r0 = t * q, nk = min(ntop, r0 + q) - r0;   // descending ranks [r0, r0 + nk)
  uint32_t c = 0u;
  unsigned long long h = 0ull, l = 0ull;
  if (nk > 0) {
    walk_down(a, n - 1 - r0, nk, [&](uint32_t key) {
      const uint32_t kc = key_count(hw, key);
      c += kc;
      if (mass_mode) {
        unsigned long long eh, el;
        key_mass(key, kc, m, invT, tbl, eh, el);
        h += eh;
        l += el;
      }
      return true;
    });
  }
  uint32_t ec, tc;
  unsigned long long eh, el, th, tl;
  block_scan3<NT>(c, h, l, a, ec, eh, el, tc, th, tl);
  if (!find) {
    if (t == 0) {
      a->ge_c = tc;
      a->ge_h = th;
      a->ge_l = tl;
    }
    __syncthreads();
    return;
  }
  const double W = fixed_to_double(th, tl);
  auto reach = [&](uint32_t rc, unsigned long long rh, unsigned long long rl) -> bool {
    return mass_mode ? fixed_to_double(rh, rl) / W >= (double)top_p : rc >= k;
  };
  if (nk > 0 && !reach(ec, eh, el) && reach(ec + c, eh + h, el + l)) {   // exactly one thread
    walk_down(a, n - 1 - r0, nk, [&](uint32_t key) {
      const uint32_t kc = key_count(hw, key);
      ec += kc;
      if (mass_mode) {
        unsigned long long xh, xl;
        key_mass(key, kc, m, invT, tbl, xh, xl);
        eh += xh;
        el += xl;
      }
      if (!reach(ec, eh, el)) return true;
      a->key = key;
      a->ge_c = ec;
      a->ge_h = eh;
      a->ge_l = el;
      return false;
    });
  }
  __syncthreads();
}

// The select for one bfloat16 row by a block of NT = 1024 threads (the
// first pass holds up to 16 vectors of 8 logits per thread in flight).
// Writes the kept list (sorted by id) when the kept set has at most kKeptCap
// tokens; returns the row's FiltRow.  tbl must be staged and visible.
template <int NT>
__device__ __forceinline__ FiltRow select_row_hist(const bf16_t* __restrict__ row, int V, int top_k, float top_p,
                                   double invT, const double* tbl, HistPool* pool, HistAux* a,
                                   Kept* __restrict__ kept) {
  static_assert(NT == 1024 && kHistWords / NT == 32, "block size");
  constexpr int U = 16;
  const int t = threadIdx.x, lane = t % kWave, wid = t / kWave;
  uint32_t* hw = pool->w;

  // 1. count every logit.  Vector j = logits 8 j .. 8 j + 7; an index past
  // the row is clamped to its last vector (loaded, never counted), so every
  // load is unconditional.  The first U vectors per thread are requested
  // before the histogram is cleared.
  const int nvec = aligned16(row) ? V / 8 : 0;
  uint4 v[U];
  if (nvec > 0) {                                 // uniform
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = *reinterpret_cast<const uint4*>(row + 8 * min(u * NT + t, nvec - 1));
  }
  for (int i = t; i < kHistWords / 4; i += NT)
    reinterpret_cast<uint4*>(hw)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  if (nvec > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u * NT + t < nvec) {
        hist_add_pair(hw, v[u].x);
        hist_add_pair(hw, v[u].y);
        hist_add_pair(hw, v[u].z);
        hist_add_pair(hw, v[u].w);
      }
    }
  }
  // rows longer than U NT vectors: the rest, four vectors in flight
  for (int j0 = U * NT; j0 < nvec; j0 += 4 * NT) {
    uint4 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = *reinterpret_cast<const uint4*>(row + 8 * (long)min(j0 + q * NT + t, nvec - 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (j0 + q * NT + t < nvec) {
        hist_add_pair(hw, w[q].x);
        hist_add_pair(hw, w[q].y);
        hist_add_pair(hw, w[q].z);
        hist_add_pair(hw, w[q].w);
      }
    }
  }
  for (int e = nvec * 8 + t; e < V; e += NT) hist_add_one(hw, row[e]);
  __syncthreads();
  if (t == 0) {                                   // -0 (key 0x7fff) counts as +0 (0x8000)
    const uint32_t nz = hw[0x3fff] >> 16;
    hw[0x3fff] &= 0xffffu;
    hw[0x4000] += nz;
  }
  __syncthreads();

  // 2. census of range t (keys [64 t, 64 t + 64), words [32 t, 32 t + 32)):
  // every counter decoded (a wrapped one leaves the total short of V), the
  // populated finite keys as a 64-bit mask, any NaN or +inf.  Quad k holds
  // words 4 ((k + t) mod 8) .. + 3, so that eight neighbouring lanes read
  // different banks.
  uint32_t tot = 0u, bad = 0u;
  unsigned long long pm = 0ull;                   // bit b: key 64 t + b populated (finite only)
  {
    uint4 qd[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) qd[k] = reinterpret_cast<const uint4*>(hw)[t * 8 + ((k + t) & 7)];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ws[4] = {qd[k].x, qd[k].y, qd[k].z, qd[k].w};
      if ((ws[0] | ws[1] | ws[2] | ws[3]) == 0u) continue;
      uint32_t byte = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tot = __builtin_amdgcn_sad_u16(ws[i], 0u, tot);
        // per half: 1 if the counter is non-zero
        const uint32_t nz = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(
            __builtin_bit_cast(ushort2_v, ws[i]), ushort2_v{1, 1}));
        byte |= ((nz & 1u) | (nz >> 15)) << (2 * i);
      }
      pm |= (unsigned long long)byte << (8 * ((k + t) & 7));
    }
    // ranges 0, 1, 1022, 1023 hold the non-finite keys: -inf (0x7f, the top
    // key of range 1) is allowed and not counted as finite, the rest is NaN or +inf
    if (t <= 1 || t >= kRanges - 2) {
      const unsigned long long nonfin = t == 1 ? (pm & ~(1ull << 63)) : pm;
      bad = nonfin != 0ull;
      pm = 0ull;
    }
  }
  const uint32_t np = (uint32_t)__popcll(pm);
  uint32_t mkey = pm ? 64u * t + 63u - (uint32_t)__clzll((long long)pm) : 0u;
  // block totals, and np's exclusive prefix (range order = ascending keys)
  const uint32_t nincl = wave_incl_scan_u32(np);
  tot = wave_sum_u32(tot);
  bad = wave_or_u32(bad);
  mkey = wave_max_u32(mkey);
  if (lane == kWave - 1) {
    a->wt[wid] = tot;
    a->wb[wid] = bad;
    a->wm[wid] = mkey;
    a->wc[wid] = nincl;
  }
  __syncthreads();
  uint32_t noff = nincl - np, ntot = 0u;
  tot = bad = mkey = 0u;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    tot += a->wt[w];
    bad |= a->wb[w];
    mkey = max(mkey, a->wm[w]);
    if (w < wid) noff += a->wc[w];
    ntot += a->wc[w];
  }
  a->pmask[t] = pm;
  a->roff[t] = noff;
  if (t == NT - 1) a->roff[kRanges] = ntot;
  if (bad || tot != (uint32_t)V) {                // uniform: the general select
    __syncthreads();                              // every thread is done with the histogram
    return select_row<bf16_t, NT>(row, V, true, top_k, top_p, invT, tbl, &pool->sel, kept);
  }
  FiltRow out;
  out.pad = 0;
  // finite logits: all but the -inf ones (NaN and +inf sent the row away)
  const uint32_t fin = (uint32_t)V - (hw[kKey16NegInf >> 1] >> 16);
  if (fin == 0u) {
    out.m = -INFINITY;
    out.tau = INFINITY;
    out.S = 0.0;
    out.count = 0;
    out.status = 2;                               // no finite logit
    return out;
  }
  const float m = unkey(key32_of(mkey));
  __syncthreads();                                // the masks and offsets are visible

  // 3. the cuts: top-k on counts, then top-p (or the kept mass) on the masses
  // of the keys >= the top-k cut
  const int n = (int)ntot;
  const bool topk_on = top_k > 0 && (uint32_t)top_k < fin;
  const bool topp_on = top_p < 1.0f;
  uint32_t floor16 = kKey16Lo;
  int ntop = n;
  uint32_t cnt = fin;
  if (topk_on) {
    hist_cut<NT>(hw, n, n, false, true, (uint32_t)top_k, 1.0f, m, invT, tbl, a);
    floor16 = a->key;
    cnt = a->ge_c;
    const int rf = (int)(floor16 >> 6);           // the floor key's ascending index
    const int sf = (int)a->roff[rf] + __popcll(a->pmask[rf] & ((1ull << (floor16 & 63u)) - 1ull));
    ntop = n - sf;
  }
  hist_cut<NT>(hw, n, ntop, true, topp_on, 0u, top_p, m, invT, tbl, a);
  uint32_t tau16 = floor16;
  if (topp_on) {
    tau16 = a->key;
    cnt = a->ge_c;
  }
  const unsigned long long mh = a->ge_h, ml = a->ge_l;
  // no cut at all keeps every finite key: the threshold is the one past -inf
  const uint32_t tau = (topk_on || topp_on) ? key32_of(tau16) : kNegInfKey + 1u;

  // 5. the kept list when it fits, in id order: the kept ids are marked in a
  // bitmap over the row (in place of the list; one more read of the row, all
  // of a thread's vectors in flight), then thread t emits the ids of bitmap words
  // [t pw, t pw + pw) from its exclusive prefix on, reading each kept logit
  // back.  -0 was counted as +0, so a cut at +0 keeps it.
  if (cnt <= (uint32_t)kKeptCap) {
    if (V > kBitmapBits) {                        // uniform: the bitmap does not fit
      __syncthreads();
      return select_row<bf16_t, NT>(row, V, true, top_k, top_p, invT, tbl, &pool->sel, kept);
    }
    const uint32_t tl16 = tau16 == 0x8000u ? 0x7fffu : tau16;
    uint32_t* bm = pool->w;
    const int nw = (V + 31) / 32;
    for (int i = t; i < nw; i += NT) bm[i] = 0u;
    __syncthreads();
    auto mark_word = [&](uint32_t u, int id0) {   // the two logits of word u, ids id0, id0 + 1
      const uint32_t kk = key_pair(u);
      if ((kk & 0xffffu) >= tl16) atomicOr(&bm[id0 >> 5], 1u << (id0 & 31));
      if ((kk >> 16) >= tl16) atomicOr(&bm[(id0 + 1) >> 5], 1u << ((id0 + 1) & 31));
    };
    auto mark_vec = [&](const uint4& w4, int j) {
      mark_word(w4.x, 8 * j);
      mark_word(w4.y, 8 * j + 2);
      mark_word(w4.z, 8 * j + 4);
      mark_word(w4.w, 8 * j + 6);
    };
    if (nvec > 0) {                               // the first pass's vectors, read again
      uint4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        r[u] = *reinterpret_cast<const uint4*>(row + 8 * min(u * NT + t, nvec - 1));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u * NT + t < nvec) mark_vec(r[u], u * NT + t);
    }
    for (int j0 = U * NT; j0 < nvec; j0 += NT)
      if (j0 + t < nvec) mark_vec(*reinterpret_cast<const uint4*>(row + 8 * (long)(j0 + t)), j0 + t);
    for (int e = nvec * 8 + t; e < V; e += NT)
      if ((key_pair(row[e]) & 0xffffu) >= tl16) atomicOr(&bm[e >> 5], 1u << (e & 31));
    __syncthreads();
    const int pw = (nw + NT - 1) / NT;
    const int w_lo = min(nw, t * pw), w_hi = min(nw, w_lo + pw);
    uint32_t mine = 0u;
    for (int i = w_lo; i < w_hi; ++i) mine += __popc(bm[i]);
    const uint32_t incl = wave_incl_scan_u32(mine);
    if (lane == kWave - 1) a->wc[wid] = incl;     // a's last readers passed the barriers above
    __syncthreads();
    uint32_t pos = incl - mine;
    for (int w = 0; w < wid; ++w) pos += a->wc[w];
    if (mine) {
      for (int i = w_lo; i < w_hi; ++i) {
        uint32_t bits = bm[i];
        while (bits) {
          const int id = 32 * i + __builtin_ctz(bits);
          bits &= bits - 1u;
          if (pos >= (uint32_t)kKeptCap) break;   // unreachable: the map holds cnt logits
          const uint32_t h = row[id];
          Kept e;
          e.id = id;
          e.z = __uint_as_float(h == 0x8000u ? 0u : h << 16);   // -0 stored as +0
          kept[pos++] = e;
        }
      }
    }
  }
  out.m = m;
  out.tau = unkey(tau);
  out.S = fixed_to_double(mh, ml);
  out.count = (int)cnt;
  out.status = 0;
  return out;
}

}  // namespace specv
