// Top-k / top-p threshold of one row for any k and any kept-set size, by one
// workgroup: a radix select over the logits' order-preserving keys.
//
// p and q are the distributions after temperature, top-k and top-p, each row
// filtered on its own (nickwang.xyz "推测解码：草稿、验证与实际加速", section
// "接受与拒绝怎样保住分布": both include those settings).  top-k keeps every
// logit >= the k-th largest; top-p then keeps the shortest prefix of the
// renormalised top-k distribution, by logit descending, whose mass reaches
// top_p, with the crossing token and its ties.  Both cuts are thresholds on
// the logit, so the kept set is {z >= tau}:
//   tau_k = the largest value v with #{z >= v} >= k,
//   tau_p = the largest value v >= tau_k with M(v) >= top_p * M(tau_k),
//   M(v)  = sum over z >= v of exp((z - m) / T)   (m the row maximum).
//
// The select walks down the 32-bit key in three digits (11, 11 and 10 bits;
// bfloat16 logits are resolved after two, their low bits being fixed).  Each
// digit is one pass over the row that histograms the keys sharing the digits
// chosen so far, then the digit where the count (top-k) or the mass (top-p)
// accumulated from the largest key reaches its target is kept.  Masses are
// float64 weights accumulated exactly in 2^-64 fixed point (two 64-bit LDS
// sums per digit, integer atomics), so the histograms, the cut and the kept
// normaliser are the same on every run and carry no rounding beyond the
// weights themselves: the top-p decision matches a float64 evaluation
// except within a few 1e-16 of top_p.  The row is read from memory once per
// digit; no candidate list is kept, so any k and any kept-set size work.
// When the kept set has at most kKeptCap tokens one more pass lists them,
// sorted by id, for the list sampler.
#pragma once

#include "common.h"
#include "exp64.h"
#include "wave_scan.h"

namespace specv {

constexpr int kSelDigits = 2048;          // 11-bit digits; the last float32 digit uses 10 bits
constexpr int kSelMaxWaves = 16;          // workgroups of up to 1024 threads

struct SelectLds {
  uint32_t cnt[kSelDigits];               // keys per digit
  unsigned long long hi[kSelDigits];      // sum of floor(w 2^24) per digit
  unsigned long long lo[kSelDigits];      // sum of floor(frac(w 2^24) 2^40) per digit
  uint32_t wc[kSelMaxWaves];              // wave totals of the digit scan
  unsigned long long wh[kSelMaxWaves], wl[kSelMaxWaves];
  float wmax[kSelMaxWaves];
  uint32_t wn[kSelMaxWaves];
  int digit;                              // the chosen digit of the last search
  uint32_t above_c;                       // ... and the totals of the digits above it
  unsigned long long above_h, above_l;
  unsigned long long kept_h, kept_l;      // kept-set mass of the listing pass
  int nlist;
};

// A mass in 2^-64 units, h 2^40 + l, rounded once to the nearest double.
// With h <= V 2^24 and l <= V 2^40 (V <= 2^22), it is (h + l_hi) 2^40 + l_lo
// with l = l_hi 2^40 + l_lo: both terms are exact doubles (h + l_hi < 2^53,
// l_lo < 2^40), and one fma adds them with a single rounding -- the correctly
// rounded value of the exact sum, as a 128-bit conversion would give.
__device__ __forceinline__ double fixed_to_double(unsigned long long h, unsigned long long l) {
  const unsigned long long H = h + (l >> 40), L = l & ((1ull << 40) - 1ull);
  return fma((double)H, 0x1p40, (double)L) * 0x1p-64;
}
// w in (0, 1] split exactly into floor(w 2^24) and floor(frac(w 2^24) 2^40).
__device__ __forceinline__ void fixed_parts(double w, unsigned long long& h, unsigned long long& l) {
  const double x = w * 0x1p24;
  const double f = floor(x);
  h = (unsigned long long)f;
  l = (unsigned long long)((x - f) * 0x1p40);
}

// Every logit of the row once, as f(z, id): thread t takes 16-byte vectors
// t, t + NT, ... (four in flight), then the unaligned rest element by element.
template <typename T, int NT, typename F>
__device__ __forceinline__ void for_each_logit(const T* __restrict__ row, int V, F&& f) {
  constexpr int N = Elem<T>::kPerVec;
  constexpr int U = 4;
  const long nvec = aligned16(row) ? (long)V / N : 0;
  long j = threadIdx.x;
  for (; j + (long)(U - 1) * NT < nvec; j += (long)U * NT) {
    float z[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) load_vec_fast(row, (j + (long)u * NT) * N, z[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < N; ++i) f(z[u][i], (int)((j + (long)u * NT) * N + i));
  }
  for (; j < nvec; j += NT) {
    float z[N];
    load_vec_fast(row, j * N, z);
#pragma unroll
    for (int i = 0; i < N; ++i) f(z[i], (int)(j * N + i));
  }
  for (long e = nvec * N + threadIdx.x; e < V; e += NT) f(to_f32(row[e]), (int)e);
}

// Exclusive scan over the block's threads (thread order) of a count and a
// two-part mass; also returns the block totals.  S holds the wave totals
// (wc, wh, wl; one entry per wave).
template <int NT, typename S>
__device__ __forceinline__ void block_scan3(uint32_t c, unsigned long long h, unsigned long long l,
                                            S* s, uint32_t& ec, unsigned long long& eh,
                                            unsigned long long& el, uint32_t& tc,
                                            unsigned long long& th, unsigned long long& tl) {
  constexpr int W = NT / kWave;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const uint32_t xc = wave_incl_scan_u32(c);
  const unsigned long long xh = wave_incl_scan_u64(h), xl = wave_incl_scan_u64(l);
  if (lane == kWave - 1) {
    s->wc[wid] = xc;
    s->wh[wid] = xh;
    s->wl[wid] = xl;
  }
  __syncthreads();
  ec = xc - c;
  eh = xh - h;
  el = xl - l;
  tc = 0;
  th = tl = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    if (w < wid) {
      ec += s->wc[w];
      eh += s->wh[w];
      el += s->wl[w];
    }
    tc += s->wc[w];
    th += s->wh[w];
    tl += s->wl[w];
  }
}

// Level `lv` of the key walk: bits [shift, shift + bits) of the key, among
// keys whose higher bits equal `prefix`'s.
__device__ __forceinline__ int sel_shift(int lv) { return lv == 0 ? 21 : (lv == 1 ? 10 : 0); }
__device__ __forceinline__ int sel_bits(int lv) { return lv == 2 ? 10 : 11; }
__device__ __forceinline__ uint32_t sel_himask(int lv) {
  return lv == 0 ? 0u : (0xffffffffu << (sel_shift(lv) + sel_bits(lv)));
}

template <typename T, int NT>
struct RowSelect {
  const T* row;
  int V;
  float m;             // row maximum
  double invT;
  const double* tbl;   // exp64 table in LDS
  SelectLds* s;

  __device__ __forceinline__ double weight(float z) const {
    return exp64(((double)z - (double)m) * invT, tbl);
  }

  // One histogram pass: finite keys >= floor_key whose bits above the level's
  // digit equal prefix's, by digit; masses only when `mass`.
  __device__ void level_pass(int lv, uint32_t prefix, uint32_t floor_key, bool mass) {
    for (int d = threadIdx.x; d < kSelDigits; d += NT) {
      s->cnt[d] = 0u;
      s->hi[d] = s->lo[d] = 0ull;
    }
    __syncthreads();
    const int shift = sel_shift(lv);
    const uint32_t dmask = (1u << sel_bits(lv)) - 1u, hm = sel_himask(lv), want = prefix & hm;
    for_each_logit<T, NT>(row, V, [&](float z, int) {
      const uint32_t k = fkey(z);
      if (k > kNegInfKey && k >= floor_key && (k & hm) == want) {
        const int d = (int)((k >> shift) & dmask);
        atomicAdd(&s->cnt[d], 1u);
        if (mass) {
          unsigned long long h, l;
          fixed_parts(weight(z), h, l);
          if (h) atomicAdd(&s->hi[d], h);
          if (l) atomicAdd(&s->lo[d], l);
        }
      }
    });
    __syncthreads();
  }

  // The topmost digit whose cumulative total from the largest key (plus the
  // `above` totals of the digits chosen before) reaches the target: count >= k
  // (mass_mode false) or mass / W >= top_p.  Leaves the digit and the totals
  // strictly above it in s->digit / s->above_*; returns the level's totals.
  __device__ void search(bool mass_mode, uint32_t k, double W, float top_p, uint32_t above_c,
                         unsigned long long above_h, unsigned long long above_l,
                         unsigned long long& tot_h, unsigned long long& tot_l) {
    constexpr int kPer = kSelDigits / NT;
    uint32_t c = 0;
    unsigned long long h = 0, l = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = kSelDigits - 1 - (kPer * (int)threadIdx.x + i);
      c += s->cnt[d];
      h += s->hi[d];
      l += s->lo[d];
    }
    if (threadIdx.x == 0) {                // a defined digit even if no crossing were found
      s->digit = 0;
      s->above_c = above_c;
      s->above_h = above_h;
      s->above_l = above_l;
    }
    uint32_t ec, tc;
    unsigned long long eh, el;
    block_scan3<NT>(c, h, l, s, ec, eh, el, tc, tot_h, tot_l);   // its barrier orders the default
    const double Wd = W > 0.0 ? W : fixed_to_double(above_h + tot_h, above_l + tot_l);
    auto reach = [&](uint32_t rc, unsigned long long rh, unsigned long long rl) -> bool {
      return mass_mode ? fixed_to_double(rh, rl) / Wd >= (double)top_p : rc >= k;
    };
    uint32_t rc = above_c + ec;
    unsigned long long rh = above_h + eh, rl = above_l + el;
    bool before = reach(rc, rh, rl);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = kSelDigits - 1 - (kPer * (int)threadIdx.x + i);
      const uint32_t nc = rc + s->cnt[d];
      const unsigned long long nh = rh + s->hi[d], nl = rl + s->lo[d];
      const bool after = reach(nc, nh, nl);
      if (!before && after) {              // exactly one digit of the block
        s->digit = d;
        s->above_c = rc;
        s->above_h = rh;
        s->above_l = rl;
      }
      before = after;
      rc = nc;
      rh = nh;
      rl = nl;
    }
    __syncthreads();
  }

  // Walk the key down to one value.  Returns its key, and the count and mass
  // of the keys >= it (masses only in mass mode).  floor_key: keys below it
  // are left out (the top-k cut, for top-p).  W: top-p's total, 0 to take it
  // from the first level.
  __device__ uint32_t descend(bool bf16, bool mass_mode, uint32_t k, float top_p,
                              uint32_t floor_key, double& W, uint32_t& ge_c,
                              unsigned long long& ge_h, unsigned long long& ge_l) {
    uint32_t prefix = 0u, above_c = 0u;
    unsigned long long above_h = 0ull, above_l = 0ull;
    const int levels = bf16 ? 2 : 3;
    uint32_t dc = 0u;
    unsigned long long dh = 0ull, dl = 0ull;
    for (int lv = 0; lv < levels; ++lv) {
      level_pass(lv, prefix, floor_key, mass_mode);
      unsigned long long th, tl;
      search(mass_mode, k, lv == 0 ? 0.0 : W, top_p, above_c, above_h, above_l, th, tl);
      if (lv == 0 && mass_mode) W = fixed_to_double(th, tl);
      const int d = s->digit & (kSelDigits - 1);
      prefix |= (uint32_t)d << sel_shift(lv);
      above_c = s->above_c;
      above_h = s->above_h;
      above_l = s->above_l;
      dc = s->cnt[d];
      dh = s->hi[d];
      dl = s->lo[d];
      __syncthreads();                     // every thread has read the search's result
    }
    ge_c = above_c + dc;
    ge_h = above_h + dh;
    ge_l = above_l + dl;
    // bfloat16 keys have their low 16 bits fixed: 0 for a positive logit,
    // all ones for a negative one, so the two digits determine the key
    if (bf16 && !(prefix & 0x80000000u)) prefix |= 0x3ffu;
    return prefix;
  }
};

// The kept list from its (id << 32 | logit bits) entries in LDS, any order:
// an ascending bitonic sort by id over the next power of two (padding sorts
// last, within kKeptCap entries), then the first n written out.  The caller
// has made the entries visible (a barrier after the last append).
template <int NT>
__device__ void sort_kept_by_id(unsigned long long* ids, int n, Kept* __restrict__ kept) {
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = n + threadIdx.x; i < P; i += NT) ids[i] = ~0ull;
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < P / 2; i += NT) {
        const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long a = ids[lo], b = ids[hi];
        if ((a > b) == up) {
          ids[lo] = b;
          ids[hi] = a;
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    Kept e;
    e.id = (int)(ids[i] >> 32);
    e.z = __uint_as_float((uint32_t)ids[i]);
    kept[i] = e;
  }
}

// The whole select for one row.  Writes the kept list (sorted by id) when
// the kept set has at most kKeptCap tokens; returns the row's FiltRow.
// top_k: 0 or >= V is off; top_p: 1 is off (at least one is on).  NT is the
// block size; tbl must already be staged and visible.
template <typename T, int NT>
__device__ FiltRow select_row(const T* __restrict__ row, int V, bool bf16, int top_k, float top_p,
                              double invT, const double* tbl, SelectLds* s,
                              Kept* __restrict__ kept) {
  static_assert(NT % kWave == 0 && NT / kWave <= kSelMaxWaves && kSelDigits % NT == 0,
                "block size");
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  FiltRow out;
  out.pad = 0;

  // row maximum and the number of finite logits
  float mx = -INFINITY;
  uint32_t nf = 0u;
  for_each_logit<T, NT>(row, V, [&](float z, int) {
    mx = fmaxf(mx, z);
    nf += z > -INFINITY ? 1u : 0u;
  });
  mx = wave_max(mx);
  nf = wave_sum_u32(nf);
  if (lane == 0) {
    s->wmax[wid] = mx;
    s->wn[wid] = nf;
  }
  __syncthreads();
  float m = -INFINITY;
  uint32_t nfin = 0u;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    m = fmaxf(m, s->wmax[w]);
    nfin += s->wn[w];
  }
  if (nfin == 0u) {
    out.m = -INFINITY;
    out.tau = INFINITY;
    out.S = 0.0;
    out.count = 0;
    out.status = 2;                        // no finite logit
    return out;
  }

  RowSelect<T, NT> rs{row, V, m, invT, tbl, s};
  const bool topk_on = top_k > 0 && (uint32_t)top_k < nfin;
  const bool topp_on = top_p < 1.0f;
  uint32_t tau = kNegInfKey + 1u;          // every finite key
  uint32_t cnt = nfin;
  unsigned long long mh = 0ull, ml = 0ull;
  bool have_mass = false;
  double W = 0.0;
  if (topk_on) {
    unsigned long long h, l;
    tau = rs.descend(bf16, false, (uint32_t)top_k, 1.0f, 0u, W, cnt, h, l);
  }
  if (topp_on) {
    W = 0.0;
    tau = rs.descend(bf16, true, 0u, top_p, tau, W, cnt, mh, ml);
    have_mass = true;
  }

  // The listing pass: the kept tokens (key >= tau), their mass when the walk
  // did not give it, and their ids when they fit the list.
  const bool list = cnt <= (uint32_t)kKeptCap;
  if (list || !have_mass) {
    unsigned long long* ids = s->hi;       // the histogram is free now
    if (threadIdx.x == 0) {
      s->nlist = 0;
      s->kept_h = s->kept_l = 0ull;
    }
    __syncthreads();
    for_each_logit<T, NT>(row, V, [&](float z, int id) {
      const uint32_t k = fkey(z);
      if (k > kNegInfKey && k >= tau) {
        if (!have_mass) {
          unsigned long long h, l;
          fixed_parts(rs.weight(z), h, l);
          if (h) atomicAdd(&s->kept_h, h);
          if (l) atomicAdd(&s->kept_l, l);
        }
        if (list) {
          const int slot = atomicAdd(&s->nlist, 1);
          if (slot < kKeptCap)
            ids[slot] = ((unsigned long long)(uint32_t)id << 32) | __float_as_uint(z + 0.0f);
        }
      }
    });
    __syncthreads();
    if (!have_mass) {
      mh = s->kept_h;
      ml = s->kept_l;
    }
    if (list) sort_kept_by_id<NT>(ids, (int)cnt, kept);
  }
  out.m = m;
  out.tau = unkey(tau);
  out.S = fixed_to_double(mh, ml);
  out.count = (int)cnt;
  out.status = 0;
  return out;
}

}  // namespace specv
