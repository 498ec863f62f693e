// Small-batch verification: the whole call in one kernel, for calls with few
// (request, row pair, chunk) triples.
//
// The method is the one of row_stats.hip, accept.hip and sample.hip: the row
// statistics, the accept scan of each request (nickwang.xyz
// "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布"), then an
// inverse-CDF draw from max(p_j - q_j, 0) after a rejection at j or from p_n
// after full acceptance (same page, sections "候选已知，验证才能并行" and
// "算完三个 token 的全部概率"), in float64 with the same chunk pass and draw
// code.  At these sizes the four kernels of the general path are bound by
// their launch and dependency latency rather than by their work (tbxsx.cn
// "推测解码采样验证优化策略 —— 深度调研报告", section "6. 扩展性与安全性", operator
// fusion, names cutting launch overhead as the purpose).  Here every stage
// starts at launch: the chunk pass does not wait for the accept scan's choice
// of row pair but runs for every pair the request could draw from (rows
// j < n_b: residual of target and draft row j; row n_b: the bonus row
// alone), (n_b + 1) times the float64 work of the general path, which is
// small here; and no stage waits for a kernel boundary to read the row
// statistics.
//
// Grid, in this order: one workgroup per (request, row, 8192- or 4096-element
// chunk) for the row statistics; then per request one workgroup per (row
// pair j <= K, 1024-token chunk) for the chunk pass and, last, one for the
// accept scan and the draw.  A workgroup waits only for workgroups earlier in
// the grid, which the hardware dispatches first (in order on every XCD), so
// the grid needs no co-residency: the earliest waiting workgroup always has
// everything it waits for dispatched.  Every wait is bounded; one that runs
// out turns its request into a per-request error (n_emitted = -1) instead of
// hanging.
//
// Publication.  A row-statistics partial is two 64-bit words, (max | tag) and
// (sum | tag), stored and polled as agent-scope atomics, which are coherent
// across the XCDs' L2 caches; a chunk pass writes its records with ordinary
// stores and then a flag with an agent-scope release (the XCD's L2 written
// back), which the draw polls and follows with an agent-scope acquire.
//
// Tags make the workspace reusable without clearing.  A tag is a bijective
// mix of the request's call counter -- a word in the workspace that only the
// request's draw advances, after every workgroup of the request that
// publishes has read it -- keyed by the word's position and by a salt of the
// call's sizes (B, K, V, dtype).  The counter advances by an odd stride drawn
// from the salt.  So a word left by an earlier call of the same sizes never
// passes for this call's (the counter has moved on), and neither, but for a
// 2^-32 chance per word, does anything else: a fresh allocation, or words and
// counters left by a call of other sizes that shared the memory (their
// counters run on another stride, so they do not keep in step with these).
// The salt also mixes in a sequence number of the launch: if a wait runs out
// (its request then reports an error), the draw advances the counter before
// every workgroup of the request may have read it, and one that reads it
// late tags its words with the advanced counter -- under this launch's salt,
// which no later launch shares.  A captured graph replays one launch's
// arguments, so there only the counter tells replays apart, and after such
// an error the workspace is to be zeroed before the next replay.
#include <atomic>

#include "accept_core.h"
#include "row_core.h"
#include "sample_core.h"

namespace specv {

constexpr int kTinyMaxRecs = 1024;          // row partials one workgroup stages in LDS
constexpr int kTinyMaxPoll = 1 << 18;       // polls of one word before a wait gives up
std::atomic<int> g_small_poll_limit{kTinyMaxPoll};   // lowered only by a test hook

// A bijective mix of 32-bit words (multiply-xorshift rounds).
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x7FEB352Du;
  h ^= h >> 15;
  h *= 0x846CA68Bu;
  h ^= h >> 16;
  return h;
}
// Tag of word id in the call of a request whose call counter is nc, for
// calls of the sizes whose salt is salt: bijective in nc for a given word.
__device__ __forceinline__ uint32_t tiny_tag(uint32_t nc, uint32_t id, uint32_t salt) {
  return mix32(nc ^ mix32(id ^ salt));
}
// The counter after a call: an odd stride, so it never repeats within 2^32
// calls of these sizes.
__device__ __forceinline__ uint32_t next_call(uint32_t nc, uint32_t salt) {
  return nc + (mix32(salt ^ 0x68E31DA4u) | 1u);
}
constexpr uint32_t kIdZx = 1u << 28;        // id domains: partial words below, then zx, flags
constexpr uint32_t kIdFlag = 1u << 29;

__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t bits, uint32_t tag) {
  __hip_atomic_store(p, (uint64_t)tag << 32 | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Polls two tagged words until they carry tag0 and tag1 (false if the wait
// ran out), both loads in flight at once: each poll is a round trip to
// memory, so polling them one after the other takes two.
__device__ __forceinline__ bool poll_tagged2(const uint64_t* p0, const uint64_t* p1,
                                             uint32_t tag0, uint32_t tag1, uint32_t& bits0,
                                             uint32_t& bits1, int max_poll) {
  for (int i = 0; i < max_poll; ++i) {
    const uint64_t w0 = __hip_atomic_load(p0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t w1 = __hip_atomic_load(p1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w0 >> 32) == tag0 && (uint32_t)(w1 >> 32) == tag1) {
      bits0 = (uint32_t)w0;
      bits1 = (uint32_t)w1;
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  bits0 = bits1 = 0;
  return false;
}
__device__ __forceinline__ bool poll_flag(const uint32_t* p, uint32_t tag, int max_poll) {
  for (int i = 0; i < max_poll; ++i) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Staging of row partials: entry i of the list (row slot i / nch_row, chunk
// i % nch_row) polled from row row_of(i / nch_row) of request b into st[i]
// as (max, sum).  extra() runs in every thread before the closing barrier
// (other waits of the caller, overlapped with these), and returns false if
// one of them ran out.  Returns false, block-wide, if any wait ran out.
template <typename RowOf, typename Extra>
__device__ __forceinline__ bool stage_partials(const uint64_t* __restrict__ part, int b, int R,
                                               int nch_row, int count, uint32_t nc,
                                               uint32_t salt, RowOf row_of, float2* st,
                                               int* s_fail, int max_poll, Extra extra) {
  if (threadIdx.x == 0) *s_fail = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < count; i += kSampThreads) {
    const int r = row_of(i / nch_row), ch = i % nch_row;
    const size_t pi = ((size_t)b * R + r) * nch_row + ch;
    uint32_t m, s;
    if (!poll_tagged2(part + 2 * pi, part + 2 * pi + 1, tiny_tag(nc, 2 * (uint32_t)pi, salt),
                      tiny_tag(nc, 2 * (uint32_t)pi + 1, salt), m, s, max_poll))
      *s_fail = 1;
    st[i] = make_float2(__uint_as_float(m), __uint_as_float(s));
  }
  if (!extra()) *s_fail = 1;
  __syncthreads();
  return *s_fail == 0;
}

// One row's combined statistics from n staged partials, the steps and order
// of combine_rows (the same bits as the general path's accept scan) over the
// real entries only: a batch's padding (-inf, 0) changes neither its maximum
// nor its sum, so skipping it saves the dependent chain of a full batch per
// row (a row of these small vocabularies has 1 to 4 partials).
__device__ __forceinline__ void combine_staged(const float2* st, int n, float c, float& M,
                                               float& S) {
  float m = -INFINITY, s = 0.f;
  for (int base = 0; base < n; base += kCombineBatch) {
    const int nb = min(kCombineBatch, n - base);
    float mb = m;
    for (int j = 0; j < nb; ++j) mb = fmaxf(mb, st[base + j].x);
    if (mb != -INFINITY) {
      const float mbc = __fmul_rn(mb, c);
      if (m != -INFINITY) s *= __builtin_amdgcn_exp2f(__fmul_rn(m, c) - mbc);
      for (int j = 0; j < nb; ++j)
        if (st[base + j].x != -INFINITY)
          s += st[base + j].y * __builtin_amdgcn_exp2f(__fmul_rn(st[base + j].x, c) - mbc);
    }
    m = mb;
  }
  M = m;
  S = s;
}

template <typename T>
__global__ __launch_bounds__(kSampThreads) void verify_small_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ tokens,
    const int* __restrict__ draft_len, const float* __restrict__ u,
    const float* __restrict__ u_final, int K, int V, int nch_row, int nch, float c, double invT,
    int eos_id, int nrs, uint64_t* __restrict__ part, uint64_t* __restrict__ zxw,
    ChunkRec* __restrict__ recs, Tie* __restrict__ ties, PairStat* __restrict__ pstat,
    uint32_t* __restrict__ flags, uint32_t* __restrict__ calls, uint32_t salt, int max_poll,
    AcceptOut out) {
  __shared__ DrawLds s;
  __shared__ Tie tl[kTieCap];
  __shared__ int tcnt[2];
  __shared__ float2 st[kTinyMaxRecs];
  __shared__ float2 red[kRowThreads / kWave];
  __shared__ int s_fail;
  const int R = 2 * K + 1;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;

  if ((int)blockIdx.x < nrs) {
    // (1) Row statistics of chunk `chunk` of row r of request b (the
    // arithmetic of row_stats.hip), published as two tagged words.
    constexpr int N = Elem<T>::kPerVec;
    constexpr int kChunk = kRowThreads * kRowVecs * N;
    const int chunk = blockIdx.x % nch_row;
    const int rq = blockIdx.x / nch_row;
    const int r = rq % R, b = rq / R;
    const int nb = draft_len ? draft_len[b] : 0;      // null: no drafts (sampling)
    const uint32_t nc = calls[b];
    if (nb < 0 || nb > K) return;                    // the accept scan reports the error
    const bool is_target = r <= K;
    const int k = is_target ? r : r - (K + 1);
    if (k > (is_target ? nb : nb - 1)) return;       // row not needed for this request
    const T* row = is_target ? tgt + target_row_off(b, k, K, V) : dft + draft_row_off(b, k, K, V);
    uint4 w[kRowVecs];
    const long e_base = (long)chunk * kChunk;
    row_chunk_load<T, kRowVecs>(row, e_base, V, w);
    int gx = -1;
    float gz = 0.f;
    if (tokens && k < K) {
      const int x = tokens[(size_t)b * K + k];
      if (x >= 0 && x < V && x >= e_base && x < e_base + kChunk) {
        gx = x;
        gz = to_f32(row[x]);
      }
    }
    const float2 ws = row_wave_partial<T, kRowVecs>(w, c);
    if (lane == 0) red[wid] = ws;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float2 cp = row_combine_waves(red, c);
      const size_t pi = ((size_t)b * R + r) * nch_row + chunk;
      put_tagged(part + 2 * pi, __float_as_uint(cp.x), tiny_tag(nc, 2 * (uint32_t)pi, salt));
      put_tagged(part + 2 * pi + 1, __float_as_uint(cp.y), tiny_tag(nc, 2 * (uint32_t)pi + 1, salt));
      if (gx >= 0) {
        const uint32_t zi = (uint32_t)((size_t)b * 2 * K + (is_target ? k : K + k));
        put_tagged(zxw + zi, __float_as_uint(gz), tiny_tag(nc, kIdZx | zi, salt));
      }
    }
    return;
  }

  const int per = (K + 1) * nch + 1;                 // workgroups per request after the rows
  const int b = (blockIdx.x - nrs) / per, slot = (blockIdx.x - nrs) % per;
  auto pairs_of = [&](int nb) { return (nb < 0 || nb > K) ? 0 : nb + 1; };
  Exp64Stage<kSampThreads> xs;
  xs.fetch();

  if (slot < per - 1) {
    // (2) Chunk pass of chunk cc of row pair j.  The logits are requested at
    // once (target row j <= K and draft row j < K exist whatever draft_len is).
    const int j = slot / nch, cc = slot % nch;
    const bool has_d = j < K;
    const T* trow = tgt + target_row_off(b, j, K, V);
    const T* drow = has_d ? dft + draft_row_off(b, j, K, V) : nullptr;
    Raw8<T, kSmallPerThread> rt, rd;
    load_raw8<T, kSmallPerThread>(trow, (long)cc * kSmallChunk, V, rt);
    if (has_d) load_raw8<T, kSmallPerThread>(drow, (long)cc * kSmallChunk, V, rd);
    const int nb_raw = draft_len ? draft_len[b] : 0;
    const uint32_t nc = calls[b];
    if (j >= pairs_of(nb_raw)) return;               // a pair this request never draws from
    const bool rej = j < nb_raw;                     // j = n_b: the bonus row alone
    const bool ok = stage_partials(
        part, b, R, nch_row, (rej ? 2 : 1) * nch_row, nc, salt,
        [&](int q) { return q == 0 ? j : K + 1 + j; }, st, &s_fail, max_poll,
        [] { return true; });
    float Mt, St, Md = -INFINITY, Sd = 0.f;
    combine_staged(st, nch_row, c, Mt, St);
    if (rej) combine_staged(st + nch_row, nch_row, c, Md, Sd);
    const double g = rej ? normaliser_ratio(Mt, St, Md, Sd, c) : 0.0;
    const double mti = (double)Mt * invT, mdi = rej ? (double)Md * invT : 0.0;   // m / T
    xs.store(s.tbl);
    if (threadIdx.x == 0) tcnt[0] = 0;
    __syncthreads();                                 // table staged, tie counter clear
    float zt[kSmallPerThread], zd[kSmallPerThread];
    unpack8<T, kSmallPerThread>(rt, zt);
    if (rej) unpack8<T, kSmallPerThread>(rd, zd);
    const long e0 = (long)cc * kSmallChunk + (long)threadIdx.x * kSmallPerThread;
    const size_t pr = (size_t)b * (K + 1) + j;
    pass_chunk<kSmallPerThread>(zt, zd, rej, e0, mti, mdi, invT, g, s.tbl, s.dl, tl, &tcnt[0],
                                &tcnt[1],
               recs + pr * nch + cc, ties + (pr * nch + cc) * kTieCap);
    if (cc == 0 && threadIdx.x == 0) {
      PairStat ps;
      ps.mt = Mt;
      ps.md = rej ? Md : 0.f;
      ps.g = g;
      pstat[pr] = ps;
    }
    // Publish: every wave's stores complete before the barrier, then thread
    // 0's release writes them back and sets the flag (tag + 1 if a wait ran
    // out: the draw then reports the request as an error).
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t fi = (uint32_t)(pr * nch + cc);
      const uint32_t tag = tiny_tag(nc, kIdFlag | fi, salt);
      __hip_atomic_store(flags + fi, ok ? tag : tag + 1u, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // (3) The accept scan and the draw of request b.
  const int nb_raw = draft_len ? draft_len[b] : 0;
  const uint32_t nc = calls[b];
  const float uf = u_final[b];
  const int npair = pairs_of(nb_raw);
  const int nb = npair > 0 ? nb_raw : 0;
  int x = -1;
  float uk = 0.f, zt = -INFINITY, zd = -INFINITY;
  if (wid == 0 && lane < K) {
    x = tokens[(size_t)b * K + lane];
    uk = u[(size_t)b * K + lane];
  }
  const bool xin = wid == 0 && lane < K && x >= 0 && x < V;
  // the statistics of target rows 0..n_b, then of draft rows 0..n_b-1, and
  // (polled by the last wave meanwhile) the logits at the drafted tokens of
  // rows 0..n_b-1, recorded with the statistics
  __shared__ float2 zxs[kWave];
  bool ok = true;
  if (npair > 0)
    ok = stage_partials(
        part, b, R, nch_row, (2 * nb + 1) * nch_row, nc, salt,
        [&](int q) { return q <= nb ? q : K + 1 + (q - nb - 1); }, st, &s_fail, max_poll, [&] {
          const int zl = (int)threadIdx.x - (kSampThreads - kWave);
          if (zl < 0 || zl >= nb) return true;
          const int xz = tokens[(size_t)b * K + zl];
          if (xz < 0 || xz >= V) return true;
          const uint32_t zi = (uint32_t)((size_t)b * 2 * K + zl);
          uint32_t bt, bd;
          const bool zok = poll_tagged2(zxw + zi, zxw + zi + K, tiny_tag(nc, kIdZx | zi, salt),
                                        tiny_tag(nc, kIdZx | (zi + K), salt), bt, bd, max_poll);
          zxs[zl] = make_float2(__uint_as_float(bt), __uint_as_float(bd));
          return zok;
        });
  if (wid == 0) {
    if (npair > 0 && lane < nb && xin) {
      zt = zxs[lane].x;
      zd = zxs[lane].y;
    }
    LaneRows rs;
    if (npair > 0) {
      if (lane <= nb) combine_staged(st + lane * nch_row, nch_row, c, rs.Mt, rs.St);
      if (lane < nb) combine_staged(st + (nb + 1 + lane) * nch_row, nch_row, c, rs.Md, rs.Sd);
      if (nb == kWave) combine_staged(st + kWave * nch_row, nch_row, c, rs.Mk, rs.Sk);
    }
    // a wait that ran out makes the request an error, as a bad draft_len does
    accept_scan<false>(b, lane, K, c, invT, eos_id, ok ? nb_raw : -1, uf, x, uk, xin, zt, zd, rs,
                       out);
  }
  __syncthreads();                                   // the plan, written by wave 0
  const Plan pl = out.plan[b];

  // Every chunk pass of the request publishes before the draw reads, and
  // before the call counter moves on (each of them read it first).
  if (threadIdx.x == 0) s_fail = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < npair * nch; i += kSampThreads) {
    const size_t fi = (size_t)b * (K + 1) * nch + i;
    if (!poll_flag(flags + fi, tiny_tag(nc, kIdFlag | (uint32_t)fi, salt), max_poll)) s_fail = 1;
  }
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();                                   // records visible to every wave
  const bool fail = s_fail != 0;
  if ((pl.path == kPathReject || pl.path == kPathBonus) && !fail) {
    const size_t pr = (size_t)b * (K + 1) + pl.stop;
    const ChunkRec* rb = recs + pr * nch;
    const Tie* tb = ties + pr * nch * kTieCap;
    DrawPre pre;
    draw_prefetch(rb, tb, nch, pre);
    const PairStat ps = pstat[pr];
    Plan pd = pl;                                    // the pass's own maxima and ratio
    pd.mt = ps.mt;
    pd.md = ps.md;
    pd.g = ps.g;
    draw_request<T, kSmallPerThread>(tgt, dft, uf, b, K, V, nch, invT, pd, rb, tb, pre, xs, s,
                                     out.out_tokens, out.rmass_out);
  } else if (fail) {                                 // a chunk pass's wait ran out
    for (int k = threadIdx.x; k <= K; k += kSampThreads)
      out.out_tokens[(size_t)b * (K + 1) + k] = -1;
    if (threadIdx.x == 0) {
      if (out.n_emitted) out.n_emitted[b] = -1;
      if (out.stop_out) out.stop_out[b] = -1;
      if (out.path_out) out.path_out[b] = kPathError;
      if (out.rmass_out) out.rmass_out[b] = 0.0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) calls[b] = next_call(nc, salt);   // every word of this call is read
}

int set_small_poll_limit(int limit) {
  return g_small_poll_limit.exchange(limit < 1 ? kTinyMaxPoll : limit);
}

// Whether the one-kernel path serves these sizes: its workgroups stage at
// most kTinyMaxRecs row partials.
bool small_fits(int K, int V, int nch_row) {
  const size_t nch = ((size_t)V + kSmallChunk - 1) / kSmallChunk;
  return nch <= (size_t)kMaxSampChunks && (size_t)(2 * K + 1) * nch_row <= (size_t)kTinyMaxRecs;
}

// Workgroups of the small-batch kernel after the row statistics (0 if out of range).
size_t small_blocks(int B, int K, int V) {
  const size_t nch = ((size_t)V + kSmallChunk - 1) / kSmallChunk;
  if (nch > (size_t)kMaxSampChunks) return 0;
  return (size_t)B * ((size_t)(K + 1) * nch + 1);
}

hipError_t launch_verify_small(bool bf16, const void* tgt, const void* dft, const int* tokens,
                               const int* draft_len, const float* u, const float* u_final, int B,
                               int K, int V, int nch_row, float c, double invT, int eos_id,
                               uint64_t* part, uint64_t* zxw, ChunkRec* recs, Tie* ties,
                               PairStat* pstat, uint32_t* flags, uint32_t* calls,
                               const AcceptOut& out, hipStream_t stream) {
  const size_t tail = small_blocks(B, K, V);
  const size_t nrs = (size_t)B * (2 * K + 1) * nch_row;
  if (tail == 0 || !small_fits(K, V, nch_row) || nrs + tail > 0x7fffffffu)
    return hipErrorInvalidConfiguration;
  const int nch = (V + kSmallChunk - 1) / kSmallChunk;
  // salt of these sizes and this launch (FNV-1a over B, K, V, the dtype, the
  // chunk counts and the launch's sequence number)
  static std::atomic<uint32_t> launch_seq{0};
  const uint32_t seq = launch_seq.fetch_add(1, std::memory_order_relaxed);
  uint32_t salt = 2166136261u;
  for (uint32_t v : {(uint32_t)B, (uint32_t)K, (uint32_t)V, (uint32_t)bf16, (uint32_t)nch_row,
                     (uint32_t)nch, seq})
    for (int i = 0; i < 4; ++i) salt = (salt ^ ((v >> (8 * i)) & 0xffu)) * 16777619u;
#define SPECV_SMALL(TT)                                                                        \
  verify_small_kernel<TT><<<dim3((unsigned)(nrs + tail)), dim3(kSampThreads), 0, stream>>>(    \
      static_cast<const TT*>(tgt), static_cast<const TT*>(dft), tokens, draft_len, u, u_final, \
      K, V, nch_row, nch, c, invT, eos_id, (int)nrs, part, zxw, recs, ties, pstat, flags,      \
      calls, salt, g_small_poll_limit.load(std::memory_order_relaxed), out)
  if (bf16) SPECV_SMALL(bf16_t); else SPECV_SMALL(float);
#undef SPECV_SMALL
  return hipGetLastError();
}

}  // namespace specv
