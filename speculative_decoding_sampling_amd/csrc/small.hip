// Small-batch verification: everything after the row-statistics pass in one
// kernel, for calls with few (request, row pair, chunk) triples.
//
// The method is the one of accept.hip and sample.hip: the accept scan of
// each request (nickwang.xyz "推测解码：草稿、验证与实际加速", section
// "接受与拒绝怎样保住分布"), then an inverse-CDF draw from max(p_j - q_j, 0)
// after a rejection at j or from p_n after full acceptance (same page,
// sections "候选已知，验证才能并行" and "算完三个 token 的全部概率"), in float64 with
// the same chunk pass and draw code.  At these sizes the four kernels of the
// general path are bound by their launch latency rather than by their work
// (tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告", section "6. 扩展性与安全性",
// operator fusion, names cutting launch overhead as the purpose), so this
// kernel removes the dependency that forces the split: the chunk pass does
// not wait for the accept scan's choice of row pair but runs for every pair
// the request could draw from (rows j < n_b: residual of target and draft
// row j; row n_b: the bonus row alone), (n_b + 1) times the float64 work of
// the general path, which is small here.
//
// Workgroups of request b: slot 0 runs the accept scan (one wave) and writes
// the plan; slot 1 + j * nch + c runs the chunk pass of chunk c of pair j.
// Each one that has work arrives once at the request's counter (cleared by
// the row-statistics pass before this kernel) with an agent-scope acq_rel
// add after all its stores have completed; the last of the
// (n_b + 1) * nch + 1 arrivals reads the plan and draws from the records of
// the pair it names.  No workgroup waits for another, so the grid needs no
// co-residency.  On gfx950 the release writes back the XCD's L2 (without
// it, dirty lines of two XCDs would be merged in no fixed order, and the
// accept scan's placeholder token and the draw's token share their bytes);
// the writebacks of one XCD serialise, which is cheap for the few hundred
// workgroups of this kernel and far too costly for the general path's
// thousands.  A variant publishing through agent-scope atomic stores and
// loads instead measured only ~0.3 us faster.
#include "accept_core.h"
#include "sample_core.h"

namespace specv {

template <typename T>
__global__ __launch_bounds__(kSampThreads) void verify_small_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ tokens,
    const int* __restrict__ draft_len, const float* __restrict__ u,
    const float* __restrict__ u_final, int K, int V, int nch_row, int nch, float c, double invT,
    int eos_id, const float2* __restrict__ part, const float* __restrict__ zx,
    ChunkRec* __restrict__ recs, Tie* __restrict__ ties, PairStat* __restrict__ pstat,
    int* __restrict__ arrivals, AcceptOut out) {
  __shared__ DrawLds s;
  __shared__ Tie tl[kTieCap];
  __shared__ int tcnt[2];
  __shared__ int s_last;

  const int per = (K + 1) * nch + 1;                 // workgroups per request
  const int b = blockIdx.x / per, slot = blockIdx.x % per;
  const int R = 2 * K + 1;
  // Row pairs the request can draw from (none for an error request); read
  // inside each branch, after that branch's loads are issued.
  auto pairs_of = [&](int nb) { return (nb < 0 || nb > K) ? 0 : nb + 1; };
  int npair;
  Exp64Stage<kSampThreads> xs;
  xs.fetch();
  if (slot == 0) {
    if (threadIdx.x < kWave)
      accept_request<T, false>(b, threadIdx.x, tgt, dft, tokens, draft_len, u, u_final, K, V,
                               nch_row, c, invT, eos_id, part, zx, nullptr, out);
    npair = pairs_of(draft_len ? draft_len[b] : 0);   // null: no drafts (sampling)
  } else {
    const int j = (slot - 1) / nch, cc = (slot - 1) % nch;
    // The logits and the row partials are requested together with draft_len
    // (target row j <= K and draft row j < K exist whatever draft_len is), so
    // the pass starts one round trip after the launch.  The partials of rows
    // the request does not use are stale and go unused.
    const bool has_d = j < K;
    const T* trow = tgt + target_row_off(b, j, K, V);
    const T* drow = has_d ? dft + draft_row_off(b, j, K, V) : nullptr;
    Raw8<T> rt, rd;
    load_raw8(trow, (long)cc * kSampChunk, V, rt);
    if (has_d) load_raw8(drow, (long)cc * kSampChunk, V, rd);
    // the pair's statistics from the row partials, combined as the accept
    // scan combines them
    const float2* prow = part + (size_t)b * R * nch_row;
    float Mt, St, Md, Sd;
    combine_rows(prow + (size_t)j * nch_row, prow + (size_t)(K + 1 + j) * nch_row, nch_row, c,
                 true, has_d, Mt, St, Md, Sd);
    const int nb_raw = draft_len ? draft_len[b] : 0;
    npair = pairs_of(nb_raw);
    if (j >= npair) return;                          // a pair this request never draws from
    const bool rej = j < nb_raw;                     // j = n_b: the bonus row alone
    const double g = rej ? normaliser_ratio(Mt, St, Md, Sd, c) : 0.0;
    const double mti = (double)Mt * invT, mdi = rej ? (double)Md * invT : 0.0;   // m / T
    xs.store(s.tbl);
    if (threadIdx.x == 0) tcnt[0] = 0;
    __syncthreads();                                 // table staged, tie counter clear
    float zt[kSampPerThread], zd[kSampPerThread];
    unpack8(rt, zt);
    if (rej) unpack8(rd, zd);
    const long e0 = (long)cc * kSampChunk + (long)threadIdx.x * kSampPerThread;
    const size_t pr = (size_t)b * (K + 1) + j;
    pass_chunk(zt, zd, rej, e0, mti, mdi, invT, g, s.tbl, s.dl, tl, &tcnt[0], &tcnt[1],
               recs + pr * nch + cc, ties + (pr * nch + cc) * kTieCap);
    if (cc == 0 && threadIdx.x == 0) {
      PairStat ps;
      ps.mt = Mt;
      ps.md = rej ? Md : 0.f;
      ps.g = g;
      pstat[pr] = ps;
    }
  }

  // Arrival.  Every wave waits for its own stores to complete before the
  // barrier; thread 0's release then covers all of them, and its acquire
  // (as the last arriver) the loads of every wave after the second barrier.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(arrivals + b, 1, __ATOMIC_ACQ_REL,
                                    __HIP_MEMORY_SCOPE_AGENT) == npair * nch;
  __syncthreads();
  if (!s_last) return;                               // uniform per block

  // The last arrival: the plan and every record of the request are visible.
  const Plan pl = out.plan[b];
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per block
  const size_t pr = (size_t)b * (K + 1) + pl.stop;
  const ChunkRec* rb = recs + pr * nch;
  const Tie* tb = ties + pr * nch * kTieCap;
  DrawPre pre;
  draw_prefetch(rb, tb, nch, pre);
  const PairStat ps = pstat[pr];
  Plan pd = pl;                                      // the pass's own maxima and ratio
  pd.mt = ps.mt;
  pd.md = ps.md;
  pd.g = ps.g;
  draw_request<T>(tgt, dft, u_final[b], b, K, V, nch, invT, pd, rb, tb, pre, xs, s,
                  out.out_tokens, out.rmass_out);
}

// Workgroups of the small-batch kernel for these sizes (0 if out of range).
size_t small_blocks(int B, int K, int V) {
  const size_t nch = ((size_t)V + kSampChunk - 1) / kSampChunk;
  if (nch > (size_t)kMaxSampChunks) return 0;
  return (size_t)B * ((size_t)(K + 1) * nch + 1);
}

hipError_t launch_verify_small(bool bf16, const void* tgt, const void* dft, const int* tokens,
                               const int* draft_len, const float* u, const float* u_final, int B,
                               int K, int V, int nch_row, float c, double invT, int eos_id,
                               const float2* part, const float* zx, ChunkRec* recs, Tie* ties,
                               PairStat* pstat, int* arrivals, const AcceptOut& out,
                               hipStream_t stream) {
  const size_t blocks = small_blocks(B, K, V);
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const int nch = (V + kSampChunk - 1) / kSampChunk;
#define SPECV_SMALL(TT)                                                                        \
  verify_small_kernel<TT><<<dim3((unsigned)blocks), dim3(kSampThreads), 0, stream>>>(          \
      static_cast<const TT*>(tgt), static_cast<const TT*>(dft), tokens, draft_len, u, u_final, \
      K, V, nch_row, nch, c, invT, eos_id, part, zx, recs, ties, pstat, arrivals, out)
  if (bf16) SPECV_SMALL(bf16_t); else SPECV_SMALL(float);
#undef SPECV_SMALL
  return hipGetLastError();
}

}  // namespace specv
