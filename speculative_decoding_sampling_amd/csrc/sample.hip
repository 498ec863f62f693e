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
#include "sample_core.h"

namespace specv {

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
// Everything that does not depend on the plan is requested with it: the exp
// table, this thread's first chunk record and that chunk's first near-tie
// slots.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void sample_finish_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const float* __restrict__ u_final,
    int K, int V, int nch, double invT, const Plan* __restrict__ plan,
    const ChunkRec* __restrict__ recs, const Tie* __restrict__ ties, int* __restrict__ out_tokens,
    double* __restrict__ rmass_out) {
  __shared__ DrawLds s;
  const int b = blockIdx.x;
  Exp64Stage<kSampThreads> xs;
  xs.fetch();
  const Plan pl = plan[b];
  const float uf = u_final[b];
  const ChunkRec* rb = recs + (size_t)b * nch;
  const Tie* tb = ties + (size_t)b * nch * kTieCap;
  DrawPre pre;
  draw_prefetch(rb, tb, nch, pre);
  if (pl.path != kPathReject && pl.path != kPathBonus) return;   // uniform per block
  draw_request<T>(tgt, dft, uf, b, K, V, nch, invT, pl, rb, tb, pre, xs, s, out_tokens,
                  rmass_out);
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

