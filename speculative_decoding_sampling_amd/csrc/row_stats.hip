// Row statistics: per (request, needed row, vocabulary chunk), the chunk's
// maximum logit m and its partial normaliser s = sum 2^(z*c - fl(m*c)), with
// c = log2(e) / T in float32 and fl() the float32 product (never fused).
// These give the softmax normaliser of the target and draft distributions
// (tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告", section
// "4. 实现逻辑": softmax of logits over temperature; nickwang.xyz
// "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布").
//
// The workgroup whose chunk holds a row's drafted token also records that
// token's logit, so the accept scan needs no gather of its own.
//
// This pass reads every needed row once and carries nearly all of the call's
// HBM traffic.  Each workgroup streams one chunk with coalesced 16-byte loads
// issued up front, reduces with wave64 shuffles and combines its four waves
// in LDS.  Partials are combined later in a fixed order, so the result is
// deterministic and a draft row equal to its target row gets bit-identical
// statistics.
#include "row_core.h"

namespace specv {

template <typename T, int VECS, bool STREAM>
__global__ __launch_bounds__(kRowThreads) void row_stats_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    const int* __restrict__ tokens, int K, int V, int nchunk, int row_lo, int pairs_only,
    float c, float2* __restrict__ part, float* __restrict__ zx) {
  constexpr int N = Elem<T>::kPerVec;
  constexpr int kChunk = kRowThreads * VECS * N;
  const int R = 2 * K + 1;
  // The grid covers rows row_lo .. 2K of every request (row_lo = K + 1: draft
  // rows only, when the target rows' statistics come from elsewhere), or with
  // pairs_only the rows of drafted positions alone: target and draft rows
  // k < n_b, never the bonus row K.
  const int nrow = pairs_only ? 2 * K : R - row_lo;
  const int chunk = blockIdx.x % nchunk;
  const int rq = blockIdx.x / nchunk;
  const int q = rq % nrow;
  const int r = pairs_only ? (q < K ? q : q + 1) : row_lo + q;
  const int b = rq / nrow;
  const size_t rr = (size_t)b * R + r;
  const int nb = draft_len ? draft_len[b] : 0;      // null: no drafts (sampling)
  if (nb < 0 || nb > K) return;                      // the accept scan reports the error
  const bool is_target = r <= K;
  const int k = is_target ? r : r - (K + 1);
  if (k > (is_target && !pairs_only ? nb : nb - 1)) return;   // row not needed
  const T* row = is_target ? tgt + target_row_off(b, k, K, V) : dft + draft_row_off(b, k, K, V);

  uint4 w[VECS];
  const long e_base = (long)chunk * kChunk;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  row_chunk_load<T, VECS, STREAM>(row, e_base, V, w);

  // Arrival counter of the end-of-workgroup combine, cleared while the loads
  // are in flight: every wave waits on memory here anyway.
  __shared__ float2 red[kRowThreads / kWave];
  __shared__ int arrived;
  if (threadIdx.x == 0) arrived = 0;
  __syncthreads();

  // Drafted token of this row (draft position k < K): its logit, read after
  // the stream is in flight and stored at the end.  zx[b][k] is the target
  // row's, zx[b][K + k] the draft row's.
  int gx = -1;
  float gz = 0.f;
  if (tokens && k < K) {
    const int x = tokens[(size_t)b * K + k];
    if (x >= 0 && x < V && x >= e_base && x < e_base + kChunk) {
      gx = x;
      gz = to_f32(row[x]);
    }
  }

  const float2 ws = row_wave_partial<T, VECS>(w, c);

  // The last wave to finish combines the four wave partials; the others
  // exit at once instead of waiting at a barrier.  The arrival increment is
  // a workgroup-scope acquire-release: each wave's partial is written before
  // it arrives, and the last arriver reads them after.
  if (lane == 0) {
    red[wid] = ws;
    const int before = __hip_atomic_fetch_add(&arrived, 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_WORKGROUP);
    if (before != kRowThreads / kWave - 1) return;

    const float2 cp = row_combine_waves(red, c);
    part[(size_t)rr * nchunk + chunk] = cp;
    if (gx >= 0) zx[(size_t)b * 2 * K + (is_target ? k : K + k)] = gz;
  }
}

int row_stats_chunk(bool bf16) {
  return kRowThreads * kRowVecs * (bf16 ? Elem<bf16_t>::kPerVec : Elem<float>::kPerVec);
}

hipError_t launch_row_stats(bool bf16, const void* tgt, const void* dft, const int* draft_len,
                            const int* tokens, int B, int K, int V, int nchunk, float c,
                            float2* part, float* zx, hipStream_t stream, int row_lo, bool cached,
                            bool pairs_only) {
  if (row_lo < 0 || row_lo > 2 * K || (pairs_only && row_lo != 0)) return hipErrorInvalidValue;
  const size_t blocks = (size_t)B * (pairs_only ? 2 * K : 2 * K + 1 - row_lo) * nchunk;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
#define SPECV_ROWS(TT, ST)                                                                    \
  row_stats_kernel<TT, kRowVecs, ST><<<dim3((unsigned)blocks), dim3(kRowThreads), 0, stream>>>( \
      static_cast<const TT*>(tgt), static_cast<const TT*>(dft), draft_len, tokens, K, V, nchunk, \
      row_lo, (int)pairs_only, c, part, zx)
  if (bf16) {
    if (cached) SPECV_ROWS(bf16_t, false); else SPECV_ROWS(bf16_t, true);
  } else {
    if (cached) SPECV_ROWS(float, false); else SPECV_ROWS(float, true);
  }
#undef SPECV_ROWS
  return hipGetLastError();
}

}  // namespace specv
