// Accept scan kernel: one wave64 per request, lane k owns draft position k
// (K <= 64; target row 64, the bonus row of 64 drafts, is read by every lane).
// The decision itself is accept_scan (accept_core.h); this kernel gathers
// its inputs.  Without filters the row statistics are the chunk partials of
// the row-statistics pass and the logits at the drafted tokens are the ones
// that pass recorded; with top-k / top-p they are the per-row FiltRow and two
// gathers from the logits.
//
// Latency: the kernel is a short dependency chain per request, so every load
// that does not depend on another (draft_len, u_final, tokens, uniforms, the
// recorded logits and the statistics of all K+1 target and K draft rows) is
// issued up front; rows beyond draft_len are loaded but never used.
#include "accept_core.h"

namespace specv {

template <typename T, bool FILT>
__global__ __launch_bounds__(kWave) void accept_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ tokens,
    const int* __restrict__ draft_len, const float* __restrict__ u,
    const float* __restrict__ u_final, int K, int V, int nch_row, float c, double invT,
    int eos_id, const float2* __restrict__ part, const float* __restrict__ zx,
    const FiltRow* __restrict__ frows, AcceptOut out) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int R = 2 * K + 1;
  const int nb_raw = draft_len ? draft_len[b] : 0;   // null: no drafts (sampling)
  const float uf = u_final[b];
  int x = -1;
  float uk = 0.f, zt = -INFINITY, zd = -INFINITY;
  if (lane < K) {
    x = tokens[(size_t)b * K + lane];
    uk = u[(size_t)b * K + lane];
    if constexpr (!FILT) {
      zt = zx[(size_t)b * 2 * K + lane];            // meaningful where the scan reads it
      zd = zx[(size_t)b * 2 * K + K + lane];
    }
  }
  const bool xin = lane < K && x >= 0 && x < V;
  LaneRows rs;
  if constexpr (FILT) {
    if (xin) {
      zt = to_f32(tgt[target_row_off(b, lane, K, V) + x]);
      zd = to_f32(dft[draft_row_off(b, lane, K, V) + x]);
    }
    if (lane <= K) rs.ft = frows[(size_t)b * R + lane];
    if (lane < K) rs.fd = frows[(size_t)b * R + K + 1 + lane];
    if (K == kWave) rs.fk = frows[(size_t)b * R + K];       // uniform: the bonus row of 64 drafts
  } else {
    const float2* prow = part + (size_t)b * R * nch_row;
    combine_rows(prow + (size_t)lane * nch_row, prow + (size_t)(K + 1 + lane) * nch_row, nch_row,
                 c, lane <= K, lane < K, rs.Mt, rs.St, rs.Md, rs.Sd);
    if (K == kWave) {                                        // uniform: the bonus row of 64 drafts
      float md, sd;
      combine_rows(prow + (size_t)K * nch_row, prow, nch_row, c, true, false, rs.Mk, rs.Sk, md, sd);
    }
  }
  accept_scan<FILT>(b, lane, K, c, invT, eos_id, nb_raw, uf, x, uk, xin, zt, zd, rs, out);
}

hipError_t launch_accept(bool bf16, bool filt, const void* tgt, const void* dft, const int* tokens,
                         const int* draft_len, const float* u, const float* u_final, int B,
                         int K, int V, int nch_row, float c, double invT, int eos_id,
                         const float2* part, const float* zx, const FiltRow* frows,
                         const AcceptOut& out, hipStream_t stream) {
#define SPECV_ACCEPT(TT, FF)                                                                     \
  accept_kernel<TT, FF><<<dim3(B), dim3(kWave), 0, stream>>>(                                    \
      static_cast<const TT*>(tgt), static_cast<const TT*>(dft), tokens, draft_len, u, u_final, K, \
      V, nch_row, c, invT, eos_id, part, zx, frows, out)
  if (bf16) {
    if (filt) SPECV_ACCEPT(bf16_t, true); else SPECV_ACCEPT(bf16_t, false);
  } else {
    if (filt) SPECV_ACCEPT(float, true); else SPECV_ACCEPT(float, false);
  }
#undef SPECV_ACCEPT
  return hipGetLastError();
}

}  // namespace specv
