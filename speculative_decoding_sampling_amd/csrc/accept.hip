// Accept scan kernel: one wave64 per request, lane k owns draft position k
// (K <= 64; target row 64, the bonus row of 64 drafts, is read by every lane).
// The decision is accept_scan and the gather of its inputs accept_request
// (accept_core.h), which the small-batch kernel runs as well.
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
  accept_request<T, FILT>(blockIdx.x, threadIdx.x, tgt, dft, tokens, draft_len, u, u_final, K, V,
                          nch_row, c, invT, eos_id, part, zx, frows, out);
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
