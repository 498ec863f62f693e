// The radix-select path of the filters: the top-k / top-p threshold of every
// needed row by one workgroup per row, for any top_k, top-p with or without
// top-k, and any kept-set size (nickwang.xyz "推测解码：草稿、验证与实际加速",
// section "接受与拒绝怎样保住分布": p and q both include temperature, top-k and
// top-p).  bfloat16 rows go through the one-read histogram select
// (hist_select.h), float32 rows through the multi-pass radix select
// (radix_select.h), which is also the former's fallback.
#include "common.h"
#include "exp64.h"
#include "filter_common.h"
#include "hist_select.h"
#include "radix_select.h"

namespace specv {

// ---------------------------------------------------------------------------
// filter_rows: the general select (radix_select.h) for every needed row, one
// 1024-thread workgroup per row: any top_k, top-p with or without top-k, any
// kept-set size.
constexpr int kSelThreads = 1024;

template <typename T>
__global__ __launch_bounds__(kSelThreads) void filter_rows_kernel(
    const T* __restrict__ tgt, const T* __restrict__ dft, const int* __restrict__ draft_len,
    int K, int V, int top_k, float top_p, double invT, FiltRow* __restrict__ rows,
    Kept* __restrict__ kept) {
  __shared__ SelectLds sl;
  __shared__ double tbl[SPECV_EXP64_N];
  const int R = 2 * K + 1;
  const int rr = blockIdx.x;
  const int r = rr % R, b = rr / R;
  const int nb = draft_len ? draft_len[b] : 0;      // null: no drafts (sampling)
  if (nb < 0 || nb > K) return;
  bool is_target;
  int k;
  if (!row_needed(r, K, nb, is_target, k)) return;
  for (int i = threadIdx.x; i < SPECV_EXP64_N; i += kSelThreads) tbl[i] = kExp64Table[i];
  __syncthreads();
  const T* row = is_target ? tgt + target_row_off(b, k, K, V) : dft + draft_row_off(b, k, K, V);
  const FiltRow o = select_row<T, kSelThreads>(row, V, sizeof(T) == 2, top_k, top_p, invT, tbl,
                                               &sl, kept + (size_t)rr * kKeptCap);
  if (threadIdx.x == 0) rows[rr] = o;
}

// bfloat16 rows: the histogram select (hist_select.h), 142 KB of LDS, one
// workgroup per CU.
__global__ __launch_bounds__(kSelThreads) void filter_rows_hist_kernel(
    const bf16_t* __restrict__ tgt, const bf16_t* __restrict__ dft,
    const int* __restrict__ draft_len, int K, int V, int top_k, float top_p, double invT,
    FiltRow* __restrict__ rows, Kept* __restrict__ kept) {
  __shared__ HistPool pool;
  __shared__ HistAux aux;
  __shared__ double tbl[SPECV_EXP64_N];
  const int R = 2 * K + 1;
  const int rr = blockIdx.x;
  const int r = rr % R, b = rr / R;
  const int nb = draft_len ? draft_len[b] : 0;      // null: no drafts (sampling)
  if (nb < 0 || nb > K) return;
  bool is_target;
  int k;
  if (!row_needed(r, K, nb, is_target, k)) return;
  for (int i = threadIdx.x; i < SPECV_EXP64_N; i += kSelThreads) tbl[i] = kExp64Table[i];
  const bf16_t* row = is_target ? tgt + target_row_off(b, k, K, V) : dft + draft_row_off(b, k, K, V);
  // the histogram pass's first barrier makes the table visible
  const FiltRow o = select_row_hist<kSelThreads>(row, V, top_k, top_p, invT, tbl, &pool, &aux,
                                                 kept + (size_t)rr * kKeptCap);
  if (threadIdx.x == 0) rows[rr] = o;
}

hipError_t launch_filter_rows(bool bf16, const void* tgt, const void* dft, const int* draft_len,
                              int B, int K, int V, int top_k, float top_p, double invT,
                              FiltRow* rows, Kept* kept, hipStream_t stream) {
  const size_t blocks = (size_t)B * (2 * K + 1);
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (bf16)
    filter_rows_hist_kernel<<<dim3((unsigned)blocks), dim3(kSelThreads), 0, stream>>>(
        static_cast<const bf16_t*>(tgt), static_cast<const bf16_t*>(dft), draft_len, K, V,
        top_k, top_p, invT, rows, kept);
  else
    filter_rows_kernel<float><<<dim3((unsigned)blocks), dim3(kSelThreads), 0, stream>>>(
        static_cast<const float*>(tgt), static_cast<const float*>(dft), draft_len, K, V, top_k,
        top_p, invT, rows, kept);
  return hipGetLastError();
}

}  // namespace specv
