// Helpers shared by the filtered path's kernels (filter.hip, filter_rows.hip,
// sample_list.hip).
#pragma once

#include "common.h"

namespace specv {

template <typename V>
__device__ __forceinline__ V block_scan_excl(V v, V* lds, V& total) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  V x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const V y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  V excl = __shfl_up(x, 1, kWave);
  if (lane == 0) excl = V(0);
  __syncthreads();
  if (lane == kWave - 1) lds[wid] = x;
  __syncthreads();
  V off = V(0);
  total = V(0);
#pragma unroll
  for (int w = 0; w < kFiltThreads / kWave; ++w) {
    if (w < wid) off += lds[w];
    total += lds[w];
  }
  return off + excl;
}

__device__ __forceinline__ int block_min_i(int v, int* lds) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  int r = lds[0];
#pragma unroll
  for (int w = 1; w < kFiltThreads / kWave; ++w) r = min(r, lds[w]);
  return r;
}

// Row index r in [0, 2K+1) of request b: needed when it is target row
// k <= n_b or draft row k < n_b.
__device__ __forceinline__ bool row_needed(int r, int K, int nb, bool& is_target, int& k) {
  is_target = r <= K;
  k = is_target ? r : r - (K + 1);
  return k <= (is_target ? nb : nb - 1);
}

}  // namespace specv
