// Helpers shared by the filtered path's kernels (filter.hip, filter_rows.hip,
// sample_list.hip).
#pragma once

#include <type_traits>

#include "common.h"
#include "wave_scan.h"

namespace specv {

// Exclusive scan of one value per thread over the block (thread order) and
// the block total: the wave scans on DPP lane moves, the waves' totals in
// a fixed order.
template <typename V>
__device__ __forceinline__ V block_scan_excl(V v, V* lds, V& total) {
  static_assert(std::is_same<V, double>::value || std::is_same<V, int>::value,
                "double or int");
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  V x, excl;
  if constexpr (std::is_same<V, double>::value) {
    x = wave_incl_scan(v);
    excl = wave_shr1(x);
  } else {
    x = (int)wave_incl_scan_u32((uint32_t)v);
    excl = x - v;                                    // exact for integers
  }
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
  v = (int)wave_reduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) {
    return (uint32_t)min((int)a, (int)b);
  });
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
