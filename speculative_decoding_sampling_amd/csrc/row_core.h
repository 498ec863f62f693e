// Row-statistics arithmetic shared by the row-statistics pass and the
// one-kernel small-batch path: per chunk of a row, the maximum logit m and
// the partial normaliser s = sum 2^(z*c - fl(m*c)) (c = log2(e)/T), the
// softmax normaliser of the target and draft distributions in pieces
// (tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告", section "4. 实现逻辑";
// nickwang.xyz "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布").
// Both kernels run exactly these steps, so a chunk gets the same bits from
// either, and a draft row equal to its target row the same statistics.
#pragma once

#include "common.h"

namespace specv {

// The chunk's raw 16-byte vectors of one thread: each wave reads one
// contiguous segment of VECS * 1 KB (its loads 1 KB apart, so concurrent
// loads spread over the HBM channels); where the chunk is interior and the
// row 16-byte aligned, nontemporal (STREAM: rows read once) or plain cached
// loads (rows a later kernel of the call reads again, which then finds them
// in the memory-side cache), element-checked otherwise.
template <typename T, int VECS, bool STREAM = true>
__device__ __forceinline__ void row_chunk_load(const T* __restrict__ row, long e_base, int V,
                                               uint4* w) {
  constexpr int N = Elem<T>::kPerVec;
  constexpr int kChunk = kRowThreads * VECS * N;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const long e_wave = e_base + (long)wid * VECS * kWave * N + (long)lane * N;
  const bool aligned = aligned16(row);
  if (aligned && e_base + kChunk <= V) {              // uniform: interior chunk
#pragma unroll
    for (int j = 0; j < VECS; ++j)
      w[j] = STREAM ? load_raw_stream(row, e_wave + (long)j * kWave * N)
                    : *reinterpret_cast<const uint4*>(row + e_wave + (long)j * kWave * N);
  } else {
#pragma unroll
    for (int j = 0; j < VECS; ++j)
      w[j] = load_raw_checked(row, e_wave + (long)j * kWave * N, V, aligned);
  }
}

// The wave's part of the chunk partial, (max, sum), identical in every lane.
template <typename T, int VECS>
__device__ __forceinline__ float2 row_wave_partial(const uint4* w, float c) {
  constexpr int N = Elem<T>::kPerVec;
  float v[VECS][N];
#pragma unroll
  for (int j = 0; j < VECS; ++j) unpack(w[j], v[j], T{});
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < VECS; ++j)
#pragma unroll
    for (int i = 0; i < N; ++i) m = fmaxf(m, v[j][i]);
  m = wave_max(m);

  float s = 0.f;
  if (m != -INFINITY) {
    const float mc = __fmul_rn(m, c);                // the exact reference fl(m*c)
#pragma unroll
    for (int j = 0; j < VECS; ++j)
#pragma unroll
      for (int i = 0; i < N; ++i) s += __builtin_amdgcn_exp2f(fmaf(v[j][i], c, -mc));
  }
  s = wave_sum(s);
  return make_float2(m, s);
}

// The chunk partial from the workgroup's wave partials, combined in wave order.
__device__ __forceinline__ float2 row_combine_waves(const float2* red, float c) {
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kRowThreads / kWave; ++w) M = fmaxf(M, red[w].x);
  float S = 0.f;
  if (M != -INFINITY) {
    const float Mc = __fmul_rn(M, c);
#pragma unroll
    for (int w = 0; w < kRowThreads / kWave; ++w)
      if (red[w].x != -INFINITY)
        S += red[w].y * __builtin_amdgcn_exp2f(__fmul_rn(red[w].x, c) - Mc);
  }
  return make_float2(M, S);
}

}  // namespace specv
