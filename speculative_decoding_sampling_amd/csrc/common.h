// Shared device helpers for libspecverify (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

// Row-statistics pass: 256 threads, each holding kRowVecs 16-byte vectors.
constexpr int kRowThreads = 256;
constexpr int kRowVecs = 4;

// fp64 residual / bonus sampler: 256 threads x 8 contiguous elements.
constexpr int kSampThreads = 256;
constexpr int kSampPerThread = 8;
constexpr int kSampChunk = kSampThreads * kSampPerThread;

enum Path : int { kPathError = -1, kPathReject = 0, kPathBonus = 1, kPathEos = 2 };

// Per-request decision written by the accept scan and read by the sampler.
struct Plan {
  int path;   // Path
  int stop;   // rejected position, EOS position, or draft_len (bonus)
  int trow;   // target row the final draw uses (stop for reject and bonus)
  int drow;   // draft row of the residual (reject only)
  float mt;   // exact max logit of target row trow
  float md;   // exact max logit of draft row drow
  int pad0, pad1;
};
static_assert(sizeof(Plan) == 32, "Plan is 32 bytes");

// bf16 logits travel as their 16-bit patterns.
using bf16_t = uint16_t;

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPerVec = 4; };
template <> struct Elem<bf16_t> { static constexpr int kPerVec = 8; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ void unpack(const uint4 w, float* out, float) {
  out[0] = __uint_as_float(w.x);
  out[1] = __uint_as_float(w.y);
  out[2] = __uint_as_float(w.z);
  out[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void unpack(const uint4 w, float* out, bf16_t) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);            // element 2i: low half
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u); // element 2i+1: high half
  }
}

// Load the 16-byte vector of elements [e0, e0 + kPerVec) of `row` as floats.
// Elements at or beyond V read as -inf (they carry no probability mass).
// `aligned` says the row start is 16-byte aligned; e0 is a multiple of kPerVec.
template <typename T>
__device__ __forceinline__ void load_vec(const T* __restrict__ row, long e0, int V, bool aligned,
                                         float* out) {
  constexpr int N = Elem<T>::kPerVec;
  if (aligned && e0 + N <= V) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + e0);
    unpack(w, out, T{});
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = (e0 + i < V) ? to_f32(row[e0 + i]) : -INFINITY;
  }
}

// Butterfly reductions: every lane ends with the same, bit-identical value
// (each step adds the same two operands, and IEEE addition is commutative).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Row index helpers.  A request owns K+1 target rows and K draft rows; the
// row-statistics partials are indexed by r in [0, 2K+1): r <= K is target
// row r, r > K is draft row r - K - 1.
__device__ __forceinline__ size_t target_row_off(int b, int k, int K, int V) {
  return ((size_t)b * (K + 1) + k) * (size_t)V;
}
__device__ __forceinline__ size_t draft_row_off(int b, int k, int K, int V) {
  return ((size_t)b * K + k) * (size_t)V;
}

}  // namespace specv
