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
  double g;   // estimate of S_t / S_d, the two rows' natural-exp normalisers (reject only)
  double pad2;
};
static_assert(sizeof(Plan) == 48, "Plan is 48 bytes");

// fp64 sampler: per-chunk record and near-tie slots.
constexpr int kTieCap = 32;                  // near ties recorded per chunk
constexpr double kTieWindow = 1.0 / 16384.0; // relative width of the near-tie band
constexpr int kMaxSampChunks = 2048;        // V <= kMaxSampChunks * kSampChunk
struct ChunkRec {
  double et, ed;   // sum of e_t, e_d over the chunk
  double at, ad;   // sum of e_t, e_d over tokens certainly having p > q
  int ntie;        // near ties found (may exceed kTieCap: then the exact path runs)
  int pad[7];
};
static_assert(sizeof(ChunkRec) == 64, "ChunkRec is 64 bytes");
struct Tie {
  double et, ed;
  int v, pad;
};
static_assert(sizeof(Tie) == 24, "Tie is 24 bytes");

// Top-k / top-p path: candidate select, per-row merge, kept lists.
constexpr int kFiltThreads = 256;
constexpr int kFiltPerThread = 32;
constexpr int kFiltChunk = kFiltThreads * kFiltPerThread;   // 8192 tokens per chunk
constexpr int kFiltSortMax = 4096;          // candidates a row merge can sort in LDS
constexpr int kFiltMaxChunks = 32;          // V <= 32 * 8192 on the filter path
constexpr int kKeptCap = 512;               // kept tokens per row after top-k / top-p
constexpr int kFiltMaxTopK = 128;           // candidate slots stay ~1.5 k only up to here
struct FiltRow {
  float m;      // row maximum (exact)
  float tau;    // final threshold: a token is kept iff its logit >= tau
  double S;     // float64 normaliser sum_{kept} exp((z - m) / T)
  int count;    // kept tokens (list length)
  int status;   // 0 ok; 1 capacity exceeded; 2 no finite logit
  long pad;
};
static_assert(sizeof(FiltRow) == 32, "FiltRow is 32 bytes");
struct Kept {
  int id;
  float z;
};

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

// Unconditional 16-byte load of elements [e0, e0 + kPerVec) of a 16-byte
// aligned row, as floats.  Callers use it only on chunks they have checked,
// uniformly for the whole workgroup, to be aligned and inside the row: a
// per-lane bounds branch around each load would split the loads into
// exec-masked regions and serialise them.
template <typename T>
__device__ __forceinline__ void load_vec_fast(const T* __restrict__ row, long e0, float* out) {
  const uint4 w = *reinterpret_cast<const uint4*>(row + e0);
  unpack(w, out, T{});
}

// Same, with the nontemporal hint: for logits streamed exactly once.
template <typename T>
__device__ __forceinline__ void load_vec_stream(const T* __restrict__ row, long e0, float* out) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + e0);
  uint4 w;
  w.x = __builtin_nontemporal_load(p);
  w.y = __builtin_nontemporal_load(p + 1);
  w.z = __builtin_nontemporal_load(p + 2);
  w.w = __builtin_nontemporal_load(p + 3);
  unpack(w, out, T{});
}

// Checked load of the same elements for tail or unaligned chunks: a whole
// 16-byte vector when it is aligned and inside the row, element by element
// only for the one vector that straddles V.  Elements at or beyond V read as
// -inf (they carry no probability mass).
template <typename T>
__device__ __forceinline__ void load_vec_checked(const T* __restrict__ row, long e0, int V,
                                                 bool aligned, float* out) {
  constexpr int N = Elem<T>::kPerVec;
  if (aligned && e0 + N <= V) {
    load_vec_fast(row, e0, out);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = (e0 + i < V) ? to_f32(row[e0 + i]) : -INFINITY;
  }
}

// Raw-word loads: the same elements as load_vec_*, left packed so a caller
// can issue them and unpack later.  Elements at or beyond V read as -inf.
__device__ __forceinline__ uint32_t neg_inf_bits(float) { return 0xff800000u; }
__device__ __forceinline__ uint32_t neg_inf_bits(bf16_t) { return 0xff80u; }
__device__ __forceinline__ uint32_t elem_bits(const float* row, long e) {
  return __float_as_uint(row[e]);
}
__device__ __forceinline__ uint32_t elem_bits(const bf16_t* row, long e) { return row[e]; }

template <typename T>
__device__ __forceinline__ uint4 load_raw_stream(const T* __restrict__ row, long e0) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + e0);
  uint4 w;
  w.x = __builtin_nontemporal_load(p);
  w.y = __builtin_nontemporal_load(p + 1);
  w.z = __builtin_nontemporal_load(p + 2);
  w.w = __builtin_nontemporal_load(p + 3);
  return w;
}
template <typename T>
__device__ __forceinline__ uint4 load_raw_checked(const T* __restrict__ row, long e0, int V,
                                                  bool aligned) {
  constexpr int N = Elem<T>::kPerVec;
  if (aligned && e0 + N <= V) return *reinterpret_cast<const uint4*>(row + e0);
  uint32_t e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = e0 + i < V ? elem_bits(row, e0 + i) : neg_inf_bits(T{});
  if constexpr (N == 4) {
    return make_uint4(e[0], e[1], e[2], e[3]);
  } else {
    return make_uint4(e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16);
  }
}

// Order-preserving 32-bit key of a float (larger float -> larger key): the
// sign bit set for a positive float, every bit flipped for a negative one.
// Written as one XOR with a sign-derived mask, no select, so a key costs one
// register where it is kept.  -0 is first made +0 (adding +0 does that), so
// that keys compare exactly as the floats do.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float unkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
constexpr uint32_t kNegInfKey = 0x007fffffu;   // fkey(-inf)

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Wave reductions of a float: four DPP steps reduce each 16-lane row (quad
// swaps, then the half-row and row mirrors, which pair each lane with one in
// the other half once the halves are uniform), then the four row results are
// read as scalars and combined in a fixed order.  No LDS traffic and no lane
// index arithmetic; every lane gets the same, bit-identical value.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xb1>(v));      // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4e>(v));      // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));     // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));     // row_mirror
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xb1>(v);
  v += dpp_f32<0x4e>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
// The same sum for a double (each DPP step moves its two 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double lane_f64(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xb1>(v);
  v += dpp_f64<0x4e>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
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
