// Target-model LM head with the row statistics in its epilogue.
//
// The pages suggest fusing the verification-stage forward pass of the target
// model with the sampling step (tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告",
// section "6. 扩展性与安全性", operator fusion).  The last layer of that forward
// pass is the LM head: logits[m][v] = sum_d H[m][d] * W[v][d].  Here it runs on
// the matrix cores and, while each tile of logits is still in registers,
// reduces it to the softmax statistics the accept scan needs -- the maximum and
// the normaliser sum 2^(z*c - fl(m*c)) of tbxsx.cn section "4. 实现逻辑" and
// nickwang.xyz "推测解码：草稿、验证与实际加速", section "接受与拒绝怎样保住分布" --
// so the target logits are written once and never read back for statistics.
//
// Product.  C^T = W * H^T on v_mfma_f32_32x32x16_bf16: the weights are the A
// operand (32 vocabulary rows of a tile), the hidden states the B operand (32
// hidden rows), fp32 accumulation.  With this orientation the output tile
// holds one hidden row per lane and 16 vocabulary ids per register set, so
// the per-row statistics are mostly an in-register reduction.
//
// Work split.  A workgroup of 8 waves owns 256 vocabulary ids (32 per wave)
// and 320 hidden rows (10 tiles of 32; larger M runs more row blocks).  Per
// 64-wide k block each lane reads 64 contiguous bytes of its weight row
// straight into registers (the weights are streamed from HBM exactly once
// per row block), while the block's 320 x 64 hidden states are staged in LDS
// (double-buffered; rows padded to 144 bytes so the 16-byte fragment reads of
// 8 consecutive lanes cover all banks).  The k values of one MFMA step are
// {k0 + 32 h + 8 s + i : h = lane / 32, i < 8} for step s = 0..3: any
// permutation of k shared by both operands leaves the dot product unchanged,
// and this one makes each lane's weight bytes contiguous.
//
// Epilogue.  Each accumulator is rounded to bfloat16 (nearest even) and
// written; the statistics are taken over the rounded values, the logits every
// later stage reads.  Per row: the max and sum over the lane's 16 ids, the
// lane pair holding the other 16, then the 8 waves through LDS in a fixed
// order, giving one (max, normaliser) per 256-id tile.  fold_tile_stats then
// combines 32 tiles into the 8192-id chunk partials of the row-statistics
// layout, and records the logit of each row's drafted token.
#include "common.h"

namespace specv {

typedef __bf16 lm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lm_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLmThreads = 512;
constexpr int kLmWaves = kLmThreads / kWave;        // 8
constexpr int kLmVocab = kLmWaves * 32;             // 256 vocabulary ids per workgroup
constexpr int kLmMTiles = 10;
constexpr int kLmRows = kLmMTiles * 32;             // 320 hidden rows per row block
constexpr int kLmKB = 64;                           // k per block
constexpr int kLmLdsRow = kLmKB + 8;                // bf16 per LDS row (144 bytes)
constexpr int kLmHPieces = kLmRows * kLmKB / 8;     // 16-byte pieces of one hidden block
constexpr int kLmHPer = kLmHPieces / kLmThreads;    // 5 per thread
static_assert(kLmHPieces % kLmThreads == 0, "hidden block pieces per thread");
static_assert(kRowThreads * kRowVecs * 8 % kLmVocab == 0, "a statistics chunk is whole tiles");
constexpr int kLmTilesPerChunk = kRowThreads * kRowVecs * 8 / kLmVocab;   // 32

__device__ __forceinline__ lm_bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(lm_bf16x8, w); }

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kLmThreads, 1) void lm_head_kernel(
    const bf16_t* __restrict__ H, const bf16_t* __restrict__ W, int M, int D, int V, int ntile,
    float c, bf16_t* __restrict__ out, float2* __restrict__ tpart) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][kLmRows * kLmLdsRow];

  const int tile = blockIdx.x % ntile;
  const int m0 = (blockIdx.x / ntile) * kLmRows;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int h = lane / 32, l32 = lane % 32;

  // This lane's weight row (rows past V read row V - 1; their sums are dropped).
  const int v_lane = tile * kLmVocab + wave * 32 + l32;
  const bf16_t* wrow = W + (size_t)min(v_lane, V - 1) * D + 32 * h;

  // Hidden-state staging: piece q = threadIdx.x + kLmThreads * j is row q / 8,
  // 16-byte piece q % 8 of the block; rows past M are staged as zeros.
  const bf16_t* hsrc[kLmHPer];
  int hdst[kLmHPer];
  bool hok[kLmHPer];
#pragma unroll
  for (int j = 0; j < kLmHPer; ++j) {
    const int q = threadIdx.x + kLmThreads * j;
    const int r = q / 8, p = q % 8;
    hok[j] = m0 + r < M;
    hsrc[j] = H + (size_t)(hok[j] ? m0 + r : 0) * D + p * 8;
    hdst[j] = r * kLmLdsRow + p * 8;
  }
  auto load_w = [&](int k0, uint4* w) {
    const uint4* src = reinterpret_cast<const uint4*>(wrow + k0);
#pragma unroll
    for (int s = 0; s < 4; ++s) w[s] = src[s];
  };
  auto load_h = [&](int k0, uint4* hv) {
#pragma unroll
    for (int j = 0; j < kLmHPer; ++j)
      hv[j] = hok[j] ? *reinterpret_cast<const uint4*>(hsrc[j] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto store_h = [&](int buf, const uint4* hv) {
#pragma unroll
    for (int j = 0; j < kLmHPer; ++j) *reinterpret_cast<uint4*>(&lds[buf][hdst[j]]) = hv[j];
  };

  lm_f32x16 acc[kLmMTiles];
#pragma unroll
  for (int t = 0; t < kLmMTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  const int nkb = D / kLmKB;
  uint4 wa[4], wn[4], hn[kLmHPer];
  load_w(0, wa);
  load_h(0, hn);
  store_h(0, hn);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const bool more = kb + 1 < nkb;
    if (more) {                                      // next block in flight during this one
      load_w((kb + 1) * kLmKB, wn);
      load_h((kb + 1) * kLmKB, hn);
    }
    const bf16_t* hb = lds[kb & 1] + l32 * kLmLdsRow + 32 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const lm_bf16x8 a = as_bf16x8(wa[s]);
#pragma unroll
      for (int t = 0; t < kLmMTiles; ++t) {
        const lm_bf16x8 b =
            as_bf16x8(*reinterpret_cast<const uint4*>(hb + t * 32 * kLmLdsRow + 8 * s));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
    if (more) {
      store_h((kb + 1) & 1, hn);                     // that buffer's readers passed the last barrier
#pragma unroll
      for (int s = 0; s < 4; ++s) wa[s] = wn[s];
    }
    __syncthreads();
  }

  // Epilogue.  acc[t][r] is logit (row m0 + 32 t + l32, id vbase + vof(r)).
  float2* red = reinterpret_cast<float2*>(&lds[0][0]);   // [kLmWaves][kLmRows]; LDS is free now
  const int vbase = tile * kLmVocab + wave * 32 + 4 * h;
  // 8-byte stores need every row to start 8-byte aligned
  const bool vec_ok = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
#pragma unroll
  for (int t = 0; t < kLmMTiles; ++t) {
    const int m = m0 + t * 32 + l32;
    float z[16];
    uint32_t zb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      zb[r] = bf16_rne_bits(acc[t][r]);
      z[r] = __uint_as_float(zb[r] << 16);
    }
    // ids of register r: vbase + 8 (r / 4) + r % 4: four runs of four
    if (m < M) {
      bf16_t* orow = out + (size_t)m * V;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v0 = vbase + 8 * q;
        if (vec_ok && v0 + 3 < V) {
          uint2 pk;
          pk.x = zb[4 * q] | (zb[4 * q + 1] << 16);
          pk.y = zb[4 * q + 2] | (zb[4 * q + 3] << 16);
          *reinterpret_cast<uint2*>(orow + v0) = pk;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v0 + i < V) orow[v0 + i] = (bf16_t)zb[4 * q + i];
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (vbase + 8 * (r / 4) + r % 4 < V) mx = fmaxf(mx, z[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float s = 0.f;
    if (mx != -INFINITY) {
      const float mc = __fmul_rn(mx, c);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (vbase + 8 * (r / 4) + r % 4 < V) s += __builtin_amdgcn_exp2f(fmaf(z[r], c, -mc));
    }
    s += __shfl_xor(s, 32, kWave);
    if (h == 0) red[wave * kLmRows + t * 32 + l32] = make_float2(mx, s);
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < kLmRows; rr += kLmThreads) {
    const int m = m0 + rr;
    if (m >= M) continue;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kLmWaves; ++w) Mx = fmaxf(Mx, red[w * kLmRows + rr].x);
    float S = 0.f;
    if (Mx != -INFINITY) {
      const float Mc = __fmul_rn(Mx, c);
#pragma unroll
      for (int w = 0; w < kLmWaves; ++w) {
        const float2 p = red[w * kLmRows + rr];
        if (p.x != -INFINITY) S += p.y * __builtin_amdgcn_exp2f(__fmul_rn(p.x, c) - Mc);
      }
    }
    tpart[(size_t)m * ntile + tile] = make_float2(Mx, S);
  }
}

// Tile partials -> chunk partials of the row-statistics layout, one wave per
// (target row, chunk): lane i takes tile 32 q + i; the combine runs in a fixed
// tree order.  Target row m = b (K + 1) + k goes to part[(b R + k) nch + q]
// (R = 2K + 1).  The wave whose chunk holds the row's drafted token records
// that token's logit in zx[b][k].
__global__ __launch_bounds__(kWave) void fold_tile_stats_kernel(
    const float2* __restrict__ tpart, const bf16_t* __restrict__ logits,
    const int* __restrict__ tokens, int B, int K, int V, int ntile, int nch, float c,
    float2* __restrict__ part, float* __restrict__ zx) {
  const int q = blockIdx.x % nch;
  const int m = blockIdx.x / nch;
  const int b = m / (K + 1), k = m % (K + 1);
  const int lane = threadIdx.x;
  const int tl = q * kLmTilesPerChunk + lane;
  float2 p = make_float2(-INFINITY, 0.f);
  if (lane < kLmTilesPerChunk && tl < ntile) p = tpart[(size_t)m * ntile + tl];
  const float Mx = wave_max(p.x);
  float s = 0.f;
  if (Mx != -INFINITY && p.x != -INFINITY)
    s = p.y * __builtin_amdgcn_exp2f(__fmul_rn(p.x, c) - __fmul_rn(Mx, c));
  const float S = wave_sum(s);
  const int R = 2 * K + 1;
  if (lane == 0) {
    part[((size_t)b * R + k) * nch + q] = make_float2(Mx, S);
    if (tokens && k < K) {
      const int x = tokens[(size_t)b * K + k];
      const int chunk = kRowThreads * kRowVecs * 8;
      if (x >= 0 && x < V && x / chunk == q)
        zx[(size_t)b * 2 * K + k] = __uint_as_float((uint32_t)logits[(size_t)m * V + x] << 16);
    }
  }
}

int lm_head_tiles(int V) { return (V + kLmVocab - 1) / kLmVocab; }
int lm_head_rows_per_block() { return kLmRows; }
int lm_head_kblock() { return kLmKB; }

hipError_t launch_lm_head(const void* hidden, const void* weight, int M, int D, int V, float c,
                          void* logits, float2* tpart, hipStream_t stream) {
  const int ntile = lm_head_tiles(V);
  const size_t blocks = (size_t)ntile * ((M + kLmRows - 1) / kLmRows);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu || D % kLmKB != 0) return hipErrorInvalidConfiguration;
  lm_head_kernel<<<dim3((unsigned)blocks), dim3(kLmThreads), 0, stream>>>(
      static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(weight), M, D, V, ntile, c,
      static_cast<bf16_t*>(logits), tpart);
  return hipGetLastError();
}

hipError_t launch_fold_tile_stats(const float2* tpart, const void* logits, const int* tokens,
                                  int B, int K, int V, int nch, float c, float2* part, float* zx,
                                  hipStream_t stream) {
  const size_t blocks = (size_t)B * (K + 1) * nch;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  fold_tile_stats_kernel<<<dim3((unsigned)blocks), dim3(kWave), 0, stream>>>(
      tpart, static_cast<const bf16_t*>(logits), tokens, B, K, V, lm_head_tiles(V), nch, c, part,
      zx);
  return hipGetLastError();
}

}  // namespace specv
