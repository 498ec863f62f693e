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
// Work split.  A workgroup of 8 waves (one per CU, two per SIMD) owns 256
// vocabulary ids (32 per wave) and 320 hidden rows (10 tiles of 32; larger M
// runs more row blocks).  Per 64-wide k block each wave reads its 32 x 64
// weights straight into registers, two blocks ahead of their use (the
// weights are streamed from HBM exactly once per row block), while the
// block's 320 x 64 hidden states are loaded straight into LDS, also two
// blocks ahead (three buffers; 16-byte pieces XOR-swizzled by row pair so
// each 16-lane pass of a fragment read covers all 64 banks once).  One
// 8-wave workgroup stages each hidden block once per CU; two 4-wave
// workgroups per CU each staged it (330 vs 308 us per launch at M = 320,
// D = 4096, V = 128256).
// The k values of one MFMA step are {k0 + 32 h + 8 s + i : h = lane / 32,
// i < 8} for step s = 0..3: any permutation of k shared by both operands
// leaves the dot product unchanged.
//
// Weight layout.  The weights are repacked once, when the model is loaded,
// into the order the kernel reads them: [128-id tile][k block][32-id group]
// [step s][lane] 16-byte pieces, piece (t, kb, w, s, l) holding
// W[128 t + 32 w + l % 32][64 kb + 32 (l / 32) + 8 s .. + 7], zero past V.
// One load instruction then reads 1 KB of consecutive bytes and a workgroup
// streams two contiguous ranges, where the row-major matrix costs it rows
// 8 KB apart per block (measured 379 vs 326 us per launch with 4-wave
// workgroups at M = 320, D = 4096, V = 128256).
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
typedef uint32_t lm_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLmThreads = 512;
constexpr int kLmWaves = kLmThreads / kWave;        // 8
constexpr int kLmVocab = kLmWaves * 32;             // 256 vocabulary ids per workgroup
constexpr int kLmMTiles = 10;
constexpr int kLmRows = kLmMTiles * 32;             // 320 hidden rows per row block
constexpr int kLmKB = 64;                           // k per block
constexpr int kLmHPieces = kLmRows * kLmKB / 8;     // 16-byte pieces of one hidden block
constexpr int kLmHPer = kLmHPieces / kLmThreads;    // 5 per thread
static_assert(kLmHPieces % kLmThreads == 0, "hidden block pieces per thread");
static_assert(kRowThreads * kRowVecs * 8 % kLmVocab == 0, "a statistics chunk is whole tiles");
constexpr int kLmTilesPerChunk = kRowThreads * kRowVecs * 8 / kLmVocab;   // 32
constexpr int kLmPackVocab = 128;                      // vocabulary ids per packed tile
constexpr int kLmPackGroups = kLmPackVocab / 32;       // 32-id groups (one wave each) per tile
constexpr int kLmPackWave = 4 * kWave * 8;             // packed elements of one group's block
constexpr int kLmPackBlock = kLmPackGroups * kLmPackWave;   // of one tile's block (16 KB)
static_assert(kLmVocab % kLmPackVocab == 0, "a workgroup covers whole packed tiles");
// epilogue transpose: half a row block of logits, rows padded to 264 ids
constexpr int kLmTrStride = kLmVocab + 8;
constexpr int kLmTrElems = (kLmRows / 2) * kLmTrStride;
constexpr int kLmTrPieces = (kLmRows / 2) * kLmVocab / 8;   // 16-byte pieces of a half
static_assert(kLmTrPieces % kLmThreads == 0, "transpose pieces per thread");
static_assert(kLmMTiles % 2 == 0, "the epilogue stores the row block in two halves");
static_assert(kLmTrElems * 2 % 16 == 0 &&
                  kLmTrElems * 2 + kLmWaves * kLmRows * 8 <= 3 * kLmRows * kLmKB * 2,
              "transpose buffer and statistics fit the staging buffers");

__device__ __forceinline__ lm_bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(lm_bf16x8, w); }
__device__ __forceinline__ lm_bf16x8 as_bf16x8(lm_u32x4 w) { return __builtin_bit_cast(lm_bf16x8, w); }

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// s_waitcnt immediates (vector-memory count only; LDS / export counts untouched)
constexpr int kWaitVm13 = 0x0F7D;
static_assert(kLmKB == 64 && kLmHPer == 5,
              "wait immediates assume 5 staging and 4 weight loads per block");
constexpr int kLmWLoads = 4;                        // weight loads per wave and block
// the block-start wait in lm_head_kernel lets two blocks' loads fly: vmcnt(18)
static_assert(2 * (kLmHPer + kLmWLoads) == 18, "block-start wait immediate");
static_assert(kLmMTiles == 10, "the fragment pipeline is written out for 20 pairs");
static_assert(kLmTilesPerChunk <= kWave, "one chunk's tiles fold in one wave");

__global__ __launch_bounds__(kLmThreads, 1) void lm_head_kernel(
    const bf16_t* __restrict__ H, const bf16_t* __restrict__ W, int M, int D, int V, int ntile,
    float c, bf16_t* __restrict__ out, float2* __restrict__ tpart) {
  // Hidden-state blocks, unpadded: row r's 16-byte piece p sits at slot
  // p ^ ((r >> 1) & 7) of the row.  A 128-byte row covers half of the 64
  // banks (even rows one half, odd rows the other), and one 16-lane pass of a
  // fragment read (16 consecutive rows, one piece) then touches every bank
  // once: 8 distinct slots among the even rows and 8 among the odd.
  // The three buffers are one array: the epilogue reuses all of it.
  __shared__ __attribute__((aligned(16))) bf16_t lds[3 * kLmRows * kLmKB];
  bf16_t* const lds0 = lds;
  bf16_t* const lds1 = lds + kLmRows * kLmKB;
  bf16_t* const lds2 = lds + 2 * kLmRows * kLmKB;

  const int tile = blockIdx.x % ntile;
  const int m0 = (blockIdx.x / ntile) * kLmRows;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int h = lane / 32, l32 = lane % 32;

  // This wave's packed weights (packed tile ptile, group wave % 4): block kb
  // at wbase + kb * kLmPackBlock, step s of this lane at + s * 512 + lane * 8
  // elements.  Ids past V are zeros, and a packed tile wholly past V (the
  // second half of a last, half-used workgroup tile) repeats the last one:
  // their sums are dropped.
  const int ptiles = (V + kLmPackVocab - 1) / kLmPackVocab;
  const int ptile = min(tile * (kLmVocab / kLmPackVocab) + wave / kLmPackGroups, ptiles - 1);
  const bf16_t* wbase = W + ((size_t)ptile * (D / kLmKB) * kLmPackGroups + wave % kLmPackGroups) *
                                kLmPackWave + lane * 8;

  // Hidden-state staging goes straight to LDS: instruction j of wave w fills
  // slots [(5 w + j) 64, +64), rows 8 (5 w + j) .. +8; lane i fills slot i
  // of those, i.e. row 8 (5 w + j) + i / 8 at position i % 8, which holds piece
  // (i % 8) ^ ((row >> 1) & 7).  Rows past M repeat row M - 1 (their sums are
  // dropped).
  // Row r_j = r0 + 8 j of instruction j has ((r_j >> 1) & 7) equal to
  // ((r0 >> 1) & 7) ^ 4 (j & 1), so each source is formed on the fly from r0.
  const int r0 = 8 * kLmHPer * wave + lane / 8;
  const int pc0 = (lane % 8) ^ ((r0 >> 1) & 7);
  auto stage_h = [&](int k0, bf16_t* buf) {
#pragma unroll
    for (int j = 0; j < kLmHPer; ++j) {
      const int row = min(m0 + r0 + 8 * j, M - 1);
      const bf16_t* src = H + (size_t)row * D + (pc0 ^ (4 * (j & 1))) * 8 + k0;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)src,
          (__attribute__((address_space(3))) void*)(buf + (kLmHPer * wave + j) * 64 * 8), 16, 0,
          0);
    }
  };
  // The weight loads are inline asm and their waits explicit.  Left to the
  // compiler, the wait for a ring register loaded in an earlier trip of the
  // block loop below drains every load in flight, the prefetches just issued
  // included: once per trip the weights' two-block lead collapses (310 vs
  // 284 us per launch at M = 320, D = 4096, V = 128256).  The compiler sees
  // each asm output as written at once, so no register of the ring may look
  // dead while its load flies (see the final drain), and the block loop must
  // move no registers: a move of a ring register would copy a value still in
  // flight.  A CPU test compiles this file and checks the loop for moves.
  auto load_w = [&](int k0, lm_u32x4* w) {
    const bf16_t* src = wbase + (size_t)(k0 / kLmKB) * kLmPackBlock;
#define SPECV_LDW(i, off) \
  asm volatile("global_load_dwordx4 %0, %1, off offset:" #off : "=v"(w[i]) : "v"(src))
    SPECV_LDW(0, 0); SPECV_LDW(1, 1024); SPECV_LDW(2, 2048); SPECV_LDW(3, 3072);
#undef SPECV_LDW
  };

  lm_f32x16 acc[kLmMTiles];
#pragma unroll
  for (int t = 0; t < kLmMTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  // B fragment of tile t, step s: row 32 t + l32, piece 4 h + s
  int boff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) boff[s] = (((4 * h + s) ^ ((l32 >> 1) & 7)) * 8);   // 32 t: no effect

  const int nkb = D / kLmKB;
  lm_u32x4 wr0[4], wr1[4], wr2[4];                   // weight ring: blocks kb, kb+1, kb+2
  const int klast = (nkb - 1) * kLmKB;
  stage_h(0, lds0);
  load_w(0, wr0);
  stage_h(min(kLmKB, klast), lds1);
  load_w(min(kLmKB, klast), wr1);
  __builtin_amdgcn_s_waitcnt(kWaitVm13);             // block 0 staged: 13 younger loads may fly
  __builtin_amdgcn_s_barrier();

  // One k block: stage the hidden block and request the weights two blocks
  // ahead, multiply, then wait for the next block's staging only and meet.
  // The prefetches are unconditional (past the last block they repeat it:
  // valid addresses, unused data), so the count of loads in flight is the
  // same at every block boundary and the compiler's waits stay exact.
  auto block = [&](int kb, lm_u32x4* wa, lm_u32x4* w2, const bf16_t* cur, bf16_t* next) {
    stage_h(min((kb + 2) * kLmKB, klast), next);
    asm volatile("" ::: "memory");                   // keep the staging loads first in the count
    load_w(min((kb + 2) * kLmKB, klast), w2);
    // This block's weights (loaded two blocks ago) have landed once at most
    // 18 younger loads fly: the staging and weights of blocks kb + 1 and
    // kb + 2.  The wait takes the ring registers as in-out operands, so no
    // MFMA reading them can move above it.
    asm volatile("s_waitcnt vmcnt(18)" : "+v"(wa[0]), "+v"(wa[1]), "+v"(wa[2]), "+v"(wa[3]));
    // The fragment reads are inline ds_read_b128 with explicit LDS waits: the
    // compiler cannot tell them from the staging DMA into the other buffer
    // and would otherwise wait for every load, weights included, before the
    // first read.  They are software-pipelined: the next pair of fragments is
    // requested before the current pair's MFMAs, and the wait that releases a
    // pair takes its registers as in-out operands, so no MFMA can move ahead
    // of it.  The block's own staging completed before the last barrier.
    const uint32_t hbase = (uint32_t)(uintptr_t)(cur + l32 * kLmKB);
    uint32_t addr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) addr[s] = hbase + 2 * boff[s];
    lm_u32x4 f0[2], f1[2];                           // the two pair buffers
    constexpr int kTP = kLmMTiles / 2;               // tile pairs per step
#define SPECV_LDS_READ2(dst, q)                                                              \
  asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4"             \
               : "=&v"(dst[0]), "=&v"(dst[1])                                                  \
               : "v"(addr[(q) / kTP]), "i"(((q) % kTP) * 2 * 32 * kLmKB * 2),                  \
                 "i"((((q) % kTP) * 2 + 1) * 32 * kLmKB * 2))
#define SPECV_PAIR(q, cf, nf, WAITN)                                                         \
  {                                                                                          \
    if ((q) + 1 < 4 * kTP) SPECV_LDS_READ2(nf, (q) + 1 < 4 * kTP ? (q) + 1 : 0);              \
    asm volatile("s_waitcnt lgkmcnt(" #WAITN ")" : "+v"(cf[0]), "+v"(cf[1]));               \
    const lm_bf16x8 a_ = as_bf16x8(wa[(q) / kTP]);                                          \
    const int t_ = ((q) % kTP) * 2;                                                          \
    acc[t_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, as_bf16x8(cf[0]), acc[t_], 0, 0, 0); \
    acc[t_ + 1] =                                                                            \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, as_bf16x8(cf[1]), acc[t_ + 1], 0, 0, 0);  \
  }
    SPECV_LDS_READ2(f0, 0);
    SPECV_PAIR(0, f0, f1, 2) SPECV_PAIR(1, f1, f0, 2) SPECV_PAIR(2, f0, f1, 2)
    SPECV_PAIR(3, f1, f0, 2) SPECV_PAIR(4, f0, f1, 2) SPECV_PAIR(5, f1, f0, 2)
    SPECV_PAIR(6, f0, f1, 2) SPECV_PAIR(7, f1, f0, 2) SPECV_PAIR(8, f0, f1, 2)
    SPECV_PAIR(9, f1, f0, 2) SPECV_PAIR(10, f0, f1, 2) SPECV_PAIR(11, f1, f0, 2)
    SPECV_PAIR(12, f0, f1, 2) SPECV_PAIR(13, f1, f0, 2) SPECV_PAIR(14, f0, f1, 2)
    SPECV_PAIR(15, f1, f0, 2) SPECV_PAIR(16, f0, f1, 2) SPECV_PAIR(17, f1, f0, 2)
    SPECV_PAIR(18, f0, f1, 2) SPECV_PAIR(19, f1, f0, 0)
#undef SPECV_PAIR
#undef SPECV_LDS_READ2
    // Meet: block kb + 1 is in LDS (its 5 staging loads are older than the
    // 13 issued since: weights kb + 1, staging and weights kb + 2, which stay
    // in flight), and every wave's reads of this block's buffer have returned
    // (its MFMAs consumed them), so the staging issued in the next block may
    // overwrite it.  A bare barrier: the workgroup fences of __syncthreads
    // would also wait for the weight loads.
    __builtin_amdgcn_s_waitcnt(kWaitVm13);
    __builtin_amdgcn_s_barrier();
  };
  // three blocks per trip: the weight ring and the LDS buffers (three each)
  // index statically, so the compiler sees which buffer each access touches
  for (int kb = 0; kb < nkb; kb += 3) {
    block(kb, wr0, wr2, lds0, lds2);
    if (kb + 1 < nkb) block(kb + 1, wr1, wr0, lds1, lds0);
    if (kb + 2 < nkb) block(kb + 2, wr2, wr1, lds2, lds1);
  }
  // the last blocks' repeated prefetches are still landing: drain them before
  // the epilogue reuses LDS
  // The ring registers stay live until every load has landed: the
  // prefetches past the last block are never read, and a register the
  // compiler took for dead could be reused while its load is still in flight.
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(wr0[0]), "+v"(wr0[1]), "+v"(wr0[2]), "+v"(wr0[3]), "+v"(wr1[0]),
                 "+v"(wr1[1]), "+v"(wr1[2]), "+v"(wr1[3]), "+v"(wr2[0]), "+v"(wr2[1]),
                 "+v"(wr2[2]), "+v"(wr2[3]));
  __builtin_amdgcn_s_barrier();

  // Epilogue.  acc[t][r] is logit (row m0 + 32 t + l32, id vbase + vof(r)).
  // A lane holds one row, so its own stores would touch 32 rows 2 V bytes
  // apart: 64 cache lines per store instruction (the logit stores cost 16-26
  // us per launch at M = 320, D = 4096, V = 128256).  When every row starts
  // 16-byte aligned, each half of the row block (160 rows x 256 ids) goes
  // through LDS instead and the workgroup stores whole 512-byte row segments
  // (~11 us less per launch).  Rows are padded to 264 ids: 16-byte aligned
  // for the reads, at most 2-way bank conflicts for the writes.
  // The indices are derived afresh from the thread and block ids: values kept
  // live across the block loop for the epilogue made the register allocator
  // move ring registers inside the loop, copying weights still in flight.
  int e_tid = threadIdx.x, e_bid = blockIdx.x;
  asm volatile("" : "+v"(e_tid), "+s"(e_bid));
  const int e_lane = e_tid % kWave;
  const int e_wave = __builtin_amdgcn_readfirstlane(e_tid / kWave);
  const int e_h = e_lane / 32, e_l32 = e_lane % 32;
  const int e_tile = e_bid % ntile, e_m0 = (e_bid / ntile) * kLmRows;
  float2* red = reinterpret_cast<float2*>(lds + kLmTrElems);   // [kLmWaves][kLmRows]
  bf16_t* tr = lds;                                            // [kLmRows / 2][kLmTrStride]
  const int vbase = e_tile * kLmVocab + e_wave * 32 + 4 * e_h;
  const bool rows16 = (V & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  // 8-byte stores need every row to start 8-byte aligned
  const bool vec_ok = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
#pragma unroll
  for (int t = 0; t < kLmMTiles; ++t) {
    const int m = e_m0 + t * 32 + e_l32;
    float z[16];
    uint32_t zb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      zb[r] = bf16_rne_bits(acc[t][r]);
      z[r] = __uint_as_float(zb[r] << 16);
    }
    // ids of register r: vbase + 8 (r / 4) + r % 4: four runs of four
    if (rows16) {
      bf16_t* trow =
          tr + ((t % (kLmMTiles / 2)) * 32 + e_l32) * kLmTrStride + e_wave * 32 + 4 * e_h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 pk;
        pk.x = zb[4 * q] | (zb[4 * q + 1] << 16);
        pk.y = zb[4 * q + 2] | (zb[4 * q + 3] << 16);
        *reinterpret_cast<uint2*>(trow + 8 * q) = pk;
      }
    } else if (m < M) {
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
    if (e_h == 0) red[e_wave * kLmRows + t * 32 + e_l32] = make_float2(mx, s);
    if (rows16 && t % (kLmMTiles / 2) == kLmMTiles / 2 - 1) {
      // a half is in LDS: store its rows, 16 bytes per lane, 32 lanes a row
      __syncthreads();
      const int r0 = e_m0 + (t / (kLmMTiles / 2)) * (kLmRows / 2);
      const int vend = min(kLmVocab, V - e_tile * kLmVocab);   // a multiple of 8
#pragma unroll
      for (int i = 0; i < kLmTrPieces / kLmThreads; ++i) {
        const int p = threadIdx.x + i * kLmThreads;
        const int lr = p / 32, c8 = (p % 32) * 8;
        if (r0 + lr < M && c8 < vend) {
          const uint4 v = *reinterpret_cast<const uint4*>(tr + lr * kLmTrStride + c8);
          *reinterpret_cast<uint4*>(out + (size_t)(r0 + lr) * V + e_tile * kLmVocab + c8) = v;
        }
      }
      __syncthreads();                               // the next half overwrites tr
    }
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

// Weight repack, one thread per 16-byte piece of the packed matrix (the
// layout described at the top of this file).
__global__ __launch_bounds__(256) void lm_head_pack_kernel(const bf16_t* __restrict__ W,
                                                           bf16_t* __restrict__ P, int V, int D,
                                                           size_t pieces) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const int nkb = D / kLmKB;
  const int lane = (int)(i % kWave);
  size_t r = i / kWave;
  const int s = (int)(r % 4);
  r /= 4;
  const int group = (int)(r % kLmPackGroups);
  r /= kLmPackGroups;
  const int kb = (int)(r % nkb);
  const size_t tile = r / nkb;
  const size_t v = tile * kLmPackVocab + group * 32 + lane % 32;
  const int k = kb * kLmKB + 32 * (lane / 32) + 8 * s;
  uint4 val = make_uint4(0u, 0u, 0u, 0u);
  if (v < (size_t)V) val = *reinterpret_cast<const uint4*>(W + v * D + k);
  *reinterpret_cast<uint4*>(P + i * 8) = val;
}

int lm_head_tiles(int V) { return (V + kLmVocab - 1) / kLmVocab; }
size_t lm_head_packed_elems(int V, int D) {
  return (size_t)((V + kLmPackVocab - 1) / kLmPackVocab) * kLmPackVocab * D;
}

hipError_t launch_lm_head_pack(const void* weight, void* packed, int V, int D,
                               hipStream_t stream) {
  if (D % kLmKB != 0) return hipErrorInvalidConfiguration;
  const size_t pieces = lm_head_packed_elems(V, D) / 8;
  const size_t blocks = (pieces + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  lm_head_pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      static_cast<const bf16_t*>(weight), static_cast<bf16_t*>(packed), V, D, pieces);
  return hipGetLastError();
}
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
