// Wave-wide scans, reductions and broadcasts on DPP lane moves and
// v_readlane (wave64): no LDS permute, whose latency (~100 cycles) would sit
// on each of a scan's dependent steps.  Scans shift by 1, 2, 4 and 8 within
// each row of 16 lanes, then add row 15's total into rows 1 and 3, then
// lane 31's into rows 2 and 3; reductions combine within each row of 16
// (quad swaps, half-row and row mirrors) and then the four row results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

// A double moved between lanes by one DPP control (its two 32-bit halves
// each), lanes with no source or outside ROWS reading 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_take(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, true);
  return __hiloint2double(hi, lo);
}

// Inclusive prefix sum over the wave, in lane order, on DPP lane moves alone:
// shifts by 1, 2, 4 and 8 within each row of 16, then row 15's total into
// rows 1 and 3, then lane 31's into rows 2 and 3.  A fixed order of
// additions, so the sums are deterministic.
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_take<0x111, 0xf>(x);                      // row_shr:1
  x += dpp_take<0x112, 0xf>(x);                      // row_shr:2
  x += dpp_take<0x114, 0xf>(x);                      // row_shr:4
  x += dpp_take<0x118, 0xf>(x);                      // row_shr:8
  x += dpp_take<0x142, 0xa>(x);                      // row_bcast:15 into rows 1, 3
  x += dpp_take<0x143, 0xc>(x);                      // row_bcast:31 into rows 2, 3
  return x;
}

// The value of lane l - 1 at lane l, 0 at lane 0 (whole-wave shift).
__device__ __forceinline__ double wave_shr1(double x) { return dpp_take<0x138, 0xf>(x); }

// Lane L's value (L wave-uniform).
__device__ __forceinline__ double lane_value(double x, int L) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), L),
                          __builtin_amdgcn_readlane(__double2loint(x), L));
}
__device__ __forceinline__ int lane_value(int x, int L) { return __builtin_amdgcn_readlane(x, L); }

// 32- and 64-bit integers moved by one DPP control, lanes with no source or
// outside ROWS reading 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_take_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, true);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_take_u64(unsigned long long v) {
  const uint32_t lo = dpp_take_u32<CTRL, ROWS>((uint32_t)v);
  const uint32_t hi = dpp_take_u32<CTRL, ROWS>((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Inclusive prefix sums over the wave (integers: exact in any order).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp_take_u32<0x111, 0xf>(x);
  x += dpp_take_u32<0x112, 0xf>(x);
  x += dpp_take_u32<0x114, 0xf>(x);
  x += dpp_take_u32<0x118, 0xf>(x);
  x += dpp_take_u32<0x142, 0xa>(x);
  x += dpp_take_u32<0x143, 0xc>(x);
  return x;
}
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long x) {
  x += dpp_take_u64<0x111, 0xf>(x);
  x += dpp_take_u64<0x112, 0xf>(x);
  x += dpp_take_u64<0x114, 0xf>(x);
  x += dpp_take_u64<0x118, 0xf>(x);
  x += dpp_take_u64<0x142, 0xa>(x);
  x += dpp_take_u64<0x143, 0xc>(x);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  return (int)wave_incl_scan_u32((uint32_t)x);
}

// Reductions of a 32-bit value over the wave, returned wave-uniform.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false));   // quad [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false));   // quad [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));  // half mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));  // row mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x + y; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x | y; });
}

}  // namespace specv
