// Wave-wide scans and broadcasts of doubles on DPP lane moves and
// v_readlane (wave64): no LDS permute, whose latency (~100 cycles) would sit
// on each of a scan's dependent steps.
#pragma once

#include <hip/hip_runtime.h>

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

}  // namespace specv
