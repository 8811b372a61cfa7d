// Wave-wide (64-lane) scans and reductions for gfx950 built from DPP moves:
// row shifts within each 16-lane row, then row broadcasts of lane 15 and
// lane 31 across rows.  Each step is a register move between lanes, with no
// LDS crossbar traffic, so a full scan is six dependent VALU operations.
#pragma once

#include <hip/hip_runtime.h>

namespace sda {

// DPP controls (GFX9 encoding).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

// x + (lane i - shift of the same row, or the broadcast lane), for the rows
// kRowMask selects; lanes with no source lane add 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, kCtrl, kRowMask, 0xF, false);
}

// max(x, the same source lane); lanes with no source lane keep x.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_max(int x) {
  return max(x, __builtin_amdgcn_update_dpp(x, x, kCtrl, kRowMask, 0xF, false));
}

// Inclusive scan of v over the 64 lanes: shifts by 1, 2, 4 and 8 within each
// row of 16, then row 0's total into row 1 and row 2's into row 3, then lane
// 31's sum into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = dpp_add<kDppRowShr1, 0xF>(v);
  v = dpp_add<kDppRowShr2, 0xF>(v);
  v = dpp_add<kDppRowShr4, 0xF>(v);
  v = dpp_add<kDppRowShr8, 0xF>(v);
  v = dpp_add<kDppRowBcast15, 0xA>(v);
  v = dpp_add<kDppRowBcast31, 0xC>(v);
  return v;
}

// Exclusive scan of v over the 64 lanes; `total` gets the sum (uniform).
__device__ __forceinline__ int wave_exclusive_scan(int v, int& total) {
  const int x = wave_inclusive_scan(v);
  total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Sum of v over the 64 lanes (uniform).
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(v), 63);
}

// Maximum of v over the 64 lanes (uniform): the scan's steps with max; lane
// 63 sees every lane.
__device__ __forceinline__ int wave_max(int v) {
  v = dpp_max<kDppRowShr1, 0xF>(v);
  v = dpp_max<kDppRowShr2, 0xF>(v);
  v = dpp_max<kDppRowShr4, 0xF>(v);
  v = dpp_max<kDppRowShr8, 0xF>(v);
  v = dpp_max<kDppRowBcast15, 0xA>(v);
  v = dpp_max<kDppRowBcast31, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace sda
