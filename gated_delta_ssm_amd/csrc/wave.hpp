// wave.hpp -- wave64 reduction helpers for gfx950 (CDNA4).
//
// All sums are xor butterflies: at every step lane l adds lane l^m, so the two
// partners compute a+b and b+a, which IEEE addition makes bitwise equal.  Every
// lane of a group therefore ends with the bitwise-identical total, which the
// recurrence needs (all lanes of a state row must use one delta).
//
// Within a 16-lane DPP row the butterfly uses DPP moves (no LDS crossbar):
//   quad_perm [1,0,3,2]  -> lane ^ 1
//   quad_perm [2,3,0,1]  -> lane ^ 2
//   row_half_mirror      -> lane i <- 7 - i   (pairs the two quads of a half-row)
//   row_mirror           -> lane i <- 15 - i  (pairs the two halves of a row)
// After the quad steps every lane of a quad holds the same value, so the two
// mirror steps act as xor 4 / xor 8 on values.  Across rows (xor 16, xor 32)
// ds_bpermute (__shfl_xor) is used.
//
// Callers must keep every lane of the wave active when they call these.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Sum over aligned groups of WIDTH lanes (8, 16, 32 or 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64, "group width");
  if constexpr (WIDTH == 8) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror: pairs the two quads of 8 lanes
  } else {
    x = sum16(x);
  }
  if constexpr (WIDTH >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (WIDTH >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

}  // namespace gdn
