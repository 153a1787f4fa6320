// Wave primitives shared by the routing and quantizer kernels (wave64, gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// Exchanges inside rows of 16 lanes go through DPP (no LDS round trip):
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes 1 and 2 apart, the half-row and
// row mirrors pair the two quads of each half and the two halves of each row.
// After the four steps every lane of a row holds the row's reduction; the four
// rows are then combined from one lane each with readlane.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
// The same exchange for patterns that keep every lane inside its row and
// every row enabled: no lane keeps its old value, so the compiler can fold the
// move into the instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ int dpp_row_i32(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_row_f32(float v) {
  return __int_as_float(dpp_row_i32<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

}  // namespace moe
