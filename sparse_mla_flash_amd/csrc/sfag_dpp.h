// sfag_dpp.h -- reductions over the 16 lanes of a row by DPP moves (gfx950).
//
// Cross-lane shuffles (__shfl_xor) compile to ds_bpermute / ds_swizzle, which occupy the LDS pipe
// and wait for its latency; DPP moves stay in the vector ALU.  A row of 16 lanes is reduced by
// swapping in pairs and in quads, mirroring the half rows and mirroring the row: every lane of
// the row ends with the total.
#pragma once
#include <hip/hip_runtime.h>

namespace sfag {

template <int Ctrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), Ctrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f<kDppMirror>(x));
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x + dpp_f<kDppMirror>(x);
}

// Sum over the four 16-lane rows at the same position (lanes l, l ^ 16, l ^ 32, l ^ 48), by the
// row swaps of v_permlane16_swap (odd rows of one operand with even rows of the other) and
// v_permlane32_swap (upper half with lower half), both VALU: with both operands x, the two
// results of a swap hold the two rows of each pair, and their sum is the pair's sum in every lane.
__device__ __forceinline__ float col4_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace sfag
