// Exchange of a 32-bit value with lane (lane ^ OFF) of the wavefront, for the
// constant offsets of butterflies and reductions, without the LDS permute path:
//   1, 2  DPP quad permutations;
//   4     ds_swizzle in bit-mask mode (xor 4 inside each 32-lane half);
//   8     DPP row rotation by 8 (within a 16-lane row, i + 8 mod 16 = i ^ 8);
//   16    v_permlane16_swap: lanes of odd rows receive the even row's values in
//         the first result, lanes of even rows the odd row's in the second;
//   32    v_permlane32_swap: the same between the two 32-lane halves.
// Every result is the partner's value bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gale {

template <int OFF>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "xor offset");
  const int lane = (int)(threadIdx.x & 63);
  if constexpr (OFF == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (OFF == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (OFF == 4) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);               // and 0x1F, xor 4
  } else if constexpr (OFF == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// Value of the mirrored lane for reductions that need no exact xor partner:
// MIRROR 8 maps lane i to 7 - i within each group of 8 (DPP row_half_mirror),
// MIRROR 16 maps i to 15 - i within each row of 16 (DPP row_mirror).  After the
// groups of 4 (resp. 8) agree on a value, one step makes the groups of 8 (16) agree.
template <int MIRROR>
__device__ __forceinline__ uint32_t lane_mirror_u32(uint32_t v) {
  static_assert(MIRROR == 8 || MIRROR == 16, "mirror span");
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MIRROR == 8 ? 0x141 : 0x140, 0xF, 0xF, false);
}

template <int OFF>
__device__ __forceinline__ float lane_xor(float v) {
  return __uint_as_float(lane_xor_u32<OFF>(__float_as_uint(v)));
}

template <int OFF>
__device__ __forceinline__ int lane_xor(int v) {
  return (int)lane_xor_u32<OFF>((uint32_t)v);
}

}  // namespace gale
