// Device decode routines of the packed GALE format, shared by the GEMV kernels and
// the bit-exact debug exports so that the checks exercise the kernels' own decode.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gale {

// Bits of scale block d inside one of its device sign words: bit 4 i + (d % 4), i = 0..7.
__host__ __device__ inline uint32_t plane_bits(uint32_t w, int d) {
  return w & (0x11111111u << (d & 3));
}

// fp4 e2m1 MFMA operand dword of block d from one of its words: eight nibbles, one per column.
//  d % 4 < 3: nibble = b << (d % 4), the e2m1 pattern of b * 2^(d % 4 - 1) (0.5, 1, 2);
//             the MFMA's E8M0 B-scale 2^(2 - d % 4) turns it into 2 b;
//  d % 4 = 3: nibble = 0x2 | (b << 3) = (1 - 2 b) * 1.0 (sign form, no scale).
template <int D>
__device__ __forceinline__ uint32_t plane_operand(uint32_t w) {
  if constexpr ((D & 3) < 3) return w & (0x11111111u << (D & 3));
  // (w & 0x88888888) | 0x22222222 in one three-input bit operation: truth table 0xEA
  // is (S0 & S1) | S2 for the index 4 S0 + 2 S1 + S2
  else return __builtin_amdgcn_bitop3_b32(w, 0x88888888u, 0x22222222u, 0xEA);
}

template <int D>
constexpr bool plane_is_binary() { return (D & 3) < 3; }

// E8M0 exponent byte of block d's B-scale.
template <int D>
constexpr int plane_scale_e8m0() {
  if constexpr ((D & 3) < 3) return 127 + 2 - (D & 3);
  else return 127;
}

// int4 two's complement outlier value of CSR entry p (low nibble first).
__host__ __device__ inline int outlier_value(const uint8_t* vals, int64_t p) {
  const int byte = vals[p >> 1];
  const int nib = (p & 1) ? (byte >> 4) : (byte & 0xF);
  return nib - ((nib & 8) << 1);
}

}  // namespace gale
