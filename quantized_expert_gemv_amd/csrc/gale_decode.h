// Device decode routines of the packed GALE format, shared by the GEMV kernels and
// the bit-exact debug exports so that the checks exercise the kernels' own decode.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gale {

// Bits of scale block d inside a device sign word: bit (8 i + d), i = 0..3.
__host__ __device__ inline uint32_t plane_bits(uint32_t w, int d) {
  return w & (0x01010101u << d);
}

// fp8 e4m3 MFMA operand of plane d: four bytes, one per column 128 d + 4 q + i.
//  d < 7: byte = b << d, the e4m3 pattern of b * 2^e_d (e_d = -9,-8,-7,-6,-5,-3,1);
//         the MFMA's E8M0 B-scale 2^(1 - e_d) turns it into 2 b.
//  d = 7: byte = 0x38 | (b << 7) = (1 - 2 b) * 1.0 (sign form, no scale).
template <int D>
__device__ __forceinline__ uint32_t plane_operand(uint32_t w) {
  if constexpr (D < 7) return w & (0x01010101u << D);
  else return (w & 0x80808080u) | 0x38383838u;
}

// E8M0 exponent byte of plane d's B-scale.
template <int D>
constexpr int plane_scale_e8m0() {
  constexpr int e[7] = {-9, -8, -7, -6, -5, -3, 1};
  if constexpr (D < 7) return 127 + 1 - e[D];
  else return 127;
}

// int4 two's complement outlier value of CSR entry p (low nibble first).
__host__ __device__ inline int outlier_value(const uint8_t* vals, int64_t p) {
  const int byte = vals[p >> 1];
  const int nib = (p & 1) ? (byte >> 4) : (byte & 0xF);
  return nib - ((nib & 8) << 1);
}

}  // namespace gale
