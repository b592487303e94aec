// Device pieces of the sign-plane MFMA GEMV shared by the standalone GEMV
// kernel and the one-launch decode layer: operand construction, the sign pass of
// one row tile, the term reduction, the per-unit load buffers and the
// activation operands.  The arithmetic is described at the top of gale_gemv.hip.
#pragma once
#include "gale_internal.h"
#include "gale_decode.h"

namespace gale {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kColChunks = 2;    // 16-byte chunks of outlier columns per lane (1024 entries per wave)
constexpr int kValChunks = 1;    // 16-byte chunks of outlier values per lane (2048 entries per wave)
constexpr int kWaveOutBytes = 64 * 16 * (kColChunks + kValChunks);
// The same for a staging of OC column chunks (OC * 512 entries per wave)
constexpr int val_chunks(int OC) { return OC / 4 + 1; }   // 2048 entries each, one more for the offset
constexpr int wave_out_bytes(int OC) { return 64 * 16 * (OC + val_chunks(OC)); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  __half_raw r;
  r.x = (unsigned short)bits16;
  return __half2float(__half(r));
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) u32x4 lds_v4;

__device__ __forceinline__ u32x4 to_v4(const uint4 a) { return u32x4{a.x, a.y, a.z, a.w}; }

// 16-byte load at a wave-uniform base plus a 32-bit lane offset
__device__ __forceinline__ uint4 ld16(const char* base, uint32_t off) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(base + off);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// the same for data read exactly once (sign words, block scales, outlier chunks)
__device__ __forceinline__ uint4 ld16_stream(const char* base, uint32_t off) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// fp4 B operand of block D: the four words of its half, masked (the upper four
// dwords of the operand are unused for fp4).
template <int D>
__device__ __forceinline__ v8i plane_vec(const uint32_t w[8]) {
  constexpr int h = D >> 2;
  return v8i{(int)plane_operand<D>(w[4 * h + 0]), (int)plane_operand<D>(w[4 * h + 1]),
             (int)plane_operand<D>(w[4 * h + 2]), (int)plane_operand<D>(w[4 * h + 3]), 0, 0, 0, 0};
}

template <int D>
__device__ __forceinline__ v4f plane_mfma(const v8i& a, const uint32_t w[8], const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, plane_vec<D>(w), c, 0, 4, 0, 127, 0,
                                                          plane_scale_e8m0<D>());
}

// Sum over the four lane groups (the four terms of every token): two row swaps.
__device__ __forceinline__ float term_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ int sel4(int i, int a, int b, int c, int d) {
  return i == 0 ? a : (i == 1 ? b : (i == 2 ? c : d));
}

// Read-only tables are read through the constant address space: scalar loads, which
// complete on their own counter and never make the vector pipeline wait.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_const(const T* p) {
  return (const __attribute__((address_space(4))) T*)(p);
}

// Everything unit u needs from HBM, issued during unit u-1.  OC: outlier column chunks.
template <int R, int OC = kColChunks>
struct UnitBuf {
  uint32_t sw[R][8];     // sign words of the wave's R tiles (its chunk)
  uint32_t sc[R][4];     // 8 fp16 block scales of the lane's row, per tile
  uint4 oc[OC];          // outlier column chunks of the wave's 16 rows
  uint4 ov[val_chunks(OC)];  // outlier value chunks
  int ocf, ovf;          // first chunk index of each (wave-uniform)
  int rp0, rp1;          // CSR range of this thread's row in this unit
  int np0, np1;          // CSR range of this thread's row in the next unit
  uint32_t rsc;          // fp16 row scale of this thread's row
};

struct Act {
  v8i A[8];              // e4m3 terms, one operand per scale block of the chunk
  float S[6][4];         // -sum over each 0/1 block (0, 1, 2, 4, 5, 6), per slot
  int pexp[4];
};

// A operands and exponent of chunk c from an activation record in LDS.
__device__ __forceinline__ void record_activation(const uint8_t* rec, int K, int c, int lane, Act& a) {
  const int nl = lane & 15, g = lane >> 4;
  const int term = nl >> 2;
  const uint8_t* tb = rec + ra_terms_off(K) + ((size_t)c * 4 + term) * 1024 + 32 * g;
#pragma unroll
  for (int d = 0; d < 8; ++d) a.A[d] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  if ((nl & 3) == 0) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(tb + 128 * d);
      const uint4 a1 = *reinterpret_cast<const uint4*>(tb + 128 * d + 16);
      a.A[d] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
  }
  a.pexp[0] = reinterpret_cast<const int32_t*>(rec + ra_p_off(K))[c];
}

// -S per 0/1 block and slot: the MFMA against an all -1.0 operand sums each term row.
template <int NS>
__device__ __forceinline__ void block_sums(Act& a) {
  const v8i neg1 = {(int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8,
                    (int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < 7; ++d) {
    if (d == 3) continue;
    const v4f s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.A[d], neg1, zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < NS; ++i) a.S[d - (d >> 2)][i] = s[i];
  }
}

// One row tile of the sign pass: the eight block products, then the scaled sum.  A 0/1
// block contributes s (S - 2 P) with 2 P its product; a sign block s times its product.
template <int NS>
__device__ __forceinline__ void sign_tile(const Act& a, const uint32_t w[8], const uint32_t sc[4], float* acc) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const v4f d0 = plane_mfma<0>(a.A[0], w, zero);
  const v4f d1 = plane_mfma<1>(a.A[1], w, zero);
  const v4f d2 = plane_mfma<2>(a.A[2], w, zero);
  const v4f d3 = plane_mfma<3>(a.A[3], w, zero);
  const v4f d4 = plane_mfma<4>(a.A[4], w, zero);
  const v4f d5 = plane_mfma<5>(a.A[5], w, zero);
  const v4f d6 = plane_mfma<6>(a.A[6], w, zero);
  const v4f d7 = plane_mfma<7>(a.A[7], w, zero);
  const float s0 = half_bits_to_float(sc[0] & 0xFFFF), s1 = half_bits_to_float(sc[0] >> 16);
  const float s2 = half_bits_to_float(sc[1] & 0xFFFF), s3 = half_bits_to_float(sc[1] >> 16);
  const float s4 = half_bits_to_float(sc[2] & 0xFFFF), s5 = half_bits_to_float(sc[2] >> 16);
  const float s6 = half_bits_to_float(sc[3] & 0xFFFF), s7 = half_bits_to_float(sc[3] >> 16);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float v = -s0 * (d0[i] + a.S[0][i]);
    v = fmaf(-s1, d1[i] + a.S[1][i], v);
    v = fmaf(-s2, d2[i] + a.S[2][i], v);
    v = fmaf(s3, d3[i], v);
    v = fmaf(-s4, d4[i] + a.S[3][i], v);
    v = fmaf(-s5, d5[i] + a.S[4][i], v);
    v = fmaf(-s6, d6[i] + a.S[5][i], v);
    v = fmaf(s7, d7[i], v);
    acc[i] = v;
  }
}

// int4 two's complement value of outlier p from its packed byte
__device__ __forceinline__ float nibble_value(int byte, int p) {
  return (float)(((int)((uint32_t)byte << (28 - 4 * (p & 1)))) >> 28);
}

}  // namespace gale
