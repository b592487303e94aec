// Device helpers of the blocked Walsh-Hadamard transform and of the activation
// record that feeds the sign-plane MFMA GEMV (shared by the rotation kernels and
// the fused routing launch).
//
// Rotation: DeepSeek-V4-Flash GALE 1-bit model card, "What is in the pack" (signs
// stored under a blocked FWHT-1024 rotation); the DeepSeek-V4-Pro GALE page
// (serving options, the butterfly FWHT) computes it as a single-kernel butterfly.
// One wavefront transforms one 1024-block entirely in registers: each lane holds
// 16 consecutive elements, the four butterfly stages over the element bits run
// in-lane and the six stages over the lane bits exchange values across lanes.
// H is normalised by 1/32 (orthonormal, H.H = I).
#pragma once
#include "gale_internal.h"
#include "gale_lanes.h"

namespace gale {

__device__ __forceinline__ float load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == GALE_F16) return __half2float(reinterpret_cast<const __half*>(base)[i]);
  return reinterpret_cast<const float*>(base)[i];
}

// Load 16 consecutive elements [16 l, 16 l + 16) of a 1024-block.
__device__ __forceinline__ void load16(const void* blk, int dtype, int lane, float v[16]) {
  if (dtype == GALE_F16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(blk) + 16 * lane);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __half2 h2 = *reinterpret_cast<__half2*>(&w[i]);
      v[2 * i] = __low2float(h2);
      v[2 * i + 1] = __high2float(h2);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(blk) + 16 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
}

__device__ __forceinline__ void store16(void* blk, int dtype, int lane, const float v[16]) {
  if (dtype == GALE_F16) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __half2 h2 = __floats2half2_rn(v[2 * i], v[2 * i + 1]);
      w[i] = *reinterpret_cast<uint32_t*>(&h2);
    }
    uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<__half*>(blk) + 16 * lane);
    p[0] = make_uint4(w[0], w[1], w[2], w[3]);
    p[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(blk) + 16 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

// One butterfly stage over lane bit B: with a the lower lane's value and b the upper
// lane's, the lower lane becomes a + b and the upper lane a - b, each as one fused
// multiply-add by +-1 of the own value onto the partner's (exact multiply, one rounding:
// the same result as the separate add or subtract).
template <int B>
__device__ __forceinline__ void fwht_lane_stage(float v[16], int lane) {
  const float sgn = (lane & B) != 0 ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float u = lane_xor<B>(v[e]);
    v[e] = fmaf(sgn, v[e], u);
  }
}

// In-place normalised Walsh-Hadamard transform of the wavefront's 1024-block.
__device__ __forceinline__ void fwht1024_wave(float v[16], int lane) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if ((e & h) == 0) {
        float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  fwht_lane_stage<1>(v, lane);
  fwht_lane_stage<2>(v, lane);
  fwht_lane_stage<4>(v, lane);
  fwht_lane_stage<8>(v, lane);
  fwht_lane_stage<16>(v, lane);
  fwht_lane_stage<32>(v, lane);
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] *= 0.03125f;
}

// ---------------------------------------------------------------------------
// Activation preparation (one wavefront per (vector, 1024-chunk)):
//   x~ = H x (skipped for pre-rotated input), stored in fp32 for the outlier pass;
//   X = x~ * 2^p with p chosen so that max |X| lies in [128, 256) (well inside
//   e4m3's 448), split into four e4m3 terms X = t0 + t1 + t2 + t3 by repeated
//   round-to-nearest on the residual.  Each term carries ~4 significant bits, so
//   the split is exact to about 2^-16 of each element; the GEMV's MFMA consumes
//   the terms as four rows of its A operand.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

__device__ __forceinline__ void unpack4_fp8(uint32_t p, float* o) {
  o[0] = __builtin_amdgcn_cvt_f32_fp8((int)p, 0);
  o[1] = __builtin_amdgcn_cvt_f32_fp8((int)p, 1);
  o[2] = __builtin_amdgcn_cvt_f32_fp8((int)p, 2);
  o[3] = __builtin_amdgcn_cvt_f32_fp8((int)p, 3);
}

// The record pieces of one lane's 16 elements (x~, four fp8 terms, the chunk
// exponent), from its 16 input values; the wavefront's lanes together hold one
// 1024-chunk.
struct PrepLane {
  float x[16];
  uint32_t t[kTerms][4];
  int p;
};

__device__ __forceinline__ void prep_lane(const float in[16], int lane, bool rotate, PrepLane& o) {
#pragma unroll
  for (int e = 0; e < 16; ++e) o.x[e] = in[e];
  if (rotate) fwht1024_wave(o.x, lane);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(o.x[e]));
  m = fmaxf(m, lane_xor<1>(m));
  m = fmaxf(m, lane_xor<2>(m));
  m = fmaxf(m, lane_xor<4>(m));
  m = fmaxf(m, lane_xor<8>(m));
  m = fmaxf(m, lane_xor<16>(m));
  m = fmaxf(m, lane_xor<32>(m));
  int p = 0;
  if (m > 0.f && m <= 3.0e38f) {
    int ex;
    frexpf(m, &ex);          // m = f 2^ex, f in [0.5, 1)
    p = 8 - ex;              // m 2^p in [128, 256)
  }
  float r[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) r[e] = ldexpf(o.x[e], p);
#pragma unroll
  for (int t = 0; t < kTerms; ++t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o.t[t][q] = pack4_fp8(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
      float back[4];
      unpack4_fp8(o.t[t][q], back);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[4 * q + i] -= back[i];
    }
  }
  o.p = p;
}

// ---------------------------------------------------------------------------
// Coalesced lane layout of a 1024-block for the activation record: every load moves
// 8-byte granules, consecutive lanes on consecutive granules, so one load instruction
// covers 512 contiguous bytes.  The butterfly is a product over the ten index bits, so
// any assignment of index bits to (register, lane) bits computes the same transform; the
// order of the stages, and so the rounding, depends on the layout, which is therefore
// fixed per input dtype and shared by every path that prepares records:
//   fp32: register r of lane l holds element 128 (r >> 1) + 2 l + (r & 1)
//   fp16: register r of lane l holds element 256 (r >> 2) + 4 l + (r & 3)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack_f16x4(uint64_t q, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __half_raw r;
    r.x = (unsigned short)(q >> (16 * e));
    f[e] = __half2float(__half(r));
  }
}

// Plain loads of a block in the coalesced layout of its dtype.
__device__ __forceinline__ void load_block_coalesced(const void* blk, int dtype, int lane, float v[16]) {
  const uint64_t* g = reinterpret_cast<const uint64_t*>(blk);
  if (dtype == GALE_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack_f16x4(g[64 * i + lane], v + 4 * i);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t q = g[64 * j + lane];
      v[2 * j] = __uint_as_float((uint32_t)q);
      v[2 * j + 1] = __uint_as_float((uint32_t)(q >> 32));
    }
  }
}

// Store chunk c of a record from one lane's prepared values, in the layout of `dtype`
// (the dtype the block was loaded in).  rec may be global memory or LDS.
__device__ __forceinline__ void store_record_chunk(const PrepLane& o, int dtype, uint8_t* rec, int K, int c,
                                                   int lane) {
  float* xo = reinterpret_cast<float*>(rec) + (size_t)c * 1024;
  uint8_t* terms = rec + ra_terms_off(K) + (size_t)c * 4 * 1024;
  if (dtype == GALE_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      reinterpret_cast<float4*>(xo)[64 * i + lane] = make_float4(o.x[4 * i], o.x[4 * i + 1], o.x[4 * i + 2],
                                                                 o.x[4 * i + 3]);
#pragma unroll
    for (int t = 0; t < kTerms; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) reinterpret_cast<uint32_t*>(terms + t * 1024)[64 * i + lane] = o.t[t][i];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) reinterpret_cast<float2*>(xo)[64 * j + lane] = make_float2(o.x[2 * j], o.x[2 * j + 1]);
#pragma unroll
    for (int t = 0; t < kTerms; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // the word of registers 4q .. 4q+3 holds elements of granules 2q (low half) and 2q + 1
        reinterpret_cast<uint16_t*>(terms + t * 1024)[64 * (2 * q) + lane] = (uint16_t)(o.t[t][q] & 0xFFFF);
        reinterpret_cast<uint16_t*>(terms + t * 1024)[64 * (2 * q + 1) + lane] = (uint16_t)(o.t[t][q] >> 16);
      }
  }
  if (lane == 0) reinterpret_cast<int32_t*>(rec + ra_p_off(K))[c] = o.p;
}

// One wavefront prepares one (vector, 1024-chunk) of the activation record.
__device__ __forceinline__ void prep_wave(const void* __restrict__ x, int x_dtype, int64_t x_stride, int n_vec,
                                          int K, int rotated, uint8_t* __restrict__ ra, size_t ra_stride,
                                          int64_t wave) {
  const int lane = threadIdx.x & 63;
  const int C = K >> 10;
  if (wave >= (int64_t)n_vec * C) return;
  const int64_t v = wave / C;
  const int c = (int)(wave - v * C);
  const size_t isz = x_dtype == GALE_F16 ? 2 : 4;
  float f[16];
  load_block_coalesced(reinterpret_cast<const char*>(x) + (v * x_stride + (int64_t)c * 1024) * isz, x_dtype, lane, f);
  PrepLane o;
  prep_lane(f, lane, !rotated, o);
  store_record_chunk(o, x_dtype, ra + v * ra_stride, K, c, lane);
}

}  // namespace gale
