// Top-k routing of one token by one wavefront, shared by the routing kernels and
// the one-launch decode layer.
//
// Order rule (needed for exact, checkable routing): experts are ranked by logit
// descending, ties to the lower expert index; the k weights are the softmax of
// the k selected logits.
#pragma once
#include "gale_internal.h"
#include "gale_lanes.h"

namespace gale {

// a ranks before b
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Keep the better of this lane's candidate and the one of lane ^ OFF (OFF = 1, 2, 16,
// 32) or of the mirrored lane (OFF = 8: within 8, 16: within 16; see lane_mirror_u32).
template <int OFF, bool MIRROR = false>
__device__ __forceinline__ void arg_best(float& bv, int& bi) {
  uint32_t ov, oi;
  if constexpr (MIRROR) {
    ov = lane_mirror_u32<OFF>(__float_as_uint(bv));
    oi = lane_mirror_u32<OFF>((uint32_t)bi);
  } else {
    ov = lane_xor_u32<OFF>(__float_as_uint(bv));
    oi = lane_xor_u32<OFF>((uint32_t)bi);
  }
  const bool take = better(__uint_as_float(ov), (int)oi, bv, bi);
  bv = take ? __uint_as_float(ov) : bv;
  bi = take ? (int)oi : bi;
}

// Best (logit, expert) of the wavefront, in every lane: quads, groups of 8 and 16
// through DPP, rows through the permlane swaps.
__device__ __forceinline__ void wave_best(float& bv, int& bi) {
  arg_best<1>(bv, bi);
  arg_best<2>(bv, bi);
  arg_best<8, true>(bv, bi);
  arg_best<16, true>(bv, bi);
  arg_best<16>(bv, bi);
  arg_best<32>(bv, bi);
}

// The best candidate of this lane (experts lane + 64 j, j < NJ) not yet taken.
template <int NJ>
__device__ __forceinline__ void lane_best(const float v[8], int lane, int E, uint32_t taken, float& bv, int& bi) {
  bv = -INFINITY;
  bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    const bool take = e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi);
    bv = take ? v[j] : bv;
    bi = take ? e : bi;
  }
}

template <int NJ>
__device__ __forceinline__ void topk_rounds(const float v[8], int lane, int E, int k, float& m, float& my_v,
                                            int& my_i) {
  uint32_t taken = 0;
  float bv;
  int bi;
  lane_best<NJ>(v, lane, E, taken, bv, bi);
  for (int s = 0; s < k; ++s) {
    float wv = bv;
    int wi = bi;
    wave_best(wv, wi);
    m = s == 0 ? wv : m;
    my_v = lane == s ? wv : my_v;
    my_i = lane == s ? wi : my_i;
    taken |= (wi & 63) == lane ? 1u << (wi >> 6) : 0u;
    lane_best<NJ>(v, lane, E, taken, bv, bi);
  }
}

// Top-k of one token by one wavefront: each lane holds up to 8 logits (E <= 512) and
// keeps its best untaken one; each round takes the best of the wavefront, and the
// lane that owned it moves on to its next best.  Lane s keeps winner s.  The best of
// a set is unique under the order rule, so the pairing of lanes in each round does
// not change the result.
__device__ __forceinline__ void topk_wave(const float* __restrict__ lg, int E, int k, int lane, int32_t* out_idx,
                          float* out_w, int32_t* lds_idx) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? lg[e] : -INFINITY;
  }
  float m = 0.f, my_v = 0.f;
  int my_i = 0;
  if (E <= 256) topk_rounds<4>(v, lane, E, k, m, my_v, my_i);
  else topk_rounds<8>(v, lane, E, k, m, my_v, my_i);
  // softmax of the k selected logits, one slot per lane, summed in slot order
  const float ex = lane < k ? expf(my_v - m) : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < GALE_MAX_TOPK; ++s) {
    const float es = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), s));
    sum += s < k ? es : 0.f;
  }
  if (lane < k) {
    out_idx[lane] = my_i;
    out_w[lane] = ex / sum;
    lds_idx[lane] = my_i;
  }
}

}  // namespace gale
