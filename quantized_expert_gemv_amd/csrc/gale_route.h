// Top-k routing of one token by one wavefront, shared by the routing kernels and
// the one-launch decode layer.
//
// Order rule (needed for exact, checkable routing): experts are ranked by logit
// (plus the selection bias, when given) descending, ties to the lower expert index;
// the k weights are the softmax of the k selected experts' own logits.
#pragma once
#include "gale_internal.h"
#include "gale_lanes.h"

namespace gale {

// Ranking key of (logit v, expert e): larger key = ranks first.  The high word maps the
// float order onto unsigned order (-0 is folded into +0 first, so equal logits stay
// equal); the low word is ~e, so equal logits rank by ascending index.  Key 0 is never
// the key of a candidate and stands for "none".
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u ^= (u >> 31) ? 0xFFFFFFFFu : 0x80000000u;
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float key_logit(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u ^= (u >> 31) ? 0x80000000u : 0xFFFFFFFFu;
  return __uint_as_float(u);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

// Keep the larger of this lane's key and the one of lane ^ OFF (OFF = 1, 2, 16, 32) or
// of the mirrored lane (OFF = 8: within 8, 16: within 16; see lane_mirror_u32).
template <int OFF, bool MIRROR = false>
__device__ __forceinline__ void key_best(uint64_t& k) {
  uint32_t lo, hi;
  if constexpr (MIRROR) {
    lo = lane_mirror_u32<OFF>((uint32_t)k);
    hi = lane_mirror_u32<OFF>((uint32_t)(k >> 32));
  } else {
    lo = lane_xor_u32<OFF>((uint32_t)k);
    hi = lane_xor_u32<OFF>((uint32_t)(k >> 32));
  }
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  k = o > k ? o : k;
}

// Largest key of the wavefront, in every lane: quads, groups of 8 and 16 through DPP,
// rows through the permlane swaps.
__device__ __forceinline__ uint64_t wave_best(uint64_t k) {
  key_best<1>(k);
  key_best<2>(k);
  key_best<8, true>(k);
  key_best<16, true>(k);
  key_best<16>(k);
  key_best<32>(k);
  return k;
}

// Top-k of one token by one wavefront: each lane holds the keys of up to 8 logits
// (E <= 512, experts lane + 64 j) and offers its largest untaken one; each round takes
// the largest of the wavefront, and the lane that owned it zeroes that key.  Lane s
// keeps winner s.  The largest of a set of distinct keys is unique, so the pairing of
// lanes in each round does not change the result.
template <int NJ>
__device__ __forceinline__ void topk_rounds(const float* __restrict__ lg, int E, int k, int lane, float& m,
                                            float& my_v, int& my_i) {
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? rank_key(lg[e], e) : 0;
  }
  uint64_t mk = 0;
  for (int s = 0; s < k; ++s) {
    uint64_t b = key[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) b = key[j] > b ? key[j] : b;
    const uint64_t w = wave_best(b);
    mk = s == 0 ? w : mk;
    my_v = lane == s ? key_logit(w) : my_v;
    my_i = lane == s ? key_expert(w) : my_i;
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = key[j] == w ? 0 : key[j];
  }
  m = key_logit(mk);
}

// Top-k of (logit + bias) for the choice only: keys of the biased values (fp32 sums), the
// winners' own logits for the weights.
template <int NJ>
__device__ __forceinline__ void topk_rounds_biased(const float* __restrict__ lg, const float* __restrict__ bias,
                                                   int E, int k, int lane, int& my_i) {
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? rank_key(lg[e] + bias[e], e) : 0;
  }
  for (int s = 0; s < k; ++s) {
    uint64_t b = key[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) b = key[j] > b ? key[j] : b;
    const uint64_t w = wave_best(b);
    my_i = lane == s ? key_expert(w) : my_i;
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = key[j] == w ? 0 : key[j];
  }
}

// Softmax of the k selected logits (lane s holds slot s: its logit my_v and expert my_i),
// summed in slot order, and the k outputs.
__device__ __forceinline__ void topk_softmax_store(float m, float my_v, int my_i, int k, int lane, int32_t* out_idx,
                                                   float* out_w, int32_t* lds_idx) {
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

__device__ __forceinline__ void topk_wave(const RouteIn& in, int t, int E, int k, int lane, int32_t* out_idx,
                                          float* out_w, int32_t* lds_idx) {
  const float* __restrict__ lg = in.logits + (int64_t)t * E;
  float m = 0.f, my_v = 0.f;
  int my_i = 0;
  if (in.fixed == nullptr && in.bias == nullptr) {
    if (E <= 256) topk_rounds<4>(lg, E, k, lane, m, my_v, my_i);
    else topk_rounds<8>(lg, E, k, lane, m, my_v, my_i);
  } else {
    if (in.fixed != nullptr) {
      // given experts (clamped into range, so a bad table cannot reach past the logits)
      const int e = lane < k ? in.fixed[(int64_t)t * k + lane] : 0;
      my_i = e < 0 ? 0 : (e >= E ? E - 1 : e);
    } else if (E <= 256) {
      topk_rounds_biased<4>(lg, in.bias, E, k, lane, my_i);
    } else {
      topk_rounds_biased<8>(lg, in.bias, E, k, lane, my_i);
    }
    my_v = lane < k ? lg[my_i] : 0.f;
    m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    for (int s = 1; s < k; ++s) m = fmaxf(m, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), s)));
  }
  topk_softmax_store(m, my_v, my_i, k, lane, out_idx, out_w, lds_idx);
}

// Plain top-k of several tokens by one wavefront: each token's logits are loaded one token
// ahead of its selection, so only the first load's latency is exposed (E <= 256).
__device__ __forceinline__ void topk_tokens(const float* __restrict__ logits, int t0, int T, int step, int E,
                                            int k, int lane, int32_t* idx, float* w, int32_t* lds_idx) {
  float v[4], vn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = lane + 64 * j < E ? logits[(int64_t)t0 * E + lane + 64 * j] : 0.f;
  for (int t = t0; t < T; t += step) {
    const int tn = t + step < T ? t + step : t;
#pragma unroll
    for (int j = 0; j < 4; ++j) vn[j] = lane + 64 * j < E ? logits[(int64_t)tn * E + lane + 64 * j] : 0.f;
    uint64_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = lane + 64 * j < E ? rank_key(v[j], lane + 64 * j) : 0;
    float m = 0.f, my_v = 0.f;
    int my_i = 0;
    uint64_t mk = 0;
    for (int s = 0; s < k; ++s) {
      uint64_t b = key[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) b = key[j] > b ? key[j] : b;
      const uint64_t win = wave_best(b);
      mk = s == 0 ? win : mk;
      my_v = lane == s ? key_logit(win) : my_v;
      my_i = lane == s ? key_expert(win) : my_i;
#pragma unroll
      for (int j = 0; j < 4; ++j) key[j] = key[j] == win ? 0 : key[j];
    }
    m = key_logit(mk);
    topk_softmax_store(m, my_v, my_i, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k, lds_idx + t * k);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = vn[j];
  }
}

}  // namespace gale
