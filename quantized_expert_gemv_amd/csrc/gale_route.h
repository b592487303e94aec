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

// Order-preserving 32-bit key of a logit (-0 folded into +0, so equal logits stay
// equal); 0 is never the key of a logit and stands for "none" or "taken".
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float key_to_logit(uint32_t u) {
  return __uint_as_float(u ^ ((u >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}

// Largest value of the wavefront, the same in every lane: each row of 16 agrees through
// DPP (quad swaps, then the 8- and 16-lane mirrors), the four rows' maxima on the
// scalar unit.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, lane_xor_u32<1>(v));
  v = max(v, lane_xor_u32<2>(v));
  v = max(v, lane_mirror_u32<8>(v));
  v = max(v, lane_mirror_u32<16>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, lane_xor_u32<1>(v));
  v = min(v, lane_xor_u32<2>(v));
  v = min(v, lane_mirror_u32<8>(v));
  v = min(v, lane_mirror_u32<16>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// The same maximum entirely on the vector unit: the four rows agree through the row-swap
// permutes (rows r and r ^ 1, then r and r ^ 2), with no trip through scalar registers.
__device__ __forceinline__ uint32_t wave_max_u32_v(uint32_t v) {
  v = max(v, lane_xor_u32<1>(v));
  v = max(v, lane_xor_u32<2>(v));
  v = max(v, lane_mirror_u32<8>(v));
  v = max(v, lane_mirror_u32<16>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)b[0], (uint32_t)b[1]);
}
__device__ __forceinline__ uint32_t wave_sum_u32_v(uint32_t v) {
  v += lane_xor_u32<1>(v);
  v += lane_xor_u32<2>(v);
  v += lane_xor_u32<4>(v);
  v += lane_xor_u32<8>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = (uint32_t)a[0] + (uint32_t)a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (uint32_t)b[0] + (uint32_t)b[1];
}

// Top-k when no selected key is tied: round s takes the wavefront maximum m_s of the
// remaining keys and removes every key equal to it, noting s as that key's slot.  When the
// rounds removed exactly k keys in all there was no tie, and m_0 > m_1 > ... is exactly the
// order select_topk makes: the lane holding the key of slot s writes its expert to
// lds_idx[s], and lane s gets slot s (its key, its expert).  Returns false (nothing written)
// when some round met a tie: the caller then runs select_topk.  All on the vector unit.
template <int NJ>
__device__ __forceinline__ bool select_topk_untied(const uint32_t key0[NJ], int k, int lane, int& my_i,
                                                   uint32_t& my_key, uint32_t& top, int32_t* lds_idx) {
  uint32_t key[NJ];
  int slot[NJ];
  uint32_t before = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    key[j] = key0[j];
    slot[j] = -1;
    before += key0[j] == 0u ? 1u : 0u;
  }
  uint32_t mk = 0, mlast = 0;
#pragma unroll
  for (int s = 0; s < GALE_MAX_TOPK; ++s) {
    if (s < k) {
      uint32_t lb = key[0];
#pragma unroll
      for (int j = 1; j < NJ; ++j) lb = max(lb, key[j]);
      const uint32_t m = wave_max_u32_v(lb);
      if (s == 0) top = m;
      mk = lane == s ? m : mk;
      mlast = m;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool t = key[j] == m;
        slot[j] = t ? s : slot[j];
        key[j] = t ? 0u : key[j];
      }
    }
  }
  // keys removed in all: the keys that are 0 now and were not before.  With every round's
  // maximum nonzero (the maxima do not grow: the last one suffices) each round removed at
  // least one key, so k in all means exactly one each; a zero maximum (fewer than k keys)
  // would have matched the absent experts' zero keys, and is refused too.
  uint32_t after = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) after += key[j] == 0u ? 1u : 0u;
  if (mlast == 0u || __builtin_amdgcn_readfirstlane((int)wave_sum_u32_v(after - before)) != k) return false;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (slot[j] >= 0) lds_idx[slot[j]] = lane + 64 * j;
  my_key = mk;
  // one wavefront's LDS accesses complete in order: its reads below see its writes above
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  my_i = lane < k ? lds_idx[lane] : 0;
  return true;
}

// Top-k of the keys of one token by one wavefront: lane l holds the keys of experts
// l + 64 j (key 0: no expert).  Each round takes the largest key, ties to the lowest
// expert index: every lane offers its largest key (its lowest j among equal ones), the
// wavefront maximum m is found, and the winner is the one candidate lane with m -- or,
// when several lanes hold m (equal logits), the lowest expert index among them.  The
// winner's key is then taken.  Lane s keeps winner s (expert and key); top = the first
// winner's key.  The result is the order (key desc, expert asc), which no pairing of
// lanes can change.
template <int NJ>
__device__ __forceinline__ void select_topk(uint32_t key[NJ], int k, int lane, int& my_i, uint32_t& my_key,
                                            uint32_t& top) {
  for (int s = 0; s < k; ++s) {
    uint32_t lb = key[0];
    int lj = 0;
#pragma unroll
    for (int j = 1; j < NJ; ++j) {
      const bool gt = key[j] > lb;
      lb = gt ? key[j] : lb;
      lj = gt ? j : lj;
    }
    const uint32_t m = wave_max_u32(lb);
    const uint64_t cand = __ballot(lb == m);
    int e;
    if (__builtin_popcountll(cand) == 1) {
      const int wl = __builtin_ctzll(cand);
      e = wl + 64 * __builtin_amdgcn_readlane(lj, wl);
    } else {
      e = (int)wave_min_u32(lb == m ? (uint32_t)(lane + 64 * lj) : 0xFFFFFFFFu);
    }
    e = __builtin_amdgcn_readfirstlane(e);
    if (s == 0) top = m;
    my_i = lane == s ? e : my_i;
    my_key = lane == s ? m : my_key;
    const int wl = e & 63, wj = e >> 6;
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = (lane == wl && j == wj) ? 0u : key[j];
  }
}

// Top-k of one token by one wavefront: each lane holds the keys of up to NJ logits
// (experts lane + 64 j); the softmax inputs are the selected logits themselves.
template <int NJ>
__device__ __forceinline__ void topk_rounds(const float* __restrict__ lg, int E, int k, int lane, float& m,
                                            float& my_v, int& my_i, int32_t* lds_idx) {
  uint32_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? logit_key(lg[e]) : 0u;
  }
  uint32_t my_key = 0, top = 0;
  if (!select_topk_untied<NJ>(key, k, lane, my_i, my_key, top, lds_idx))
    select_topk<NJ>(key, k, lane, my_i, my_key, top);
  my_v = key_to_logit(my_key);
  m = key_to_logit(top);
}

// Top-k of (logit + bias) for the choice only: keys of the biased values (fp32 sums), the
// winners' own logits for the weights.
template <int NJ>
__device__ __forceinline__ void topk_rounds_biased(const float* __restrict__ lg, const float* __restrict__ bias,
                                                   int E, int k, int lane, int& my_i) {
  uint32_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? logit_key(lg[e] + bias[e]) : 0u;
  }
  uint32_t my_key = 0, top = 0;
  select_topk<NJ>(key, k, lane, my_i, my_key, top);
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
    if (E <= 256) topk_rounds<4>(lg, E, k, lane, m, my_v, my_i, lds_idx);
    else topk_rounds<8>(lg, E, k, lane, m, my_v, my_i, lds_idx);
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

// Plain top-k of one token from its logits already in registers (v[j]: expert lane + 64 j,
// E <= 256): the same keys and selection as topk_wave.
__device__ __forceinline__ void topk_wave_vals(const float v[4], int E, int k, int lane, int32_t* out_idx,
                                               float* out_w, int32_t* lds_idx) {
  uint32_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) key[j] = lane + 64 * j < E ? logit_key(v[j]) : 0u;
  int my_i = 0;
  uint32_t my_key = 0, top = 0;
  if (!select_topk_untied<4>(key, k, lane, my_i, my_key, top, lds_idx)) select_topk<4>(key, k, lane, my_i, my_key, top);
  topk_softmax_store(key_to_logit(top), key_to_logit(my_key), my_i, k, lane, out_idx, out_w, lds_idx);
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
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = lane + 64 * j < E ? logit_key(v[j]) : 0u;
    int my_i = 0;
    uint32_t my_key = 0, top = 0;
    if (!select_topk_untied<4>(key, k, lane, my_i, my_key, top, lds_idx + t * k))
      select_topk<4>(key, k, lane, my_i, my_key, top);
    const float my_v = key_to_logit(my_key), m = key_to_logit(top);
    topk_softmax_store(m, my_v, my_i, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k, lds_idx + t * k);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = vn[j];
  }
}

}  // namespace gale
