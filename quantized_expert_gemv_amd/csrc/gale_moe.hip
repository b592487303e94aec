// Routing (top-k with softmax-renormalised weights), stable grouping of the
// (token, slot) pairs by expert, work-item lists for the per-expert GEMVs, and
// the weighted combine.  DeepSeek-V4-Flash GALE model card, "Measured
// performance": each token is served by 6 routed experts per layer (258 = 43 x 6).
//
// Order rule (needed for exact, checkable routing): experts are ranked by logit
// descending, ties to the lower expert index; the k weights are the softmax of
// the k selected logits; the combine sums slots 0..k-1 in that order.
#include "gale_internal.h"
#include "gale_rotate.h"
#include "gale_route.h"

namespace gale {

// Exclusive scan of v over a workgroup of at most 1024 threads; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(x, off, 64);
    if (lane >= off) x += o;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = s_wave[w];
    if (w < wave) base += t;
    all += t;
  }
  *total = all;
  __syncthreads();
  return base + x - v;
}

// ---------------------------------------------------------------------------
// Decode routing: one workgroup does top-k for every token, the counting sort
// and the work-item list (n_tok * k <= 512 pairs).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void route_small_body(const RouteIn& rin, int T, int E, int k,
                                                 int max_slots, int32_t* __restrict__ idx, float* __restrict__ w,
                                                 int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                 WorkItem* __restrict__ items, int32_t* __restrict__ n_items) {
  __shared__ int32_t s_idx[GALE_MAX_DECODE_TOKENS * GALE_MAX_TOPK];
  __shared__ int32_t s_pairs[GALE_MAX_DECODE_TOKENS * GALE_MAX_TOPK];   // pairs grouped by expert
  __shared__ int32_t s_cnt[GALE_MAX_EXPERTS];
  __shared__ int32_t s_fill[GALE_MAX_EXPERTS];
  __shared__ int32_t s_off[GALE_MAX_EXPERTS + 1];
  __shared__ int32_t s_ioff[GALE_MAX_EXPERTS + 1];
  __shared__ int s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
  if (rin.bias == nullptr && rin.fixed == nullptr && E <= 256) {
    if (wave < T) topk_tokens(rin.logits, wave, T, nw, E, k, lane, idx, w, s_idx);
  } else {
    for (int t = wave; t < T; t += nw)
      topk_wave(rin, t, E, k, lane, idx + t * k, w + t * k, s_idx + t * k);
  }
  const int P = T * k;
  __syncthreads();
  // per-expert counts (integer atomics: order-free)
  for (int p = tid; p < P; p += blockDim.x) atomicAdd(&s_cnt[s_idx[p]], 1);
  __syncthreads();
  {
    // blockDim.x == 512 >= E: thread e owns expert e
    const int c = tid < E ? s_cnt[tid] : 0;
    const int ni = (c + max_slots - 1) / max_slots;
    int tot_p = 0, tot_i = 0;
    const int op = block_exclusive_scan(c, s_wave, &tot_p);
    const int oi = block_exclusive_scan(ni, s_wave, &tot_i);
    if (tid < E) { s_off[tid] = op; s_fill[tid] = op; s_ioff[tid] = oi; }
    if (tid == 0) {
      s_off[E] = tot_p;
      s_ioff[E] = tot_i;
      if (n_items) *n_items = tot_i;
    }
  }
  __syncthreads();
  // each pair into its expert's range, in any order
  for (int p = tid; p < P; p += blockDim.x) s_pairs[atomicAdd(&s_fill[s_idx[p]], 1)] = p;
  __syncthreads();
  if (offsets)
    for (int e = tid; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  // stable order: the thread of expert e sorts its few pairs by index (insertion sort),
  // then writes them and its work items
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = s_cnt[e];
    if (c == 0) continue;
    const int base = s_off[e];
    for (int i = 1; i < c; ++i) {
      const int v = s_pairs[base + i];
      int j = i - 1;
      while (j >= 0 && s_pairs[base + j] > v) {
        s_pairs[base + j + 1] = s_pairs[base + j];
        --j;
      }
      s_pairs[base + j + 1] = v;
    }
    int it = s_ioff[e], slot = 0;
    WorkItem cur;
    cur.expert = e;
    cur.n_slots = 0;
    cur.pad[0] = cur.pad[1] = 0;
    for (int i = 0; i < c; ++i) {
      const int p = s_pairs[base + i];
      if (perm) perm[base + i] = p;
      if (!items) continue;
      cur.pair[0] = slot == 0 ? p : cur.pair[0];
      cur.pair[1] = slot == 1 ? p : cur.pair[1];
      cur.pair[2] = slot == 2 ? p : cur.pair[2];
      cur.pair[3] = slot == 3 ? p : cur.pair[3];
      cur.n_slots = ++slot;
      if (slot == max_slots) {
        cur.pair[1] = slot > 1 ? cur.pair[1] : cur.pair[0];
        cur.pair[2] = slot > 2 ? cur.pair[2] : cur.pair[0];
        cur.pair[3] = slot > 3 ? cur.pair[3] : cur.pair[0];
        items[it++] = cur;
        slot = 0;
        cur.n_slots = 0;
      }
    }
    if (items && slot > 0) {
      cur.pair[1] = slot > 1 ? cur.pair[1] : cur.pair[0];
      cur.pair[2] = slot > 2 ? cur.pair[2] : cur.pair[0];
      cur.pair[3] = slot > 3 ? cur.pair[3] : cur.pair[0];
      items[it++] = cur;
    }
  }
}

__global__ void __launch_bounds__(512) route_small_kernel(const RouteIn rin, int T, int E,
                                                          int k, int max_slots, int32_t* __restrict__ idx,
                                                          float* __restrict__ w, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm, WorkItem* __restrict__ items,
                                                          int32_t* __restrict__ n_items) {
  route_small_body(rin, T, E, k, max_slots, idx, w, offsets, perm, items, n_items);
}

// Decode routing and the activation record of the layer input in one launch: the
// two are independent, so workgroup 0 routes while the others prepare x.
__global__ void __launch_bounds__(512) route_prep_kernel(const RouteIn rin, int T, int E, int k,
                                                         int max_slots, int32_t* __restrict__ idx,
                                                         float* __restrict__ w, WorkItem* __restrict__ items,
                                                         int32_t* __restrict__ n_items, const void* __restrict__ x,
                                                         int x_dtype, int K, uint8_t* __restrict__ ra,
                                                         size_t ra_stride) {
  if (blockIdx.x == 0) {
    route_small_body(rin, T, E, k, max_slots, idx, w, nullptr, nullptr, items, n_items);
  } else {
    prep_wave(x, x_dtype, K, T, K, 0, ra, ra_stride,
              (int64_t)(blockIdx.x - 1) * (blockDim.x >> 6) + (threadIdx.x >> 6));
  }
}

hipError_t launch_route_prep(const RouteIn& rin, int n_tok, int n_exp, int k, int32_t* idx, float* w,
                             WorkItem* items, int32_t* n_items, int max_slots, const void* x, int x_dtype, int K,
                             uint8_t* ra, size_t ra_stride, hipStream_t s) {
  // ra == nullptr: routing only (the GEMV rotates and splits x itself)
  const int64_t waves = ra ? (int64_t)n_tok * (K / 1024) : 0;
  const int64_t grid = 1 + (waves + 7) / 8;
  hipLaunchKernelGGL(route_prep_kernel, dim3((unsigned)grid), dim3(512), 0, s, rin, n_tok, n_exp, k, max_slots,
                     idx, w, items, n_items, x, x_dtype, K, ra, ra_stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large-batch routing: chunks of 64 tokens.
//  (1) top-k of each token and per-chunk expert counts,
//  (2) one workgroup scans counts into expert offsets and per-chunk bases,
//  (3) per chunk, the thread of expert e writes its pairs in token order.
// ---------------------------------------------------------------------------
constexpr int kRouteChunk = 64;

__global__ void __launch_bounds__(1024) route_topk_count_kernel(const RouteIn rin, int T, int E,
                                                               int k, int32_t* __restrict__ idx,
                                                               float* __restrict__ w,
                                                               int32_t* __restrict__ chunk_cnt) {
  __shared__ int32_t s_cnt[GALE_MAX_EXPERTS];
  __shared__ int32_t s_idx[kRouteChunk * GALE_MAX_TOPK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x;
  const int t0 = chunk * kRouteChunk;
  const int t1 = min(T, t0 + kRouteChunk);
  for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
  for (int t = t0 + wave; t < t1; t += (int)(blockDim.x >> 6))
    topk_wave(rin, t, E, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k,
              s_idx + (t - t0) * k);
  __syncthreads();
  for (int p = tid; p < (t1 - t0) * k; p += blockDim.x) atomicAdd(&s_cnt[s_idx[p]], 1);
  __syncthreads();
  if (chunk_cnt)
    for (int e = tid; e < E; e += blockDim.x) chunk_cnt[(int64_t)chunk * E + e] = s_cnt[e];
}

__global__ void __launch_bounds__(512) route_scan_kernel(int n_chunks, int E, int32_t* __restrict__ chunk_cnt,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int s_wave[16];
  const int tid = threadIdx.x;
  // blockDim.x == 512 >= E: thread e owns expert e
  int a = 0;
  if (tid < E) {
    for (int c = 0; c < n_chunks; ++c) {
      const int v = chunk_cnt[(int64_t)c * E + tid];
      chunk_cnt[(int64_t)c * E + tid] = a;   // becomes the chunk's base within expert e
      a += v;
    }
  }
  int total = 0;
  const int off = block_exclusive_scan(a, s_wave, &total);
  if (tid < E) offsets[tid] = off;
  if (tid == 0) offsets[E] = total;
}

__global__ void __launch_bounds__(256) route_scatter_kernel(int T, int E, int k,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm) {
  __shared__ int32_t s_idx[kRouteChunk * GALE_MAX_TOPK];
  const int chunk = blockIdx.x;
  const int t0 = chunk * kRouteChunk;
  const int t1 = min(T, t0 + kRouteChunk);
  const int p0 = t0 * k, np = (t1 - t0) * k;
  for (int p = threadIdx.x; p < np; p += blockDim.x) s_idx[p] = idx[p0 + p];
  for (int p = np + threadIdx.x; p < ((np + 7) & ~7); p += blockDim.x) s_idx[p] = -1;   // pad to 8
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int pos = offsets[e] + chunk_base[(int64_t)chunk * E + e];
    // eight entries per step, read together (broadcast reads: every thread scans the same list)
    for (int p = 0; p < np; p += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = s_idx[p + j];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (v[j] == e) perm[pos++] = p0 + p + j;
    }
  }
}

hipError_t launch_route_small(const RouteIn& rin, int n_tok, int n_exp, int k, int32_t* idx, float* w,
                              int32_t* offsets, int32_t* perm, WorkItem* items, int32_t* n_items,
                              int max_slots, hipStream_t s) {
  hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(512), 0, s, rin, n_tok, n_exp, k, max_slots, idx, w,
                     offsets, perm, items, n_items);
  return hipGetLastError();
}

hipError_t launch_route_large(const RouteIn& rin, int n_tok, int n_exp, int k, int32_t* idx, float* w,
                              int32_t* chunk_cnt, int32_t* offsets, int32_t* perm, hipStream_t s) {
  const int nc = (n_tok + kRouteChunk - 1) / kRouteChunk;
  hipLaunchKernelGGL(route_topk_count_kernel, dim3(nc), dim3(1024), 0, s, rin, n_tok, n_exp, k, idx, w,
                     chunk_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !chunk_cnt) return e;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(512), 0, s, nc, n_exp, chunk_cnt, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (perm) {
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nc), dim3(256), 0, s, n_tok, n_exp, k, idx, chunk_cnt,
                       offsets, perm);
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------------------
// combine: y[t][n] = sum_j w[t][j] * ypairs[t k + j][n], slots in order
// ---------------------------------------------------------------------------
// Four columns per thread: the partial rows (workspace, 16-byte aligned, H % 4 == 0) are read
// as float4.  Each element's sum is the same fp32 sequence as before: fma over the k slots in
// order from 0.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ yp, const float* __restrict__ w,
                                                      int T, int k, int H, void* __restrict__ y, int y_dtype) {
  const int H4 = H >> 2;
  const int64_t total = (int64_t)T * H4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / H4);
    const int n = 4 * (int)(i - (int64_t)t * H4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float wj = w[t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(yp + ((int64_t)t * k + j) * H + n);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    const int64_t o = (int64_t)t * H + n;
    if (y_dtype == GALE_F16) {
      __half* yh = reinterpret_cast<__half*>(y) + o;
      yh[0] = __float2half_rn(acc.x);
      yh[1] = __float2half_rn(acc.y);
      yh[2] = __float2half_rn(acc.z);
      yh[3] = __float2half_rn(acc.w);
    } else {
      float* yf = reinterpret_cast<float*>(y) + o;
      yf[0] = acc.x;
      yf[1] = acc.y;
      yf[2] = acc.z;
      yf[3] = acc.w;
    }
  }
}

hipError_t launch_combine(const float* ypairs, const float* w, int n_tok, int k, int hidden, void* y,
                          int y_dtype, hipStream_t s) {
  const int64_t total = (int64_t)n_tok * (hidden / 4);
  if (total == 0) return hipSuccess;
  int g = (int)std::min<int64_t>((total + 255) / 256, 16384);
  hipLaunchKernelGGL(combine_kernel, dim3(g), dim3(256), 0, s, ypairs, w, n_tok, k, hidden, y, y_dtype);
  return hipGetLastError();
}

__global__ void cast_kernel(const float* __restrict__ src, void* __restrict__ dst, int dtype, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (dtype == GALE_F16) reinterpret_cast<__half*>(dst)[i] = __float2half_rn(src[i]);
    else reinterpret_cast<float*>(dst)[i] = src[i];
  }
}

hipError_t launch_cast(const float* src, void* dst, int dst_dtype, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int g = (int)std::min<int64_t>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(cast_kernel, dim3(g), dim3(256), 0, s, src, dst, dst_dtype, n);
  return hipGetLastError();
}

}  // namespace gale
