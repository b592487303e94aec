// Grouped prefill: work items over the token-sorted (token, slot) pairs.
//
// After routing, the pairs of a large batch are sorted by expert (stable: token
// order within an expert).  Each expert's run of pairs is cut into work items of
// at most `slots` pairs; one GEMV work item streams the expert's weights once for
// all of its pairs (DeepSeek-V4-Pro GALE page, serving options: the batched mode
// of the direct GEMV).
#include "gale_internal.h"

namespace gale {

// One workgroup: items per expert and their exclusive scan over experts (E <= 512,
// thread e owns expert e), then every thread writes items i = tid, tid + 512, ...,
// finding each item's expert by binary search over the scanned starts.
__global__ void __launch_bounds__(512) build_items_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int E, int slots,
                                                          WorkItem* __restrict__ items,
                                                          int32_t* __restrict__ n_items) {
  __shared__ int32_t s_first[GALE_MAX_EXPERTS + 1];
  __shared__ int32_t s_off[GALE_MAX_EXPERTS + 1];
  __shared__ int32_t s_wave[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tid;
  const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int n = (cnt + slots - 1) / slots;
  int v = n;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < 8; ++w) {
    if (w < wave) base += s_wave[w];
    total += s_wave[w];
  }
  if (e < E) {
    s_first[e] = base + v - n;
    s_off[e] = offsets[e];
  }
  if (tid == 0) {
    s_first[E] = total;
    *n_items = total;
  }
  __syncthreads();
  for (int i = tid; i < total; i += blockDim.x) {
    // expert of item i: the last e with s_first[e] <= i (experts without items share a start)
    int lo = 0, hi = E;                      // s_first[lo] <= i < s_first[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_first[mid] <= i) lo = mid; else hi = mid;
    }
    const int j = i - s_first[lo];
    const int c = (lo + 1 < E ? s_off[lo + 1] : offsets[E]) - s_off[lo];     // pairs of expert lo
    WorkItem it;
    it.expert = lo;
    const int ns = min(slots, c - j * slots);
    it.n_slots = ns;
    it.pad[0] = it.pad[1] = 0;
    const int p0 = s_off[lo] + j * slots;
#pragma unroll
    for (int q = 0; q < 4; ++q) it.pair[q] = perm[p0 + (q < ns ? q : 0)];
    items[i] = it;
  }
}

hipError_t launch_build_items(const int32_t* offsets, const int32_t* perm, int n_exp, int slots, WorkItem* items,
                              int32_t* n_items, hipStream_t s) {
  hipLaunchKernelGGL(build_items_kernel, dim3(1), dim3(512), 0, s, offsets, perm, n_exp, slots, items, n_items);
  return hipGetLastError();
}

}  // namespace gale
