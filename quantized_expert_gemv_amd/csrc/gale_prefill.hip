// Grouped prefill: work items over the token-sorted (token, slot) pairs.
//
// After routing, the pairs of a large batch are sorted by expert (stable: token
// order within an expert).  Each expert's run of pairs is cut into work items of
// at most `slots` pairs; one GEMV work item streams the expert's weights once for
// all of its pairs (DeepSeek-V4-Pro GALE page, serving options: the batched mode
// of the direct GEMV).
#include "gale_internal.h"

namespace gale {

// One workgroup: items per expert, an exclusive scan over experts (E <= 512), then
// each expert's thread writes its items in pair order.
__global__ void __launch_bounds__(512) build_items_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int E, int slots,
                                                          WorkItem* __restrict__ items,
                                                          int32_t* __restrict__ n_items) {
  __shared__ int32_t s_n[GALE_MAX_EXPERTS];
  __shared__ int32_t s_wave[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // blockDim.x == 512 >= E: thread e owns expert e
  const int e = tid;
  const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int n = (cnt + slots - 1) / slots;
  // inclusive scan of n over the workgroup: wave scan, then wave totals
  int v = n;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  const int first = base + v - n;
  if (tid == (int)blockDim.x - 1) *n_items = base + v;
  if (e >= E || cnt == 0) return;
  const int p0 = offsets[e];
  for (int j = 0; j < n; ++j) {
    WorkItem it;
    it.expert = e;
    const int ns = min(slots, cnt - j * slots);
    it.n_slots = ns;
    it.pad[0] = it.pad[1] = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) it.pair[q] = perm[p0 + j * slots + (q < ns ? q : 0)];
    items[first + j] = it;
  }
}

hipError_t launch_build_items(const int32_t* offsets, const int32_t* perm, int n_exp, int slots, WorkItem* items,
                              int32_t* n_items, hipStream_t s) {
  hipLaunchKernelGGL(build_items_kernel, dim3(1), dim3(512), 0, s, offsets, perm, n_exp, slots, items, n_items);
  return hipGetLastError();
}

}  // namespace gale
