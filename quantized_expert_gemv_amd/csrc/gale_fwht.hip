// Blocked Walsh-Hadamard transform (gale_fwht1024) and the activation record that
// feeds the MFMA GEMV (gale_prepare_activations).  The wavefront-level transform
// and the record layout are in gale_rotate.h.
#include "gale_rotate.h"

namespace gale {

// ---------------------------------------------------------------------------
// gale_fwht1024: one wavefront per (vector, block)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) fwht_kernel(const void* __restrict__ x, void* __restrict__ y,
                                                   int64_t n_blocks, int in_dtype, int out_dtype) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (wave >= n_blocks) return;
  const size_t isz = in_dtype == GALE_F16 ? 2 : 4, osz = out_dtype == GALE_F16 ? 2 : 4;
  float v[16];
  load16(reinterpret_cast<const char*>(x) + wave * 1024 * isz, in_dtype, lane, v);
  fwht1024_wave(v, lane);
  store16(reinterpret_cast<char*>(y) + wave * 1024 * osz, out_dtype, lane, v);
}

hipError_t launch_fwht(const void* x, void* y, int64_t n_vec, int len, int in_dtype, int out_dtype,
                       hipStream_t s) {
  const int64_t nb = n_vec * (len / 1024);
  if (nb == 0) return hipSuccess;
  const int64_t grid = (nb + 3) / 4;
  hipLaunchKernelGGL(fwht_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, y, nb, in_dtype, out_dtype);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) prep_kernel(const void* __restrict__ x, int x_dtype, int64_t x_stride,
                                                   int n_vec, int K, int rotated, uint8_t* __restrict__ ra,
                                                   size_t ra_stride, const VecFilter filt) {
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (wave >= (int64_t)n_vec * (K >> 10) || !filter_keep(filt, wave / (K >> 10))) return;
  prep_wave(x, x_dtype, x_stride, n_vec, K, rotated, ra, ra_stride, wave);
}

hipError_t launch_prep(const void* x, int x_dtype, int64_t x_stride, int n_vec, int K, int rotated,
                       uint8_t* ra, size_t ra_stride, hipStream_t s, const VecFilter& filt) {
  const int64_t nw = (int64_t)n_vec * (K / 1024);
  if (nw == 0) return hipSuccess;
  const int64_t grid = (nw + 3) / 4;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, x_dtype, x_stride, n_vec, K,
                     rotated, ra, ra_stride, filt);
  return hipGetLastError();
}

}  // namespace gale
