// Packing canonical GALE matrices into the wavefront-coalesced device layout, and
// the bit-exact decode checks.  Format: DeepSeek-V4-Flash GALE 1-bit model card,
// "What is in the pack" (sign bit per weight, fp16 scale per 128-weight block,
// int4 outliers with a per-row fp16 scale).  The device layout is described in
// include/gale.h next to gale_matrix.
#include "gale_internal.h"
#include "gale_decode.h"

namespace gale {

// ---------------------------------------------------------------------------
// device pack: one thread per device word / per scale
// ---------------------------------------------------------------------------
__global__ void pack_signs_kernel(int rows, int cols, int n_mat, const uint32_t* __restrict__ cs,
                                  uint32_t* __restrict__ ds) {
  const int C = cols >> 10;
  const int64_t words = (int64_t)rows * (cols >> 5);
  const int64_t total = words * n_mat;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = gid / words;
    int64_t w = gid - m * words;
    const int e = (int)(w & 3); w >>= 2;
    const int l = (int)(w & 63); w >>= 6;
    const int h = (int)(w & 1); w >>= 1;
    const int c = (int)(w % C);
    const int t = (int)(w / C);
    const int n = 16 * t + (l & 15);
    const int g = l >> 4;
    const uint32_t* row = cs + m * words + (int64_t)n * (cols >> 5);
    // word (h, e) holds blocks d = 4 h + p at bits 4 i + p; its eight columns of block d
    // are the contiguous run 128 d + fp4_col(g, e, 0) + i, one byte of a canonical word
    const int base = fp4_col(g, e, 0);
    uint32_t out = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int col = 1024 * c + 128 * (4 * h + p) + base;
      const uint32_t byte = (row[col >> 5] >> (col & 31)) & 0xFFu;
#pragma unroll
      for (int i = 0; i < 8; ++i) out |= ((byte >> i) & 1u) << (4 * i + p);
    }
    ds[gid] = out;
  }
}

__global__ void pack_scales_kernel(int rows, int cols, int n_mat, const uint16_t* __restrict__ cs,
                                   uint16_t* __restrict__ ds) {
  const int C = cols >> 10;
  const int nb = cols >> 7;
  const int64_t per = (int64_t)rows * nb;
  const int64_t total = per * n_mat;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = gid / per;
    int64_t i = gid - m * per;
    const int d = (int)(i & 7); i >>= 3;
    const int r = (int)(i & 15); i >>= 4;
    const int c = (int)(i % C);
    const int t = (int)(i / C);
    const int n = 16 * t + r;
    ds[gid] = cs[m * per + (int64_t)n * nb + 8 * c + d];
  }
}

hipError_t launch_pack(int rows, int cols, int n_mat, const uint32_t* cs, const uint16_t* csc,
                       uint32_t* ds, uint16_t* dsc, hipStream_t s) {
  const int64_t words = (int64_t)rows * (cols >> 5) * n_mat;
  const int64_t scales = (int64_t)rows * (cols >> 7) * n_mat;
  int g1 = (int)std::min<int64_t>((words + 255) / 256, 65536);
  int g2 = (int)std::min<int64_t>((scales + 255) / 256, 65536);
  if (words > 0) {
    hipLaunchKernelGGL(pack_signs_kernel, dim3(g1), dim3(256), 0, s, rows, cols, n_mat, cs, ds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (scales > 0) {
    hipLaunchKernelGGL(pack_scales_kernel, dim3(g2), dim3(256), 0, s, rows, cols, n_mat, csc, dsc);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bit-exact decode checks, using the GEMV kernel's own plane decode
// ---------------------------------------------------------------------------
__global__ void debug_unpack_kernel(int rows, int cols, const uint32_t* __restrict__ ds,
                                    uint32_t* __restrict__ cs) {
  const int C = cols >> 10;
  const int64_t total = (int64_t)rows * (cols >> 5);
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(gid / (cols >> 5));
    const int kw = (int)(gid - (int64_t)n * (cols >> 5));   // = 32 c + 4 d + q
    const int c = kw >> 5, d = (kw >> 2) & 7, q = kw & 3;
    const int t = n >> 4;
    uint32_t out = 0;
    for (int bb = 0; bb < 4; ++bb) {
      // columns 128 d + 32 q + 8 bb + i: fp4 operand dword j, lane group g, nibble i
      const int j = (bb & 1) | ((q & 1) << 1);
      const int g = (q >> 1) | (((bb >> 1) & 1) << 1);
      const uint32_t w = ds[sign_word_index(t, c, C, d >> 2, 16 * g + (n & 15), j)];
      const uint32_t bits = plane_bits(w, d);          // the kernel's block mask, bits at 4 i + d % 4
#pragma unroll
      for (int i = 0; i < 8; ++i) out |= ((bits >> (4 * i + (d & 3))) & 1u) << (8 * bb + i);
    }
    cs[gid] = out;
  }
}

hipError_t launch_debug_unpack(int rows, int cols, const uint32_t* ds, uint32_t* cs, hipStream_t s) {
  const int64_t total = (int64_t)rows * (cols >> 5);
  int g = (int)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(debug_unpack_kernel, dim3(g), dim3(256), 0, s, rows, cols, ds, cs);
  return hipGetLastError();
}

__global__ void debug_outliers_kernel(int rows, int64_t nnz, gale_matrix m, int32_t* ro, int32_t* co,
                                      int32_t* vo) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < nnz;
       p += (int64_t)gridDim.x * blockDim.x) {
    // row of entry p: last n with row_ptr[n] <= p
    int lo = 0, hi = rows;   // invariant row_ptr[lo] <= p < row_ptr[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (m.row_ptr[mid] <= p) lo = mid; else hi = mid;
    }
    if (ro) ro[p] = lo;
    if (co) co[p] = (int32_t)m.out_cols[p];
    if (vo) vo[p] = outlier_value(m.out_vals, p);
  }
}

hipError_t launch_debug_outliers(int rows, int64_t nnz, gale_matrix m, int32_t* r, int32_t* c,
                                 int32_t* v, hipStream_t s) {
  if (nnz <= 0) return hipSuccess;
  int g = (int)std::min<int64_t>((nnz + 255) / 256, 65536);
  hipLaunchKernelGGL(debug_outliers_kernel, dim3(g), dim3(256), 0, s, rows, nnz, m, r, c, v);
  return hipGetLastError();
}

}  // namespace gale

// ---------------------------------------------------------------------------
// host packer (same index map)
// ---------------------------------------------------------------------------
using namespace gale;

extern "C" int gale_pack_host(int32_t rows, int32_t cols, const uint32_t* canon_signs,
                              const uint16_t* canon_scales, uint32_t* dev_signs, uint16_t* dev_scales) {
  if (!canon_signs || !canon_scales || !dev_signs || !dev_scales) {
    set_error("gale_pack_host: NULL pointer");
    return GALE_ERR_NULL;
  }
  if (rows <= 0 || rows % 16 || rows > GALE_MAX_ROWS || cols <= 0 || cols % 1024 || cols > GALE_MAX_COLS) {
    set_error("gale_pack_host: bad shape [%d, %d]", rows, cols);
    return GALE_ERR_SHAPE;
  }
  const int C = cols / 1024;
  const int W = cols / 32;
  for (int64_t i = 0; i < (int64_t)rows * W; ++i) dev_signs[i] = 0;
  for (int n = 0; n < rows; ++n)
    for (int k = 0; k < cols; ++k) {
      uint32_t b = (canon_signs[(int64_t)n * W + (k >> 5)] >> (k & 31)) & 1u;
      int64_t w; int bit;
      sign_position(n, k, C, &w, &bit);
      dev_signs[w] |= b << bit;
    }
  for (int n = 0; n < rows; ++n)
    for (int blk = 0; blk < cols / 128; ++blk)
      dev_scales[scale_index(n, blk, C)] = canon_scales[(int64_t)n * (cols / 128) + blk];
  return GALE_OK;
}

extern "C" int gale_unpack_host(int32_t rows, int32_t cols, const uint32_t* dev_signs,
                                const uint16_t* dev_scales, uint32_t* canon_signs, uint16_t* canon_scales) {
  if (!canon_signs || !canon_scales || !dev_signs || !dev_scales) {
    set_error("gale_unpack_host: NULL pointer");
    return GALE_ERR_NULL;
  }
  if (rows <= 0 || rows % 16 || rows > GALE_MAX_ROWS || cols <= 0 || cols % 1024 || cols > GALE_MAX_COLS) {
    set_error("gale_unpack_host: bad shape [%d, %d]", rows, cols);
    return GALE_ERR_SHAPE;
  }
  const int C = cols / 1024;
  const int W = cols / 32;
  for (int64_t i = 0; i < (int64_t)rows * W; ++i) canon_signs[i] = 0;
  for (int n = 0; n < rows; ++n)
    for (int k = 0; k < cols; ++k) {
      int64_t w; int bit;
      sign_position(n, k, C, &w, &bit);
      uint32_t b = (dev_signs[w] >> bit) & 1u;
      canon_signs[(int64_t)n * W + (k >> 5)] |= b << (k & 31);
    }
  for (int n = 0; n < rows; ++n)
    for (int blk = 0; blk < cols / 128; ++blk)
      canon_scales[(int64_t)n * (cols / 128) + blk] = dev_scales[scale_index(n, blk, C)];
  return GALE_OK;
}
