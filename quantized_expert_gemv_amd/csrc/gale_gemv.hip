// Direct GEMV out of the packed GALE record on the MI355X matrix cores.
//
// What it computes (DeepSeek-V4-Flash GALE 1-bit model card, "What is in the
// pack"): y[n] = sum_k Wq[n][k] x~[k], x~ = blockdiag(H_1024) x, with
//   Wq[n][k] = s[n][k/128] (1 - 2 b[n][k]) + r[n] q at the row's int4 outliers.
// The DeepSeek-V4-Pro GALE page (serving knobs, DSV4_DIRECT_GEMV) multiplies
// straight out of the packed record with signs, block scales and outliers decoded
// in registers; this kernel keeps that idea and re-plans it for gfx950.
//
// gfx950 plan.  A 1-bit GEMV has ~1 VALU op per weight of budget at HBM speed,
// too little for a per-bit select-and-add.  Instead each sign bit becomes one
// byte of an fp8 MFMA operand with a single AND:
//   * the device layout puts the 4 columns of scale block d that a byte covers
//     at bit position d of the word's four bytes, so (w & 0x01010101 << d) is an
//     fp8 e4m3 operand whose bytes are b * 2^e_d (b = sign bit), and the MFMA's
//     E8M0 B-scale 2^(1 - e_d) makes them exactly 2 b; plane 7 uses the sign
//     form (w & 0x80808080) | 0x38383838 = (1 - 2 b) * 1.0;
//   * the activation enters as A = four e4m3 terms of X = x~ 2^p (rows of A),
//     up to four tokens sharing the weights (so M = 4 terms x 4 tokens);
//   * with C = -sum_k X over the block (one extra MFMA against an all -1 operand),
//     D = -(sum_k (1 - 2 b) X) for planes 0..6 and +sum for plane 7, so
//     y += -/+ s[n][blk] D: one FMA per 16x128 block of a lane's row.
// One v_mfma_scale_f32_16x16x128_f8f6f4 therefore consumes one scale block of
// 16 rows: 2048 weights for 8 ANDs + 1 FMA per lane.
//
// Work split: a workgroup owns `R` row tiles (16 rows each) of one work item
// (a matrix and up to four activation vectors); its NW wavefronts split the
// 1024-column chunks (split-K) and meet in LDS.  Outliers are applied after the
// sign pass by all threads of the workgroup (a few lanes per row, CSR order),
// gathering x~ from the fp32 copy in the activation record.
#include "gale_internal.h"
#include "gale_decode.h"

namespace gale {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  __half_raw r;
  r.x = (unsigned short)bits16;
  return __half2float(__half(r));
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

template <int D>
__device__ __forceinline__ v8i plane_vec(const uint32_t w[8]) {
  v8i b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = (int)plane_operand<D>(w[j]);
  return b;
}

template <int D>
__device__ __forceinline__ v4f plane_mfma(const v8i& a, const uint32_t w[8], const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, plane_vec<D>(w), c, 0, 0, 0, 127, 0,
                                                          plane_scale_e8m0<D>());
}

template <int NS, int D>
__device__ __forceinline__ void plane_step(const v8i* A, const v4f* Cm, const uint32_t w[8], float s,
                                           float* acc) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f r = plane_mfma<D>(A[D], w, D < 7 ? Cm[D] : zero);
  const float sg = D < 7 ? -s : s;
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = fmaf(sg, r[i], acc[i]);
}

struct ItemInfo {
  int mat;
  int nslots;
  int ra_idx[4];
  int out_idx[4];
};

template <int NS>
__device__ __forceinline__ ItemInfo decode_item(const GemvParams& P, int item) {
  ItemInfo it;
  if (P.implicit_items) {
    const int mat = item / P.n_groups;
    const int grp = item - mat * P.n_groups;
    it.mat = mat;
    int ns = P.n_tok - grp * NS;
    it.nslots = ns < NS ? ns : NS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = grp * NS + (i < it.nslots ? i : 0);
      it.ra_idx[i] = (P.x_shared ? 0 : mat * P.n_tok) + tok;
      it.out_idx[i] = mat * P.n_tok + tok;
    }
  } else {
    const WorkItem w = P.items[item];
    it.mat = w.expert;
    it.nslots = w.n_slots < NS ? w.n_slots : NS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = w.pair[i < it.nslots ? i : 0];
      it.ra_idx[i] = pr / P.ra_div;
      it.out_idx[i] = pr;
    }
  }
  return it;
}

// NS: activation vectors per item (1, 2 or 4); R: row tiles per workgroup;
// NW: wavefronts per matrix (split-K); GATEUP: two matrices (w1, w3) and a SwiGLU epilogue.
template <int NS, int R, int NW, bool GATEUP>
__global__ void __launch_bounds__(NW * (GATEUP ? 2 : 1) * 64) gemv_kernel(const GemvParams P) {
  constexpr int HALVES = GATEUP ? 2 : 1;
  constexpr int THREADS = NW * HALVES * 64;
  constexpr int RI = HALVES * R * 16;                 // row instances per workgroup
  // four lanes per row for the outlier pass, whatever the workgroup shape, so that the
  // summation order (and so the result) does not depend on the launch configuration
  constexpr int TPR = 4;
  constexpr int GROUPS = THREADS / TPR;

  __shared__ float red[HALVES][NW][R * 16][NS];
  __shared__ float ored[HALVES][R * 16][NS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = GATEUP ? wave / NW : 0;
  const int wl = wave % NW;
  const int g = lane >> 4, nl = lane & 15;
  const int C = P.cols >> 10;
  const int ntiles = P.rows >> 4;

  const int n_items = P.implicit_items ? P.n_items : *P.n_items_dev;
  const int total = n_items * P.row_groups;

  for (int work = blockIdx.x; work < total; work += gridDim.x) {
    const int item = work / P.row_groups;
    const int rg = work - item * P.row_groups;
    const ItemInfo it = decode_item<NS>(P, item);
    const gale_matrix M = P.table[it.mat * P.mat_stride + (half ? P.sel1 : P.sel0)];

    float rowsum[R][NS];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < NS; ++i) rowsum[r][i] = 0.f;

    for (int c = wl; c < C; c += NW) {
      // ---- sign words and block scales of this wave's R tiles (all loads issued up front)
      uint32_t w[R][8];
      uint4 sc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int tile = rg * R + r;
        if (tile < ntiles) {
          const uint4* sw = reinterpret_cast<const uint4*>(M.signs + sign_word_index(tile, c, C, 0, lane, 0));
          const uint4 lo = sw[0], hi = sw[64];
          w[r][0] = lo.x; w[r][1] = lo.y; w[r][2] = lo.z; w[r][3] = lo.w;
          w[r][4] = hi.x; w[r][5] = hi.y; w[r][6] = hi.z; w[r][7] = hi.w;
          sc[r] = *reinterpret_cast<const uint4*>(M.block_scales + scale_index(16 * tile + nl, 8 * c, C));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[r][j] = 0;
          sc[r] = make_uint4(0, 0, 0, 0);
        }
      }
      // ---- A operand: four e4m3 terms of up to NS activation vectors, 8 planes
      const int term = nl >> 2, slot = nl & 3;
      v8i A[8];
      if (slot < it.nslots) {
        const uint8_t* tb = P.ra + (size_t)it.ra_idx[slot] * P.ra_stride + ra_terms_off(P.cols) +
                            ((size_t)c * 4 + term) * 1024 + 32 * g;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const uint4 a0 = *reinterpret_cast<const uint4*>(tb + 128 * d);
          const uint4 a1 = *reinterpret_cast<const uint4*>(tb + 128 * d + 16);
          A[d] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        }
      } else {
#pragma unroll
        for (int d = 0; d < 8; ++d) A[d] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
      int pexp[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i)
        pexp[i] = i < it.nslots
                      ? reinterpret_cast<const int32_t*>(P.ra + (size_t)it.ra_idx[i] * P.ra_stride + ra_p_off(P.cols))[c]
                      : 0;
      // ---- C operand: -sum over each scale block of each term
      v4f Cm[8];
      {
        const v8i neg1 = {(int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8,
                          (int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8, (int)0xB8B8B8B8};
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 8; ++d)
          Cm[d] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[d], neg1, zero, 0, 0, 0, 127, 0, 127);
      }
      // ---- sign pass
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float acc[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[i] = 0.f;
        const uint32_t s01 = sc[r].x, s23 = sc[r].y, s45 = sc[r].z, s67 = sc[r].w;
        plane_step<NS, 0>(A, Cm, w[r], half_bits_to_float(s01 & 0xFFFF), acc);
        plane_step<NS, 1>(A, Cm, w[r], half_bits_to_float(s01 >> 16), acc);
        plane_step<NS, 2>(A, Cm, w[r], half_bits_to_float(s23 & 0xFFFF), acc);
        plane_step<NS, 3>(A, Cm, w[r], half_bits_to_float(s23 >> 16), acc);
        plane_step<NS, 4>(A, Cm, w[r], half_bits_to_float(s45 & 0xFFFF), acc);
        plane_step<NS, 5>(A, Cm, w[r], half_bits_to_float(s45 >> 16), acc);
        plane_step<NS, 6>(A, Cm, w[r], half_bits_to_float(s67 & 0xFFFF), acc);
        plane_step<NS, 7>(A, Cm, w[r], half_bits_to_float(s67 >> 16), acc);
        // undo 2^p, then sum the four terms (lane groups g = 0..3)
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          float v = ldexpf(acc[i], -pexp[i]);
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);
          rowsum[r][i] += v;
        }
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < NS; ++i) red[half][wl][r * 16 + lane][i] = rowsum[r][i];
    }

    // ---- outliers: TPR threads per row, CSR order, x~ gathered from the fp32 record
    for (int ri = tid / TPR; ri < RI; ri += GROUPS) {
      const int sub = tid % TPR;
      const int hf = ri / (R * 16);
      const int rr = ri - hf * (R * 16);
      const int n = (rg * R + rr / 16) * 16 + (rr & 15);
      float o[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) o[i] = 0.f;
      float rs = 0.f;
      if (n < P.rows) {
        const gale_matrix Mo = P.table[it.mat * P.mat_stride + (hf ? P.sel1 : P.sel0)];
        const int p0 = Mo.row_ptr[n], p1 = Mo.row_ptr[n + 1];
        for (int p = p0 + sub; p < p1; p += TPR) {
          const int col = Mo.out_cols[p];
          const float q = (float)outlier_value(Mo.out_vals, p);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            if (i < it.nslots) {
              const float* xt = reinterpret_cast<const float*>(P.ra + (size_t)it.ra_idx[i] * P.ra_stride);
              o[i] = fmaf(q, xt[col], o[i]);
            }
          }
        }
        rs = half_bits_to_float(Mo.row_scales[n]);
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int off = TPR / 2; off >= 1; off >>= 1) o[i] += __shfl_xor(o[i], off, 64);
      }
      if (sub == 0) {
#pragma unroll
        for (int i = 0; i < NS; ++i) ored[hf][rr][i] = o[i] * rs;
      }
    }
    __syncthreads();

    // ---- final: sum the split-K partials in a fixed order, add outliers, store
    for (int e = tid; e < R * 16 * NS; e += THREADS) {
      const int rr = e / NS, i = e - rr * NS;
      const int n = (rg * R + rr / 16) * 16 + (rr & 15);
      if (n >= P.rows || i >= it.nslots) continue;
      float v[HALVES];
#pragma unroll
      for (int hf = 0; hf < HALVES; ++hf) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) acc += red[hf][q][rr][i];
        v[hf] = acc + ored[hf][rr][i];
      }
      const int64_t off = (int64_t)it.out_idx[i] * P.y_stride + n;
      if (GATEUP) {
        reinterpret_cast<float*>(P.y)[off] = silu_f(v[0]) * v[HALVES - 1];
      } else if (P.y_dtype == GALE_F16) {
        reinterpret_cast<__half*>(P.y)[off] = __float2half_rn(v[0]);
      } else {
        reinterpret_cast<float*>(P.y)[off] = v[0];
      }
    }
    __syncthreads();
  }
}

template <int NS, int R, int NW, bool G>
static hipError_t launch_t(const GemvParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<NS, R, NW, G>), dim3(grid), dim3(NW * (G ? 2 : 1) * 64), 0, s, p);
  return hipGetLastError();
}

template <int NS, int R, bool G>
static hipError_t launch_nw(const GemvParams& p, int grid, hipStream_t s) {
  const int C = p.cols >> 10;
  if (C >= 4) return launch_t<NS, R, 4, G>(p, grid, s);
  if (C >= 2) return launch_t<NS, R, 2, G>(p, grid, s);
  return launch_t<NS, R, 1, G>(p, grid, s);
}

template <int NS, bool G>
static hipError_t launch_r(const GemvParams& p, int tiles, int grid, hipStream_t s) {
  switch (tiles) {
    case 1: return launch_nw<NS, 1, G>(p, grid, s);
    case 2: return launch_nw<NS, 2, G>(p, grid, s);
    case 4: return launch_nw<NS, 4, G>(p, grid, s);
    default: return launch_nw<NS, 8, G>(p, grid, s);
  }
}

hipError_t launch_gemv(const GemvParams& p, int slots, int tiles_per_wg, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (p.gateup) {
    if (slots == 1) return launch_r<1, true>(p, tiles_per_wg, grid, s);
    if (slots == 2) return launch_r<2, true>(p, tiles_per_wg, grid, s);
    return launch_r<4, true>(p, tiles_per_wg, grid, s);
  }
  if (slots == 1) return launch_r<1, false>(p, tiles_per_wg, grid, s);
  if (slots == 2) return launch_r<2, false>(p, tiles_per_wg, grid, s);
  return launch_r<4, false>(p, tiles_per_wg, grid, s);
}

}  // namespace gale
