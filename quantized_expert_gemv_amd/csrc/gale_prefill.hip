// Grouped prefill: the token-sorted (token, slot) pairs of a large batch through
// each expert's FFN.
//
// After routing, the pairs are sorted by expert (stable: token order within an
// expert).  Two ways to run the expert FFNs over them:
//   * work items of at most four pairs of one expert for the sign-plane GEMV,
//     which streams an expert's weights once per four of its tokens (the batched
//     mode of the direct GEMV on the DeepSeek-V4-Pro GALE page, serving options);
//   * a grouped GEMM: tiles of 128 pairs of one expert x 128 weight rows, with the
//     weights dequantized into LDS as fp16 -- every sign bit becomes +-s exactly,
//     and each int4 outlier is added into its weight before the tile is used --
//     and v_mfma_f32_16x16x32_f16 on the fp16 rotated activations.  This is the
//     only dense contraction of the method (DeepSeek-V4-Flash GALE model card,
//     "What is in the pack": the dequantized weight is s (1 - 2 b) plus the
//     outlier r q, which the tile holds rounded to fp16).
#include "gale_internal.h"
#include "gale_rotate.h"
#include "gale_decode.h"

namespace gale {

// ---------------------------------------------------------------------------
// Per-expert lists from the sorted pairs (one workgroup of 512 threads; E <= 512,
// thread e owns expert e): an exclusive scan over experts of each expert's entry
// count, then every thread writes entries i = tid, tid + 512, ..., finding each
// entry's expert by binary search over the scanned starts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int expert_of_entry(const int32_t* s_first, int E, int i) {
  int lo = 0, hi = E;                      // s_first[lo] <= i < s_first[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_first[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

// Exclusive scan of n over the 512 threads into s_first[0..E), the total into s_first[E].
__device__ __forceinline__ void scan_counts(int n, int E, int32_t* s_first, int32_t* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if (tid < E) s_first[tid] = base + v - n;
  if (tid == 0) s_first[E] = total;
  __syncthreads();
}

// Items cover the experts with fewer than max_pairs pairs (all of them when max_pairs
// is INT_MAX); tiles cover the experts with at least min_pairs pairs.
__global__ void __launch_bounds__(512) build_items_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int E, int slots,
                                                          int max_pairs, WorkItem* __restrict__ items,
                                                          int32_t* __restrict__ n_items) {
  __shared__ int32_t s_first[GALE_MAX_EXPERTS + 1];
  __shared__ int32_t s_wave[8];
  const int tid = threadIdx.x;
  int cnt = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  if (cnt >= max_pairs) cnt = 0;
  scan_counts((cnt + slots - 1) / slots, E, s_first, s_wave);
  const int total = s_first[E];
  if (tid == 0) *n_items = total;
  for (int i = tid; i < total; i += blockDim.x) {
    const int e = expert_of_entry(s_first, E, i);
    const int j = i - s_first[e];
    const int c = offsets[e + 1] - offsets[e];
    WorkItem it;
    it.expert = e;
    const int ns = min(slots, c - j * slots);
    it.n_slots = ns;
    it.pad[0] = it.pad[1] = 0;
    const int p0 = offsets[e] + j * slots;
#pragma unroll
    for (int q = 0; q < 4; ++q) it.pair[q] = perm[p0 + (q < ns ? q : 0)];
    items[i] = it;
  }
}

hipError_t launch_build_items(const int32_t* offsets, const int32_t* perm, int n_exp, int slots, int max_pairs,
                              WorkItem* items, int32_t* n_items, hipStream_t s) {
  hipLaunchKernelGGL(build_items_kernel, dim3(1), dim3(512), 0, s, offsets, perm, n_exp, slots, max_pairs, items,
                     n_items);
  return hipGetLastError();
}

__global__ void __launch_bounds__(512) build_tiles_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                          int min_pairs, GemmTile* __restrict__ tiles,
                                                          int32_t* __restrict__ n_tiles) {
  __shared__ int32_t s_first[GALE_MAX_EXPERTS + 1];
  __shared__ int32_t s_wave[8];
  const int tid = threadIdx.x;
  int cnt = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  if (cnt < min_pairs) cnt = 0;
  scan_counts((cnt + bm - 1) / bm, E, s_first, s_wave);
  const int total = s_first[E];
  if (tid == 0) *n_tiles = total;
  for (int i = tid; i < total; i += blockDim.x) {
    const int e = expert_of_entry(s_first, E, i);
    GemmTile t;
    t.expert = e;
    t.m0 = (i - s_first[e]) * bm;
    tiles[i] = t;
  }
}

hipError_t launch_build_tiles(const int32_t* offsets, int n_exp, int min_pairs, GemmTile* tiles, int32_t* n_tiles,
                              hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(512), 0, s, offsets, n_exp, kGemmBM, min_pairs, tiles,
                     n_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotated rows in fp16, each group of 8 columns stored in the order
// (c0, c4, c1, c5, c2, c6, c3, c7): dword j of a group holds columns j and j + 4,
// the element order the GEMM uses for both MFMA operands.  One wavefront per
// (row, 1024-chunk).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) rotate_f16_kernel(const void* __restrict__ x, int x_dtype, int64_t n_rows,
                                                         int K, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int C = K >> 10;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (wave >= n_rows * C) return;
  const int64_t row = wave / C;
  const int c = (int)(wave - row * C);
  const size_t isz = x_dtype == GALE_F16 ? 2 : 4;
  float v[16];
  load16(reinterpret_cast<const char*>(x) + (row * K + (int64_t)c * 1024) * isz, x_dtype, lane, v);
  fwht1024_wave(v, lane);
  uint32_t w[8];
#pragma unroll
  for (int grp = 0; grp < 2; ++grp) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __half2 h2 = __floats2half2_rn(v[8 * grp + j], v[8 * grp + j + 4]);
      w[4 * grp + j] = *reinterpret_cast<uint32_t*>(&h2);
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(out + row * K + (int64_t)c * 1024 + 16 * lane);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

hipError_t launch_rotate_f16(const void* x, int x_dtype, int64_t n_rows, int K, uint16_t* out, hipStream_t s) {
  const int64_t waves = n_rows * (K / 1024);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(rotate_f16_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, x_dtype, n_rows, K,
                     out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM.  Workgroup = (tile of kGemmBM pairs of one expert) x (128 weight rows):
// gate/up takes 64 rows of w1 and the same 64 rows of w3 (SwiGLU in the epilogue),
// down 128 rows of w2.  Four wavefronts in a 2 x 2 arrangement, 64 pairs x 64 rows
// each.  K advances one 128-column scale block at a time through double-buffered
// LDS tiles:
//   A: 128 pairs x 128 fp16 rotated activations (copied from HBM);
//   B: 128 rows x 128 fp16 weights, unpacked from the device sign layout (one
//      shift, AND and XOR per two weights: the sign bit goes straight into the fp16
//      sign of the block scale), then the block's outliers added in place.
// LDS rows are 272 bytes (128 fp16 + 16 pad), so the 16 rows a 16-byte operand
// read touches start on 16 different bank quads.  The outlier entries of the 128
// rows are staged in LDS once per workgroup (columns and int4 values).
// ---------------------------------------------------------------------------
constexpr int kRowBytes = 272;
constexpr int kTileBytes = 128 * kRowBytes;
constexpr int kOutStage = 6144;                       // staged outlier entries per workgroup
constexpr int kStageBytes = 2 * kOutStage + kOutStage + 4 * 132;
constexpr size_t kGemmSmem = 4 * (size_t)kTileBytes + kStageBytes;

struct GemmParams {
  const gale_matrix* table;     // 3 descriptors per expert (w1, w3, w2)
  int sel_a, sel_b;             // matrices of B-tile rows [0, half_rows) and [half_rows, 128)
  int half_rows;                // 64 (gate/up) or 128 (down)
  int K;                        // columns of the weights
  const int32_t* offsets;       // pair offsets per expert [E + 1]
  const int32_t* perm;          // sorted position -> pair
  int top_k;
  const GemmTile* tiles;
  const int32_t* n_tiles;
  const uint16_t* A;            // fp16 rows of K (8-groups permuted)
  int a_by_token;               // A row of sorted position s: perm[s] / top_k (else the pair perm[s])
  float* out;                   // output row of sorted position s: the pair perm[s]
  int out_stride;
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_b;
typedef __attribute__((address_space(3))) u32x4 lds_q;
typedef __attribute__((address_space(3))) unsigned short lds_h;
typedef __attribute__((address_space(3))) signed char lds_i8;
typedef __attribute__((address_space(3))) int lds_i32;

__device__ __forceinline__ v8h as_v8h(const u32x4 v) {
  union { u32x4 u; v8h h; } c;
  c.u = v;
  return c.h;
}

// 16-byte group index of (lane group g, K-step e) inside a 128-column block: the
// columns base(g, e) + i of the fp4 device layout, base = 64 (g & 1) + 16 (g >> 1)
// + 32 (e >> 1) + 8 (e & 1)
__device__ __forceinline__ int group_of(int g, int e) {
  return 8 * (g & 1) + 2 * (g >> 1) + 4 * (e >> 1) + (e & 1);
}

// One B unpack item: a 16-row group of the device sign layout seen by one lane, i.e.
// B-tile row 16 tt + l % 16 and lane group l / 16 (32 of the row's columns per block).
struct BItem {
  int brow, bg;                 // B-tile row, lane group
  int cur, cend;                // outlier cursor and end (staged or CSR index)
  int ncol, nq;                 // column and value of entry cur (column INT_MAX past the end)
  int gsrc;                     // descriptor index of the row's matrix
  float rscale;                 // the row's outlier scale
  const uint32_t* sign;         // the lane's words of chunk 0
  const uint16_t* scale;        // the row's scales of chunk 0
};

// The item's sign words (both halves) and block scales of one 1024-column chunk.
struct ChunkRegs {
  uint4 wlo, whi, sc;
};

__device__ __forceinline__ BItem make_item(const GemmParams& P, int e, int n0, int C, int item, bool staged,
                                           const lds_i32* st_off, const lds_h* st_col, const lds_i8* st_val) {
  BItem b;
  const int tt = item >> 6, l = item & 63;
  const int r0 = 16 * tt;
  b.gsrc = 3 * e + (r0 >= P.half_rows ? P.sel_b : P.sel_a);
  const gale_matrix* M = P.table + b.gsrc;
  const int tg = (n0 + r0 % P.half_rows) >> 4;
  const int nl = l & 15;
  b.brow = r0 + nl;
  b.bg = l >> 4;
  b.sign = M->signs + sign_word_index(tg, 0, C, 0, l, 0);
  b.scale = M->block_scales + scale_index(16 * tg + nl, 0, C);
  const int grow = n0 + (r0 + nl) % P.half_rows;
  __half_raw hr;
  hr.x = M->row_scales[grow];
  b.rscale = __half2float(__half(hr));
  b.cur = staged ? st_off[r0 + nl] : M->row_ptr[grow];
  b.cend = staged ? st_off[r0 + nl + 1] : M->row_ptr[grow + 1];
  b.ncol = 0x7fffffff;
  b.nq = 0;
  if (b.cur < b.cend) {
    if (staged) {
      b.ncol = st_col[b.cur];
      b.nq = st_val[b.cur];
    } else {
      b.ncol = M->out_cols[b.cur];
      b.nq = outlier_value(M->out_vals, b.cur);
    }
  }
  return b;
}

__device__ __forceinline__ ChunkRegs item_load_chunk(const BItem& b, int c) {
  const uint4* w = reinterpret_cast<const uint4*>(b.sign + (int64_t)c * 512);
  ChunkRegs r;
  r.wlo = w[0];
  r.whi = w[64];
  r.sc = *reinterpret_cast<const uint4*>(b.scale + (int64_t)c * 128);
  return r;
}

// Unpack block bd of the item into B-tile rows (Bt), then add the row's outliers of
// the block that fall in the item's columns.
__device__ __forceinline__ void item_store(BItem& b, const ChunkRegs cr, lds_b* Bt, int bd, bool staged,
                                           const lds_h* st_col, const lds_i8* st_val, const gale_matrix* table) {
  const int d = bd & 7, h = d >> 2, p = d & 3;
  // element-wise selects keep the item in registers (a select of two aggregates goes
  // through memory)
  const uint32_t w0 = h ? cr.whi.x : cr.wlo.x, w1 = h ? cr.whi.y : cr.wlo.y;
  const uint32_t w2 = h ? cr.whi.z : cr.wlo.z, w3 = h ? cr.whi.w : cr.wlo.w;
  const uint32_t sw = (d >> 1) == 0 ? cr.sc.x : ((d >> 1) == 1 ? cr.sc.y : ((d >> 1) == 2 ? cr.sc.z : cr.sc.w));
  const uint32_t s16 = (d & 1) ? (sw >> 16) : (sw & 0xFFFFu);
  const uint32_t s_pair = s16 | (s16 << 16);
  lds_b* rowp = Bt + b.brow * kRowBytes;
#pragma unroll
  for (int ee = 0; ee < 4; ++ee) {
    const uint32_t W = ee == 0 ? w0 : (ee == 1 ? w1 : (ee == 2 ? w2 : w3));
    uint32_t dw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[j] = s_pair ^ ((W << (15 - 4 * j - p)) & 0x80008000u);
    *reinterpret_cast<lds_q*>(rowp + 16 * group_of(b.bg, ee)) = u32x4{dw[0], dw[1], dw[2], dw[3]};
  }
  const int k0 = 128 * bd, k1 = k0 + 128;
  // b.ncol / b.nq hold entry b.cur (or a column past the end), so the test never waits
  while (b.ncol < k1) {
    const int col = b.ncol, q = b.nq;
    ++b.cur;
    if (b.cur < b.cend) {
      if (staged) {
        b.ncol = st_col[b.cur];
        b.nq = st_val[b.cur];
      } else {
        const gale_matrix* M = table + b.gsrc;
        b.ncol = M->out_cols[b.cur];
        b.nq = outlier_value(M->out_vals, b.cur);
      }
    } else {
      b.ncol = 0x7fffffff;
    }
    const int cb = col - k0;
    if ((((cb >> 6) & 1) | (((cb >> 4) & 1) << 1)) == b.bg) {
      const int i = cb & 7;
      lds_h* hp = reinterpret_cast<lds_h*>(rowp + 16 * (cb >> 3) + 2 * (2 * (i & 3) + (i >> 2)));
      __half_raw hr;
      hr.x = *hp;
      const float v = __half2float(__half(hr)) + b.rscale * (float)q;
      hr = __half_raw(__float2half_rn(v));
      *hp = hr.x;
    }
  }
}

// A staging: chunk q = tid + 256 j -> row q / 16, 16-byte column group q % 16.
struct AStage {
  int row[8];                   // source row per chunk (-1: beyond the tile's pairs)
  uint4 reg[8];
};

__device__ __forceinline__ void a_load(AStage& a, const uint16_t* A, int K, int bd, int acg) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (a.row[j] >= 0)
      a.reg[j] = *reinterpret_cast<const uint4*>(A + (int64_t)a.row[j] * K + 128 * bd + 8 * acg);
    else
      a.reg[j] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void a_store(const AStage& a, lds_b* At, int tid, int acg) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 4) + 16 * j;
    *reinterpret_cast<lds_q*>(At + r * kRowBytes + 16 * acg) = u32x4{a.reg[j].x, a.reg[j].y, a.reg[j].z, a.reg[j].w};
  }
}

template <bool GATEUP>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(const GemmParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int n_tiles = *P.n_tiles;
  if ((int)blockIdx.y >= n_tiles) return;
  const GemmTile tile = P.tiles[blockIdx.y];
  const int e = tile.expert, m0 = tile.m0;
  const int pair0 = P.offsets[e] + m0;
  const int valid = min(kGemmBM, P.offsets[e + 1] - pair0);
  const int n0 = blockIdx.x * P.half_rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = P.K >> 10;
  const int NB = P.K >> 7;

  lds_b* const base = (lds_b*)smem;
  lds_b* const A0 = base;
  lds_b* const B0 = base + 2 * kTileBytes;
  lds_h* const st_col = reinterpret_cast<lds_h*>(base + 4 * kTileBytes);
  lds_i8* const st_val = reinterpret_cast<lds_i8*>(base + 4 * kTileBytes + 2 * kOutStage);
  lds_i32* const st_off = reinterpret_cast<lds_i32*>(base + 4 * kTileBytes + 3 * kOutStage);

  // ---- stage the outlier entries of the 128 B-tile rows: counts, scan, copy.  B-tile
  //      row r belongs to matrix (r < half_rows ? sel_a : sel_b), global row n0 + r % half_rows.
  {
    int cnt = 0;
    if (tid < 128) {
      const gale_matrix* M = P.table + 3 * e + (tid >= P.half_rows ? P.sel_b : P.sel_a);
      const int g = n0 + tid % P.half_rows;
      cnt = M->row_ptr[g + 1] - M->row_ptr[g];
    }
    // exclusive scan over the first 128 threads (two wavefronts)
    int v = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (tid == 63) st_off[129] = v;       // the first wavefront's total
    __syncthreads();
    if (tid < 128) st_off[tid] = v - cnt + (wave == 1 ? st_off[129] : 0);
    if (tid == 127) st_off[128] = v + st_off[129];
    __syncthreads();
    const int total = st_off[128];
    if (total <= kOutStage) {
      // B-tile rows [0, half_rows) and [half_rows, 128) are consecutive rows of one matrix
      // each, so their entries are (at most) two contiguous CSR ranges: copy them as such
      const gale_matrix* Ma = P.table + 3 * e + P.sel_a;
      const gale_matrix* Mb = P.table + 3 * e + P.sel_b;
      const int na = st_off[P.half_rows];
      const int ba = Ma->row_ptr[n0];
      const int bb = P.half_rows < 128 ? Mb->row_ptr[n0] : 0;
      for (int i = tid; i < total; i += 256) {
        const bool in_a = i < na;
        const gale_matrix* M = in_a ? Ma : Mb;
        const int src = in_a ? ba + i : bb + (i - na);
        st_col[i] = M->out_cols[src];
        st_val[i] = (signed char)outlier_value(M->out_vals, src);
      }
    }
    __syncthreads();
  }
  const bool staged = st_off[128] <= kOutStage;

  AStage as;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 4) + 16 * j;
    int src = -1;
    if (r < valid) {
      const int s = pair0 + r;
      src = P.a_by_token ? P.perm[s] / P.top_k : P.perm[s];
    }
    as.row[j] = src;
  }
  const int acg = tid & 15;

  BItem b0 = make_item(P, e, n0, C, tid, staged, st_off, st_col, st_val);
  BItem b1 = make_item(P, e, n0, C, tid + 256, staged, st_off, st_col, st_val);

  // ---- accumulators: wave (wm, wn) = pairs [64 wm, +64) x B rows [64 wn, +64)
  const int wm = wave & 1, wn = wave >> 1;
  v4f acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) acc[f][nf] = v4f{0.f, 0.f, 0.f, 0.f};
  const int nfrag_m = max(0, min(4, (valid - 64 * wm + 15) >> 4));   // fragments holding pairs
  const int ml = lane & 15, lg = lane >> 4;

  // ---- prologue: block 0
  ChunkRegs c0 = item_load_chunk(b0, 0);
  ChunkRegs c1 = item_load_chunk(b1, 0);
  a_load(as, P.A, P.K, 0, acg);
  a_store(as, A0, tid, acg);
  item_store(b0, c0, B0, 0, staged, st_col, st_val, P.table);
  item_store(b1, c1, B0, 0, staged, st_col, st_val, P.table);
  __syncthreads();

  for (int bd = 0; bd < NB; ++bd) {
    const int buf = bd & 1;
    const bool more = bd + 1 < NB;
    if (more) {
      if (((bd + 1) & 7) == 0) {
        c0 = item_load_chunk(b0, (bd + 1) >> 3);
        c1 = item_load_chunk(b1, (bd + 1) >> 3);
      }
      a_load(as, P.A, P.K, bd + 1, acg);
    }
    const lds_b* At = A0 + buf * kTileBytes;
    const lds_b* Bt = B0 + buf * kTileBytes;
    // four K-steps of 32
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
      const int goff = 16 * group_of(lg, ee);
      v8h bf[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bf[nf] = as_v8h(*reinterpret_cast<const lds_q*>(Bt + (64 * wn + 16 * nf + ml) * kRowBytes + goff));
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (f < nfrag_m) {
          const v8h af = as_v8h(*reinterpret_cast<const lds_q*>(At + (64 * wm + 16 * f + ml) * kRowBytes + goff));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            acc[f][nf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[nf], acc[f][nf], 0, 0, 0);
        }
      }
    }
    if (more) {
      lds_b* Bn = B0 + (buf ^ 1) * kTileBytes;
      a_store(as, A0 + (buf ^ 1) * kTileBytes, tid, acg);
      item_store(b0, c0, Bn, bd + 1, staged, st_col, st_val, P.table);
      item_store(b1, c1, Bn, bd + 1, staged, st_col, st_val, P.table);
    }
    __syncthreads();
  }

  // ---- epilogue.  Fragment layout: lane l, register i -> pair 16 f + 4 (l / 16) + i,
  //      B row 16 nf + l % 16 of the wave's range.
  if (GATEUP) {
    // the waves of w3 rows hand their products to the waves of the same w1 rows
    float* U = reinterpret_cast<float*>(smem);
    if (wn == 1) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          *reinterpret_cast<float4*>(U + ((wm * 16 + f * 4 + nf) * 64 + lane) * 4) =
              make_float4(acc[f][nf][0], acc[f][nf][1], acc[f][nf][2], acc[f][nf][3]);
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const float4 u = *reinterpret_cast<const float4*>(U + ((wm * 16 + f * 4 + nf) * 64 + lane) * 4);
          const float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 64 * wm + 16 * f + 4 * lg + i;
            if (m >= valid) continue;
            const float g = acc[f][nf][i];
            const int s = pair0 + m;
            const int orow = P.perm[s];
            P.out[(int64_t)orow * P.out_stride + n0 + 16 * nf + ml] = g / (1.0f + __expf(-g)) * uu[i];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 64 * wm + 16 * f + 4 * lg + i;
          if (m >= valid) continue;
          const int s = pair0 + m;
          const int orow = P.perm[s];
          P.out[(int64_t)orow * P.out_stride + n0 + 64 * wn + 16 * nf + ml] = acc[f][nf][i];
        }
      }
    }
  }
}

hipError_t launch_grouped_gemm(const gale_matrix* table, int gateup, int rows, int K, const int32_t* offsets,
                               const int32_t* perm, int top_k, const GemmTile* tiles, const int32_t* n_tiles,
                               int max_tiles, const uint16_t* A, float* out, int out_stride, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  GemmParams P;
  P.table = table;
  P.sel_a = gateup ? 0 : 2;
  P.sel_b = gateup ? 1 : 2;
  P.half_rows = gateup ? 64 : 128;
  P.K = K;
  P.offsets = offsets;
  P.perm = perm;
  P.top_k = top_k;
  P.tiles = tiles;
  P.n_tiles = n_tiles;
  P.A = A;
  P.a_by_token = gateup;
  P.out = out;
  P.out_stride = out_stride;
  // the row tiles of one pair tile are neighbours in launch order, so they share its
  // activation rows in the caches
  const dim3 grid((unsigned)(rows / P.half_rows), (unsigned)max_tiles);
  hipError_t err;
  if (gateup) {
    err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kGemmSmem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_kernel<true>, grid, dim3(256), kGemmSmem, s, P);
  } else {
    err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kGemmSmem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_kernel<false>, grid, dim3(256), kGemmSmem, s, P);
  }
  return hipGetLastError();
}

}  // namespace gale
