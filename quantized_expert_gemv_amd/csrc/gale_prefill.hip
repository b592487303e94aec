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
                                                         int K, uint16_t* __restrict__ out, const VecFilter filt) {
  const int lane = threadIdx.x & 63;
  const int C = K >> 10;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (wave >= n_rows * C) return;
  const int64_t row = wave / C;
  if (!filter_keep(filt, row)) return;
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

hipError_t launch_rotate_f16(const void* x, int x_dtype, int64_t n_rows, int K, uint16_t* out, hipStream_t s,
                             const VecFilter& filt) {
  const int64_t waves = n_rows * (K / 1024);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(rotate_f16_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, x_dtype, n_rows, K,
                     out, filt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM.  Workgroup = (tile of kGemmBM pairs of one expert) x (128 weight rows):
// gate/up takes 64 rows of w1 and the same 64 rows of w3 (SwiGLU in the epilogue),
// down 128 rows of w2.  Eight wavefronts in two roles, two per SIMD: four producers
// load and unpack, four consumers run the products in a 2 x 2 arrangement, 64 pairs x
// 64 rows each, so one role's waits overlap the other's work.  K advances one
// 128-column scale block at a time through double-buffered LDS tiles:
//   A: 128 pairs x 128 fp16 rotated activations (copied from HBM);
//   B: 128 rows x 128 fp16 weights, unpacked from the device sign layout (one
//      shift, AND and XOR per two weights: the sign bit goes straight into the fp16
//      sign of the block scale), then the block's outliers added in place.
// LDS rows are 272 bytes (128 fp16 + 16 pad), so the 16 rows a 16-byte operand
// read touches start on 16 different bank quads.
//
// Outliers.  At the start, the workgroup sorts the outlier entries of its 128 rows
// into buckets of (group of 16 rows, block) in LDS, one 32-bit entry each (column
// within the block, row within the group, int4 value, and the row's fp16 scale).
// The counting tables of the sort live in the second A buffer, which the K loop
// fills only after them.  The wavefront that
// unpacks a group of 16 rows also patches them: after its sign stores, lane i adds
// the bucket's entry i into its weight (LDS operations of one wavefront complete in
// order, so no barrier is needed).  Rows whose entries exceed the staging space,
// or K beyond the bucket table, take a per-lane walk over the CSR lists in HBM.
// ---------------------------------------------------------------------------
constexpr int kRowBytes = 272;
constexpr int kTileBytes = 128 * kRowBytes;
constexpr int kOutStage = 6000;                       // staged outlier entries per workgroup
constexpr int kStageBlocks = 56;                      // bucket table: K <= 7168
constexpr int kBuckets = 8 * kStageBlocks;
// entries u32 [kOutStage]; eight i32 for the total and the scan; output rows i32 [128].
// In the second A buffer during the sort: bucket starts i32 [kBuckets + 1], fill cursors
// i32 [kBuckets].
constexpr int kStageBytes = 4 * kOutStage + 4 * 8 + 4 * 128;
static_assert(4 * (2 * kBuckets + 1) <= kTileBytes, "sort tables fit the second A buffer");
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
// fp16 weights patched in place: may alias the 16-byte sign stores of the same tile, so the
// compiler keeps each patch after the stores before it
typedef __attribute__((address_space(3), may_alias)) unsigned short lds_h_alias;
typedef __attribute__((address_space(3))) int lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

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

// Byte offset in a B tile of (row, column cb of the block): the 16-byte group of cb
// holds its 8 columns in the order (c0, c4, c1, c5, c2, c6, c3, c7).
__device__ __forceinline__ int b_offset(int row, int cb) {
  return row * kRowBytes + 16 * (cb >> 3) + 2 * (2 * (cb & 3) + ((cb >> 2) & 1));
}

// One B unpack item: a 16-row group of the device sign layout seen by one lane, i.e.
// B-tile row 16 tt + l % 16 and lane group l / 16 (32 of the row's columns per block).
struct BItem {
  int brow, bg;                 // B-tile row, lane group
  int cur, cend;                // unstaged outliers: CSR cursor and end
  int ncol, nq;                 // column and value of entry cur (column INT_MAX past the end)
  int gsrc;                     // descriptor index of the row's matrix
  float rscale;                 // the row's outlier scale
  const uint32_t* sign;         // the lane's words of chunk 0
  const uint16_t* scale;        // the row's scales of chunk 0
};

// Global-memory views of device pointers: a load through them is a global load, which
// only the vector-memory counter tracks (a load through a generic pointer is a flat
// load, and every wait for LDS results would wait for it as well).  The 16-byte load
// goes through the builtin vector type: uint4's copy constructor takes a generic
// reference and would turn it back into a flat load.
typedef const __attribute__((address_space(1))) u32x4 g_u4;
typedef const __attribute__((address_space(1))) uint32_t g_u32;

__device__ __forceinline__ uint4 gload16(const void* p) {
  const u32x4 v = *(g_u4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t gload4(const void* p) { return *(g_u32*)p; }

__device__ __forceinline__ BItem make_item(const GemmParams& P, int e, int n0, int C, int item) {
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
  b.cur = b.cend = 0;
  b.ncol = 0x7fffffff;
  b.nq = 0;
  b.rscale = 0.f;
  return b;
}

// Unstaged outliers: the item's cursor on its row's CSR list.
__device__ __forceinline__ void item_walk_init(const GemmParams& P, int e, int n0, BItem& b) {
  const gale_matrix* M = P.table + b.gsrc;
  const int grow = n0 + b.brow % P.half_rows;
  __half_raw hr;
  hr.x = M->row_scales[grow];
  b.rscale = __half2float(__half(hr));
  b.cur = M->row_ptr[grow];
  b.cend = M->row_ptr[grow + 1];
  if (b.cur < b.cend) {
    b.ncol = M->out_cols[b.cur];
    b.nq = outlier_value(M->out_vals, b.cur);
  }
}

// Producer threads of a workgroup (eight wavefronts): each stages four A chunks and
// unpacks one B item per block.
constexpr int kProducerThreads = 512;
constexpr int kAChunks = kGemmBM * 16 / kProducerThreads;

// A staging: chunk q = tid + 512 j -> tile row q / 16, 16-byte column group q % 16.
// Rows past the tile's pairs load the first pair's row (so every load is unconditional) and
// are not stored into LDS.  Their LDS rows keep older data, which only reaches MFMA output
// rows of the same pairs (a product row depends on its own A row alone), never stored.
struct AStage {
  int row[kAChunks];
};

// Everything block j of the K loop takes from global memory, loaded two blocks ahead of
// its store into LDS: the thread's four A chunks and, for its B item, the sign words of
// the block's half-chunk and the word holding the block's scale.  The loads are
// unconditional, so the wait before the store counts exactly the newer set.
struct BlockRegs {
  uint4 a[kAChunks];
  uint4 w;
  uint32_t s;
};

__device__ __forceinline__ void block_load(BlockRegs& r, const AStage& as, const BItem& b, const uint16_t* A, int K,
                                           int j, int acg) {
#pragma unroll
  for (int q = 0; q < kAChunks; ++q) r.a[q] = gload16(A + (int64_t)as.row[q] * K + 128 * j + 8 * acg);
  const int c = j >> 3, d = j & 7;
  const int64_t wo = (int64_t)c * 512 + 256 * (d >> 2);   // words of half d / 4 of chunk c
  const int64_t so = (int64_t)c * 128 + 2 * (d >> 1);     // scales of blocks d & ~1 and d | 1
  r.w = gload16(b.sign + wo);
  r.s = gload4(b.scale + so);
}

__device__ __forceinline__ void a_store(const BlockRegs& r, lds_b* At, int tid, int acg, int valid) {
#pragma unroll
  for (int q = 0; q < kAChunks; ++q) {
    const int row = (tid >> 4) + (kProducerThreads / 16) * q;
    if (row < valid)
      *reinterpret_cast<lds_q*>(At + row * kRowBytes + 16 * acg) = u32x4{r.a[q].x, r.a[q].y, r.a[q].z, r.a[q].w};
  }
}

// Unpack block bd of the item into B-tile rows (Bt).  w: the sign words of the block's
// half, sw: the scale word holding the block's scale.
__device__ __forceinline__ void sign_store(const BItem& b, const uint4 w, const uint32_t sw, lds_b* Bt, int bd) {
  const int p = bd & 3;
  // the block's fp16 scale in both halves of a dword.  The asm statement keeps this
  // step here: folded back onto the loop-carried load, it would wait for the newest loads.
  uint32_t s_pair;
  const uint32_t sel = (bd & 1) ? 0x03020302u : 0x01000100u;
  asm volatile("v_perm_b32 %0, %1, %1, %2" : "=v"(s_pair) : "v"(sw), "v"(sel));
  lds_b* rowp = Bt + b.brow * kRowBytes;
#pragma unroll
  for (int ee = 0; ee < 4; ++ee) {
    const uint32_t W = ee == 0 ? w.x : (ee == 1 ? w.y : (ee == 2 ? w.z : w.w));
    uint32_t dw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[j] = s_pair ^ ((W << (15 - 4 * j - p)) & 0x80008000u);
    *reinterpret_cast<lds_q*>(rowp + 16 * group_of(b.bg, ee)) = u32x4{dw[0], dw[1], dw[2], dw[3]};
  }
}

// Add one outlier into the fp16 weight at byte offset off of the tile: the sum is
// taken in fp32 and rounded to fp16 once.
__device__ __forceinline__ void add_outlier(lds_b* Bt, int off, float add) {
  lds_h_alias* hp = reinterpret_cast<lds_h_alias*>(Bt + off);
  __half_raw hr;
  hr.x = *hp;
  hr = __half_raw(__float2half_rn(__half2float(__half(hr)) + add));
  *hp = hr.x;
}

// Unstaged outliers: the item's own walk over its row's CSR list in HBM, adding the
// entries of block bd that fall in the item's columns.
__device__ __forceinline__ void walk_outliers(BItem& b, lds_b* Bt, int bd, const gale_matrix* table) {
  const int k0 = 128 * bd, k1 = k0 + 128;
  // b.ncol / b.nq hold entry b.cur (or a column past the end), so the test never waits
  while (b.ncol < k1) {
    const int col = b.ncol, q = b.nq;
    ++b.cur;
    if (b.cur < b.cend) {
      const gale_matrix* M = table + b.gsrc;
      b.ncol = M->out_cols[b.cur];
      b.nq = outlier_value(M->out_vals, b.cur);
    } else {
      b.ncol = 0x7fffffff;
    }
    const int cb = col - k0;
    if ((((cb >> 6) & 1) | (((cb >> 4) & 1) << 1)) == b.bg) add_outlier(Bt, b_offset(b.brow, cb), b.rscale * (float)q);
  }
}

// Staged outliers of bucket (row group tt, block j) for one wavefront: lane i takes
// entry i.  starts: lane l holds the start of bucket (tt, l), l <= NB.  The entry is read
// one block ahead of its use, so its LDS latency is hidden behind a block of products.
constexpr uint32_t kNoEntry = 0x8000u;   // bit 15 is never set in an entry

struct Patch {
  int s0, s1;                   // the bucket's entry range (uniform)
  uint32_t ent;                 // the lane's entry (kNoEntry: none)
};

// entry: column in the block (bits 0..6), row in the group (7..10), int4 value (11..14),
// the row's fp16 outlier scale (16..31)
__device__ __forceinline__ uint32_t pack_entry(int cb, int rl, int q, uint16_t rs) {
  return (uint32_t)cb | ((uint32_t)rl << 7) | ((uint32_t)(q & 15) << 11) | ((uint32_t)rs << 16);
}

// Byte offset and addend of an entry.  A lane without an entry patches its own pad
// bytes of the row group (bytes 256..271 of a row, which no operand read touches) with
// 0, so the patch needs no branch.
__device__ __forceinline__ void decode_entry(uint32_t ent, int tt, int lane, int& off, float& add) {
  const int rl = (ent >> 7) & 15, cb = ent & 127;
  const int q = (int)(ent << 17) >> 28;                      // int4 in bits 11..14
  __half_raw hr;
  hr.x = (unsigned short)(ent >> 16);
  const bool none = (ent & kNoEntry) != 0;
  off = none ? (16 * tt + (lane & 15)) * kRowBytes + 256 + 2 * (lane >> 4) : b_offset(16 * tt + rl, cb);
  add = none ? 0.f : __half2float(__half(hr)) * (float)q;
}

// j < NB: bucket (tt, j); j >= NB: no entries
__device__ __forceinline__ Patch patch_prep(const lds_u32* st_ent, int starts, int tt, int j, int NB, int lane) {
  Patch pt;
  const int jj = j < NB ? j : NB - 1;
  pt.s0 = __builtin_amdgcn_readlane(starts, jj);
  pt.s1 = j < NB ? __builtin_amdgcn_readlane(starts, jj + 1) : pt.s0;
  pt.ent = pt.s0 + lane < pt.s1 ? st_ent[pt.s0 + lane] : kNoEntry;
  return pt;
}

// After the wavefront's own sign stores of the bucket's rows: the first 64 entries,
// without a branch.
__device__ __forceinline__ void patch_apply(const Patch pt, lds_b* Bt, int tt, int lane) {
  int off;
  float add;
  decode_entry(pt.ent, tt, lane, off, add);
  add_outlier(Bt, off, add);
}

// Entries past the first 64 of a dense bucket (a uniform branch, after the block's region).
__device__ __forceinline__ void patch_rest(const Patch pt, lds_b* Bt, const lds_u32* st_ent, int tt, int lane) {
  int off;
  float add;
  for (int base = pt.s0 + 64; base < pt.s1; base += 64) {
    const int i = base + lane;
    decode_entry(i < pt.s1 ? st_ent[i] : kNoEntry, tt, lane, off, add);
    add_outlier(Bt, off, add);
  }
}

// The products of one 128-column block for one wavefront: four K-steps of 32, each
// reading four B and NF A fragments (16 bytes per lane) from LDS.  NF is the number of
// 16-pair fragments of the wave's 64 pairs that hold tile pairs (the last tile of an expert
// is partly empty); the others are neither read nor multiplied.  The count is uniform per
// wavefront, so the products run without branches.
template <int NF>
__device__ __forceinline__ void mfma_frags(v8h (&af)[4], v8h (&bf)[4], const lds_b* At, const lds_b* Bt, int wm,
                                           int wn, int ml, int goff) {
#pragma unroll
  for (int nf = 0; nf < 4; ++nf)
    bf[nf] = as_v8h(*reinterpret_cast<const lds_q*>(Bt + (64 * wn + 16 * nf + ml) * kRowBytes + goff));
#pragma unroll
  for (int f = 0; f < NF; ++f)
    af[f] = as_v8h(*reinterpret_cast<const lds_q*>(At + (64 * wm + 16 * f + ml) * kRowBytes + goff));
}

// The fragments of K-step ee + 1 are read while the products of step ee run.
template <int NF>
__device__ __forceinline__ void mfma_block(v4f (&acc)[4][4], const lds_b* At, const lds_b* Bt, int wm, int wn,
                                           int ml, int lg) {
  v8h af[2][4], bf[2][4];
  mfma_frags<NF>(af[0], bf[0], At, Bt, wm, wn, ml, 16 * group_of(lg, 0));
#pragma unroll
  for (int ee = 0; ee < 4; ++ee) {
    if (ee < 3) mfma_frags<NF>(af[(ee + 1) & 1], bf[(ee + 1) & 1], At, Bt, wm, wn, ml, 16 * group_of(lg, ee + 1));
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        acc[f][nf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[ee & 1][f], bf[ee & 1][nf], acc[f][nf], 0, 0, 0);
  }
}

// Stores block j into the B buffer Bt (and A into At): A chunks, sign unpack, outliers.
template <bool STAGED>
__device__ __forceinline__ void store_block(const BlockRegs& r, BItem& b, lds_b* At, lds_b* Bt, int j, int tid, int acg,
                                            const Patch pt, int tt, const gale_matrix* table, int valid) {
  a_store(r, At, tid, acg, valid);
  sign_store(b, r.w, r.s, Bt, j);
  if (STAGED) patch_apply(pt, Bt, tt, tid & 63);
  else walk_outliers(b, Bt, j, table);
}

// The K loop over blocks of 128 columns, two LDS buffers, split by role.  Producers
// (wavefronts 0..7) fill the buffers: while the consumers run block bd from one buffer,
// block bd + 1 is stored into the other from registers, and the registers are refilled
// with block bd + 3.  NB (blocks) is a multiple of 8, so the loop takes blocks in pairs
// and each register set serves one parity.  The last pass also stores a block NB (a
// copy of block NB - 1's words, no outliers left) that nothing reads.  Both roles pass
// the same 1 + NB barriers.  Producer wavefront w unpacks and patches B row group w.
template <bool STAGED>
__device__ __forceinline__ void producer_loop(const GemmParams& P, lds_b* A0, lds_b* B0, const AStage& as, BItem& b,
                                              int NB, int tid, int acg, const lds_u32* st_ent, int starts,
                                              BlockRegs& re, BlockRegs& ro, int valid) {
  lds_b* const A1 = A0 + kTileBytes;
  lds_b* const B1 = B0 + kTileBytes;
  const int lane = tid & 63, tt = b.brow >> 4;
  const Patch none = {0, 0, kNoEntry};
  // patch entries of the block stored next (x) and of the one after (y)
  Patch px = none, py = none;
  // re holds block 0 and ro block 1 (loaded before the outlier staging)
  if (STAGED) {
    px = patch_prep(st_ent, starts, tt, 0, NB, lane);
    py = patch_prep(st_ent, starts, tt, 1, NB, lane);
  }
  store_block<STAGED>(re, b, A0, B0, 0, tid, acg, px, tt, P.table, valid);
  if (STAGED) patch_rest(px, B0, st_ent, tt, lane);
  __builtin_amdgcn_sched_barrier(0);
  block_load(re, as, b, P.A, P.K, 2, acg);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  for (int bd = 0; bd < NB; bd += 2) {
    // block bd (buffer 0) runs; block bd + 1 into buffer 1
    if (STAGED) px = patch_prep(st_ent, starts, tt, bd + 2, NB, lane);
    store_block<STAGED>(ro, b, A1, B1, bd + 1, tid, acg, py, tt, P.table, valid);
    block_load(ro, as, b, P.A, P.K, min(bd + 3, NB - 1), acg);
    if (STAGED) patch_rest(py, B1, st_ent, tt, lane);
    __syncthreads();
    // block bd + 1 (buffer 1) runs; block bd + 2 into buffer 0
    if (STAGED) py = patch_prep(st_ent, starts, tt, bd + 3, NB, lane);
    store_block<STAGED>(re, b, A0, B0, bd + 2, tid, acg, px, tt, P.table, valid);
    block_load(re, as, b, P.A, P.K, min(bd + 4, NB - 1), acg);
    if (STAGED) patch_rest(px, B0, st_ent, tt, lane);
    __syncthreads();
  }
}

// Consumers (wavefronts 8..11): the products of each block, alternating buffers.
template <int NF>
__device__ __forceinline__ void consumer_loop(v4f (&acc)[4][4], const lds_b* A0, const lds_b* B0, int NB, int wm,
                                              int wn, int ml, int lg) {
  const lds_b* const A1 = A0 + kTileBytes;
  const lds_b* const B1 = B0 + kTileBytes;
  __syncthreads();
  for (int bd = 0; bd < NB; bd += 2) {
    if (NF > 0) mfma_block<NF>(acc, A0, B0, wm, wn, ml, lg);
    __syncthreads();
    if (NF > 0) mfma_block<NF>(acc, A1, B1, wm, wn, ml, lg);
    __syncthreads();
  }
}

template <bool GATEUP>
__global__ void __launch_bounds__(kProducerThreads + 256) grouped_gemm_kernel(const GemmParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int n_tiles = *P.n_tiles;
  if ((int)blockIdx.y >= n_tiles) return;
  const GemmTile tile = P.tiles[blockIdx.y];
  const int e = tile.expert, m0 = tile.m0;
  const int pair0 = P.offsets[e] + m0;
  const int valid = min(kGemmBM, P.offsets[e + 1] - pair0);
  const int n0 = blockIdx.x * P.half_rows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // wavefronts 0..7 load, unpack and patch (tid 0..511); 8..11 run the products
  const bool producer = wave < kProducerThreads / 64;
  const int tid = threadIdx.x & (kProducerThreads - 1);
  const int C = P.K >> 10;
  const int NB = P.K >> 7;

  lds_b* const base = (lds_b*)smem;
  lds_b* const A0 = base;
  lds_b* const B0 = base + 2 * kTileBytes;
  lds_u32* const st_ent = reinterpret_cast<lds_u32*>(base + 4 * kTileBytes);
  lds_i32* const st_misc = reinterpret_cast<lds_i32*>(base + 4 * kTileBytes + 4 * kOutStage);
  lds_i32* const s_orow = st_misc + 8;                       // output row of tile pair m
  lds_i32* const st_start = reinterpret_cast<lds_i32*>(A0 + kTileBytes);   // during the sort
  lds_i32* const st_fill = st_start + kBuckets + 1;

  AStage as;
  const int acg = tid & 15;
  BItem b;
  BlockRegs re, ro;   // blocks of even and of odd index
  if (producer) {
    const int first_row = P.a_by_token ? P.perm[pair0] / P.top_k : P.perm[pair0];
#pragma unroll
    for (int j = 0; j < kAChunks; ++j) {
      const int rr = (tid >> 4) + (kProducerThreads / 16) * j;
      int src = first_row;
      if (rr < valid) {
        const int s = pair0 + rr;
        src = P.a_by_token ? P.perm[s] / P.top_k : P.perm[s];
      }
      as.row[j] = src;
    }
    b = make_item(P, e, n0, C, tid);
    // blocks 0 and 1 load while the outliers are staged; the two sets issue in order (no
    // interleaving), so the K loop's waits count whole sets
    __builtin_amdgcn_sched_barrier(0);
    block_load(re, as, b, P.A, P.K, 0, acg);
    __builtin_amdgcn_sched_barrier(0);
    block_load(ro, as, b, P.A, P.K, 1, acg);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- outlier staging by the producers (the consumers pass the same barriers).  Row
  //      r = tid / 4 of the B tile (matrix sel_a for r < half_rows, else sel_b; global row
  //      n0 + r % half_rows) is walked by four threads, entries p with p % 4 = tid % 4: count
  //      per bucket, scan (wavefronts 0..3, two buckets per thread), then place each entry.
  const int r = tid >> 2, par = tid & 3;
  const bool scanner = threadIdx.x < 256;
  const gale_matrix* Mr = P.table + 3 * e + (r >= P.half_rows ? P.sel_b : P.sel_a);
  const int gr = n0 + r % P.half_rows;
  int rp0 = 0, rp1 = 0;
  if (producer) {
    rp0 = Mr->row_ptr[gr];
    rp1 = Mr->row_ptr[gr + 1];
  }
  const int nbk = 8 * NB;                                    // buckets in use
  if (threadIdx.x == 0) st_misc[0] = 0;
  if (threadIdx.x < kGemmBM) s_orow[threadIdx.x] = (int)threadIdx.x < valid ? P.perm[pair0 + threadIdx.x] : 0;
  for (int i = threadIdx.x; i < kBuckets; i += blockDim.x) st_fill[i] = 0;
  __syncthreads();
  if (producer && par == 0) __atomic_fetch_add(st_misc, rp1 - rp0, __ATOMIC_RELAXED);
  __syncthreads();
  const bool staged = st_misc[0] <= kOutStage && NB <= kStageBlocks;
  const int bucket0 = (r >> 4) * NB;
  int starts = 0;
  if (staged) {
    // the walks take the thread's entries eight at a time, loads first (clamped into the
    // row's range) so that eight are in flight
    if (producer) {
      for (int p0 = rp0 + par; p0 < rp1; p0 += 32) {
        int col[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) col[k] = Mr->out_cols[min(p0 + 4 * k, rp1 - 1)];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (p0 + 4 * k < rp1) __atomic_fetch_add(st_fill + bucket0 + (col[k] >> 7), 1, __ATOMIC_RELAXED);
      }
    }
    __syncthreads();
    // exclusive scan of the bucket counts, two per thread
    int c0 = 0, c1 = 0, v = 0;
    if (scanner) {
      c0 = 2 * tid < nbk ? st_fill[2 * tid] : 0;
      c1 = 2 * tid + 1 < nbk ? st_fill[2 * tid + 1] : 0;
      v = c0 + c1;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
      }
      if (lane == 63) st_misc[1 + wave] = v;
    }
    __syncthreads();
    if (scanner) {
      int ex = v - c0 - c1;
      for (int w = 0; w < wave; ++w) ex += st_misc[1 + w];
      if (2 * tid < nbk) st_start[2 * tid] = st_fill[2 * tid] = ex;
      if (2 * tid + 1 < nbk) st_start[2 * tid + 1] = st_fill[2 * tid + 1] = ex + c0;
      if (tid == 255) st_start[nbk] = ex + c0 + c1;
    }
    __syncthreads();
    if (producer) {
      const uint16_t rs = Mr->row_scales[gr];
      for (int p0 = rp0 + par; p0 < rp1; p0 += 32) {
        int col[8], q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int p = min(p0 + 4 * k, rp1 - 1);
          col[k] = Mr->out_cols[p];
          q[k] = outlier_value(Mr->out_vals, p);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (p0 + 4 * k < rp1) {
            const int slot = __atomic_fetch_add(st_fill + bucket0 + (col[k] >> 7), 1, __ATOMIC_RELAXED);
            st_ent[slot] = pack_entry(col[k] & 127, r & 15, q[k], rs);
          }
        }
      }
    }
    // bucket starts of the producer wavefront's row group, lane l: block l (l <= NB)
    if (producer) starts = lane <= NB ? st_start[wave * NB + lane] : 0;
    __syncthreads();
  }

  // ---- accumulators of consumer (wm, wn) = pairs [64 wm, +64) x B rows [64 wn, +64)
  const int wm = wave & 1, wn = (wave >> 1) & 1;   // consumer wavefronts 8..11
  const int ml = lane & 15, lg = lane >> 4;
  v4f acc[4][4];
  if (producer) {
    if (staged) {
      producer_loop<true>(P, A0, B0, as, b, NB, tid, acg, st_ent, starts, re, ro, valid);
    } else {
      item_walk_init(P, e, n0, b);
      producer_loop<false>(P, A0, B0, as, b, NB, tid, acg, st_ent, 0, re, ro, valid);
    }
  } else {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[f][nf] = v4f{0.f, 0.f, 0.f, 0.f};
    // 16-pair fragments of this wave's 64 pairs that hold tile pairs
    const int nfrag = __builtin_amdgcn_readfirstlane(max(0, min(4, (valid - 64 * wm + 15) >> 4)));
    switch (nfrag) {
      case 4: consumer_loop<4>(acc, A0, B0, NB, wm, wn, ml, lg); break;
      case 3: consumer_loop<3>(acc, A0, B0, NB, wm, wn, ml, lg); break;
      case 2: consumer_loop<2>(acc, A0, B0, NB, wm, wn, ml, lg); break;
      case 1: consumer_loop<1>(acc, A0, B0, NB, wm, wn, ml, lg); break;
      default: consumer_loop<0>(acc, A0, B0, NB, wm, wn, ml, lg); break;
    }
  }

  // ---- epilogue (consumers).  Fragment layout: lane l, register i -> pair 16 f + 4 (l / 16)
  //      + i, B row 16 nf + l % 16 of the wave's range.
  if (GATEUP) {
    // the waves of w3 rows hand their products to the waves of the same w1 rows
    float* U = reinterpret_cast<float*>(smem);
    if (!producer && wn == 1) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          *reinterpret_cast<float4*>(U + ((wm * 16 + f * 4 + nf) * 64 + lane) * 4) =
              make_float4(acc[f][nf][0], acc[f][nf][1], acc[f][nf][2], acc[f][nf][3]);
    }
    __syncthreads();
    if (!producer && wn == 0) {
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
            const int orow = s_orow[m];
            P.out[(int64_t)orow * P.out_stride + n0 + 16 * nf + ml] = g / (1.0f + __expf(-g)) * uu[i];
          }
        }
      }
    }
  } else if (!producer) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 64 * wm + 16 * f + 4 * lg + i;
          if (m >= valid) continue;
          const int orow = s_orow[m];
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
    hipLaunchKernelGGL(grouped_gemm_kernel<true>, grid, dim3(kProducerThreads + 256), kGemmSmem, s, P);
  } else {
    err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kGemmSmem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_kernel<false>, grid, dim3(kProducerThreads + 256), kGemmSmem, s, P);
  }
  return hipGetLastError();
}

}  // namespace gale
