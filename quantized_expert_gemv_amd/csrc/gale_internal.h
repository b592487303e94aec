// Internal declarations shared by the libgale translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

#include "gale.h"

namespace gale {

// ---------------------------------------------------------------------------
// Device layout index map (host and device).  A "tile" is 16 rows x 1024
// columns; C = cols / 1024 chunks per row tile.  Within a tile, lane l of a
// wavefront owns row (l % 16) and lane group g = l / 16; its 8 words sit at
// half h = 0, 1 (element e = 0..3 of each half).  Word 4 h + j holds four scale
// blocks d = 4 h + p (p = 0..3) at bit positions 4 i + p, i = 0..7: masking one
// bit position of every nibble selects exactly one scale block, as the eight
// 4-bit elements of one dword of an fp4 MFMA operand.  The column of (g, j, i)
// within block d follows the fp4 operand order of the 16x16x128 MFMA:
//   kh = 64 (g & 1) + 16 (g >> 1) + 32 (j >> 1) + 8 (j & 1) + i.
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t sign_word_index(int t, int c, int C, int h, int l, int e) {
  return ((((int64_t)t * C + c) * 2 + h) * 64 + l) * 4 + e;
}

__host__ __device__ inline int fp4_col(int g, int j, int i) {
  return 64 * (g & 1) + 16 * (g >> 1) + 32 * (j >> 1) + 8 * (j & 1) + i;
}

// canonical (n, k) -> (device word index, bit position)
__host__ __device__ inline void sign_position(int n, int k, int C, int64_t* word, int* bit) {
  const int t = n >> 4, nl = n & 15;
  const int c = k >> 10, kk = k & 1023;
  const int d = kk >> 7, kh = kk & 127;
  const int i = kh & 7;
  const int j = ((kh >> 3) & 1) | (((kh >> 5) & 1) << 1);
  const int g = ((kh >> 6) & 1) | (((kh >> 4) & 1) << 1);
  *word = sign_word_index(t, c, C, d >> 2, 16 * g + nl, j);
  *bit = 4 * i + (d & 3);
}

__host__ __device__ inline int64_t scale_index(int n, int blk, int C) {
  // s[n][blk], blk = 8 c + d  ->  [n/16][c][n%16][d]
  int t = n >> 4, r = n & 15, c = blk >> 3, d = blk & 7;
  return (((int64_t)t * C + c) * 16 + r) * 8 + d;
}

// ---------------------------------------------------------------------------
// Rotated-activation record ("RA"): one per activation vector of length K.
//   [0, 4K)          x~ = blockdiag(H) x, fp32
//   [4K, 8K)         fp8 e4m3 terms: chunk c, term t at 4K + (4 c + t) * 1024,
//                    X = x~ * 2^p_c = t0 + t1 + t2 + t3 elementwise
//   [8K, 8K + 4C)    p_c (int32), one per 1024-chunk
// padded to a multiple of 256 bytes.
// ---------------------------------------------------------------------------
__host__ __device__ inline size_t ra_bytes(int K) {
  size_t b = (size_t)8 * K + 4 * (size_t)(K / 1024);
  return (b + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t ra_terms_off(int K) { return (size_t)4 * K; }
__host__ __device__ inline size_t ra_p_off(int K) { return (size_t)8 * K; }

constexpr int kTerms = 4;

// Work item of the explicit (routed) GEMV mode.
struct WorkItem {
  int32_t expert;     // item matrix index in the descriptor table (times stride)
  int32_t n_slots;    // 1..4 activation vectors
  int32_t pair[4];    // pair ids (RA index = pair / ra_div, output index = pair)
  int32_t pad[2];
};

struct GemvParams {
  const gale_matrix* table;  // descriptor table
  int mat_stride;            // descriptors per item
  int sel0, sel1;            // descriptor offsets (sel1: second matrix for gate/up)
  int rows, cols;
  const uint8_t* ra;         // RA records
  size_t ra_stride;
  // implicit items: item i = (mat i / n_groups, token group i % n_groups)
  int implicit_items;
  int n_tok;
  int n_groups;
  int x_shared;
  int n_items;               // implicit item count
  // explicit items
  const WorkItem* items;
  const int32_t* n_items_dev;
  int ra_div;
  // output
  void* y;
  int y_dtype;
  int64_t y_stride;          // elements between consecutive output vectors
  int gateup;                // SwiGLU epilogue (y = fp32 h)
  int row_groups;            // units per item along rows
  int stage_xt;              // copy x~ into LDS for the outlier gathers
  int out_chunks;            // outlier column chunks staged per wavefront and unit (2, 4 or 8)
  // raw activations (one vector per item): each workgroup rotates and splits an item's x
  // into an LDS record itself instead of reading a prepared record (ra unused)
  const void* x;
  int x_dtype;
  int x_rotated;
  int64_t x_stride;          // elements between consecutive x vectors
};

// Which vectors of a grouped layer a side needs.  Vector v is a token (per_token: its
// top_k experts idx[v k + s]) or a pair (its expert idx[v]).  An expert with fewer than
// split pairs runs as GEMV items, the others as GEMM tiles; a vector is kept when one of its
// experts runs on the side asked for (items_side).  idx == nullptr keeps every vector.
struct VecFilter {
  const int32_t* idx = nullptr;
  const int32_t* offsets = nullptr;   // pair offsets per expert [E + 1]
  int top_k = 1, per_token = 0, split = 0, items_side = 0;
};

__device__ __forceinline__ bool filter_keep(const VecFilter& f, int64_t v) {
  if (f.idx == nullptr) return true;
  const int n = f.per_token ? f.top_k : 1;
  const int32_t* ex = f.idx + (f.per_token ? v * f.top_k : v);
  bool keep = false;
  for (int s = 0; s < n; ++s) {
    const int e = __builtin_amdgcn_readfirstlane(ex[s]);
    const bool items = f.offsets[e + 1] - f.offsets[e] < f.split;
    keep = keep || (items == (f.items_side != 0));
  }
  return keep;
}

// launches (return hipError_t of the launch)
hipError_t launch_prep(const void* x, int x_dtype, int64_t x_stride, int n_vec, int K, int rotated,
                       uint8_t* ra, size_t ra_stride, hipStream_t s, const VecFilter& filt = VecFilter());
hipError_t launch_fwht(const void* x, void* y, int64_t n_vec, int len, int in_dtype, int out_dtype,
                       hipStream_t s);
// max_units: upper bound of the number of units (items x row groups); the launch is a
// persistent grid of at most that many workgroups.
// threads of a GEMV workgroup: 64 per 1024-column chunk of each matrix
constexpr int kGemvMaxThreads = 1024;
hipError_t launch_gemv(const GemvParams& p, int slots, int tiles_per_unit, int64_t max_units, hipStream_t s);
size_t gemv_smem_bytes(int cols, int slots, int tiles, int gateup, int stage_xt, int out_chunks, int fused = 0);
constexpr size_t kGemvMaxLds = 160 * 1024;   // LDS per workgroup on gfx950
int device_cu_count();
hipError_t launch_pack(int rows, int cols, int n_mat, const uint32_t* cs, const uint16_t* csc,
                       uint32_t* ds, uint16_t* dsc, hipStream_t s);
hipError_t launch_debug_unpack(int rows, int cols, const uint32_t* ds, uint32_t* cs, hipStream_t s);
hipError_t launch_debug_outliers(int rows, int64_t nnz, gale_matrix m, int32_t* r, int32_t* c,
                                 int32_t* v, hipStream_t s);

// routing
// Routing inputs of a batch: logits [T][E]; an optional selection bias [E], added to the
// logits for the choice of the k experts only (the balancing term of the DeepSeek-V4-Pro
// GALE page's serving notes, which never enters the weights); optional fixed experts [T][k]
// (hash-routed layers, DeepSeek-V4-Flash 180B REAP card: the experts come from a table, in
// slot order).  The k weights are always the softmax of the chosen experts' own logits.
struct RouteIn {
  const float* logits;
  const float* bias;      // NULL: none
  const int32_t* fixed;   // NULL: top-k
};

hipError_t launch_route_small(const RouteIn& rin, int n_tok, int n_exp, int k, int32_t* idx, float* w,
                              int32_t* offsets, int32_t* perm, WorkItem* items, int32_t* n_items,
                              int max_slots, hipStream_t s);
hipError_t launch_route_prep(const RouteIn& rin, int n_tok, int n_exp, int k, int32_t* idx, float* w,
                             WorkItem* items, int32_t* n_items, int max_slots, const void* x, int x_dtype, int K,
                             uint8_t* ra, size_t ra_stride, hipStream_t s);
hipError_t launch_route_large(const RouteIn& rin, int n_tok, int n_exp, int k, int32_t* idx, float* w,
                              int32_t* chunk_cnt, int32_t* offsets, int32_t* perm, hipStream_t s);
inline size_t route_chunk_count_bytes(int n_tok, int n_exp) {
  return (size_t)4 * ((n_tok + 63) / 64) * n_exp;
}
hipError_t launch_combine(const float* ypairs, const float* w, int n_tok, int k, int hidden,
                          void* y, int y_dtype, hipStream_t s);
hipError_t launch_cast(const float* src, void* dst, int dst_dtype, int64_t n, hipStream_t s);

// grouped path: work items of at most `slots` pairs per expert from the sorted pairs
hipError_t launch_build_items(const int32_t* offsets, const int32_t* perm, int n_exp, int slots, int max_pairs,
                              WorkItem* items, int32_t* n_items, hipStream_t s);
// grouped GEMM: tiles of kGemmBM sorted pairs of one expert
constexpr int kGemmBM = 128;
struct GemmTile {
  int32_t expert, m0;
};
hipError_t launch_build_tiles(const int32_t* offsets, int n_exp, int min_pairs, GemmTile* tiles, int32_t* n_tiles,
                              hipStream_t s);
// rows of K rotated into fp16 with every 8-column group in MFMA operand order
hipError_t launch_rotate_f16(const void* x, int x_dtype, int64_t n_rows, int K, uint16_t* out, hipStream_t s,
                             const VecFilter& filt = VecFilter());
// gateup: out[pair][inter] = silu(w1 x~) * (w3 x~), A = rotated x by token; else out[pair][hidden] = w2 h~,
// A = rotated h by pair (fp32 outputs)
hipError_t launch_grouped_gemm(const gale_matrix* table, int gateup, int rows, int K, const int32_t* offsets,
                               const int32_t* perm, int top_k, const GemmTile* tiles, const int32_t* n_tiles,
                               int max_tiles, const uint16_t* A, float* out, int out_stride, hipStream_t s);

// one-launch decode of one token through one MoE layer or a stack of layers (route, gate/up +
// SwiGLU, rotate h, down, combine per layer); sync: kDecodeSyncBytes of synchronisation words
// (zero-filled before the first call), h: decode_stack_h_bytes(inter, top_k) of fp32 h,
// rec: decode_stack_rec_bytes(inter, top_k) for the activation records of the rotated h
constexpr size_t kDecodeSyncBytes = GALE_SYNC_BYTES;
bool decode_layer_supported(int hidden, int inter, int top_k);
size_t decode_stack_h_bytes(int inter, int top_k);
size_t decode_stack_rec_bytes(int inter, int top_k);
hipError_t launch_decode_stack(const gale_layer_io& io0, const gale_layer_io* layers_dev, int L, int E, int k,
                               int hidden, int inter, float* h, uint8_t* rec, uint64_t* sync, int tiles,
                               int64_t wait_ticks, hipStream_t s);
hipError_t launch_sync_init(void* sync, hipStream_t s);
// 0: valid and no error; 1: the words were never zeroed; 2: a barrier wait gave up
int sync_words_state(const uint64_t words[3]);
// device address of this GPU's GALE_STATIC_SCRATCH_BYTES array (looked up once per device)
hipError_t static_scratch(void** out);

void set_error(const char* fmt, ...);

}  // namespace gale
