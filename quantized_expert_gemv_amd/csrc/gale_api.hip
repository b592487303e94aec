// C-ABI entry points of libgale: host-side validation, workspace layout and the
// launch sequence of each call.  No call allocates, synchronises or copies
// between host and device; every launch goes on the caller's stream.
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>

#include "gale_internal.h"

namespace gale {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static inline int dtype_ok(int d) { return d == GALE_F16 || d == GALE_F32; }

static inline int dsize(int d) { return d == GALE_F16 ? 2 : 4; }

static int check_matrix_shape(const char* fn, int rows, int cols) {
  if (rows < 16 || rows % 16 || rows > GALE_MAX_ROWS) {
    set_error("%s: rows=%d must be a positive multiple of 16 up to %d", fn, rows, GALE_MAX_ROWS);
    return GALE_ERR_SHAPE;
  }
  if (cols < 1024 || cols % 1024 || cols > GALE_MAX_COLS) {
    set_error("%s: cols=%d must be a positive multiple of 1024 up to %d", fn, cols, GALE_MAX_COLS);
    return GALE_ERR_SHAPE;
  }
  return GALE_OK;
}

static int hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) {
    set_error("%s: %s", fn, hipGetErrorString(e));
    return GALE_ERR_HIP;
  }
  return GALE_OK;
}

static int stage_ok(int cols, int slots) { return (int64_t)slots * cols * 4 <= 65536 ? 1 : 0; }

// Outlier column chunks staged per wavefront and unit, from flags bits 14..15 (2, 4 or 8;
// eight only with one vector per item, else four), fewer where the workgroup's staging
// would not fit the LDS next to its other buffers.
//
// The flag describes the matrices of ref_cols columns (an expert's w1/w3: hidden).  The
// budget is a share of each row, so a phase over fewer columns (w2: inter) stages
// proportionally fewer entries: with the default, 512 per 16 rows for inter = hidden / 2,
// which frees LDS (one more workgroup per CU for four-vector items) and registers.
static int pick_out_chunks(uint32_t flags, int slots, int cols, int gateup, int ref_cols) {
  const int v = (int)((flags >> GALE_OUTLIER_STAGE_SHIFT) & 3);
  int oc = v == 0 ? 2 : (v == 1 || slots > 1 ? 4 : 8);
  if (!gateup) {
    // oc * cols / ref_cols chunks, at least one
    int64_t c = cols;
    while (oc > 1 && 2 * c <= ref_cols) {
      oc >>= 1;
      c *= 2;
    }
  }
  while (oc > 2 && gemv_smem_bytes(cols, slots, 4, gateup, stage_ok(cols, slots), oc) > kGemvMaxLds) oc >>= 1;
  return oc;
}

// Row tiles per unit: at most the chunk count (four lanes per row serve the outliers),
// at most what the registers hold next to the outlier staging (two chunks: 4, or 3 with
// four activation vectors; one or four chunks: 3, or 2 with four vectors; eight chunks: 2), and
// small enough that the units cover the GPU at least twice; flags bits 8..11 force a value
// (1, 2 or 4).  A unit's loads are issued one unit ahead, so wider units keep more bytes in
// flight per CU: with one or two vectors, four tiles stream ~1.4x faster than two.
static int pick_tiles(int64_t items, int ntiles, int cols, int slots, int out_chunks, uint32_t flags) {
  const int C = cols / 1024;
  int r = 4;
  const int forced = (int)((flags >> GALE_TILES_SHIFT) & 0xF);
  if (forced) r = 1 << (forced - 1);
  if (r > 4) r = 4;
  const int cap = out_chunks == 8 ? 2 : (out_chunks == 4 || out_chunks == 1 ? (slots >= 4 ? 2 : 3) : (slots >= 4 ? 3 : 4));
  if (r > cap) r = cap;                           // the kernel's register budget
  if (r > C) r = C >= 3 ? 3 : C;                  // three chunks: units of three tiles
  if (r == 3 && forced) r = 2;
  if (!forced) {
    const int64_t want = 2 * (int64_t)device_cu_count();
    while (r > 1 && items * ((ntiles + r - 1) / r) < want) r >>= 1;
  }
  return r;
}


static int pick_slots(int n_tok) { return n_tok >= 4 ? 4 : (n_tok >= 2 ? 2 : 1); }

// Whether a phase of one vector per item can take raw activations (the GEMV rotates and
// splits x itself): at most eight chunks per matrix (sixteen wavefronts for a gate/up pair
// do not fit), a staging the raw-activation builds cover, and an LDS layout (record and x
// copies on top of the staging) that keeps as many workgroups per CU as the prepared path:
// the kernels hold two wavefronts per SIMD (more than 128 registers), eight per CU.
static bool raw_x_ok(int cols, int gateup, uint32_t flags, int ref_cols) {
  const int C = cols >> 10;
  if (C > (gateup ? 4 : 8)) return false;
  const int oc = pick_out_chunks(flags, 1, cols, gateup, ref_cols);
  if (gateup ? (oc != 2 && oc != 4) : (oc != 1 && oc != 2 && oc != 4 && oc != 8)) return false;
  const size_t raw = gemv_smem_bytes(cols, 1, 4, gateup, 1, oc, 1);
  const size_t prep = gemv_smem_bytes(cols, 1, 4, gateup, 1, oc, 0);
  if (raw > kGemvMaxLds) return false;
  const int by_regs = std::max(1, 8 / ((gateup ? 2 : 1) * C));
  const int occ_raw = std::min(by_regs, (int)(kGemvMaxLds / raw));
  const int occ_prep = std::min(by_regs, (int)(kGemvMaxLds / prep));
  return occ_raw >= occ_prep;
}

// Activation vectors per GEMV work item of the MoE layer.  Decode batches spread their pairs
// thinly (T k / E pairs per expert on average): items of one or two vectors then run the
// wider row-tile units of the single-vector builds and waste no MFMA rows on empty slots
// (measured on 256 experts, top-6: T = 4 and 16 fastest with one, T = 32 with two).  The
// grouped path keeps four: its items serve experts with many pairs each.
static int pick_moe_slots(int n_tok, int k, int E, bool grouped) {
  if (grouped) return pick_slots(n_tok);
  const int64_t pairs2 = 2 * (int64_t)n_tok * k;      // twice the pairs: compare against E / 2 and 3 E / 2
  if (pairs2 <= E) return 1;
  if (pairs2 <= 3 * (int64_t)E) return 2;
  return pick_slots(n_tok);
}

// ---- workspace layouts -------------------------------------------------------
struct GemvWs {
  size_t ra, total;
};
static GemvWs gemv_ws(int cols, int64_t n_x) {
  GemvWs w;
  w.ra = 0;
  w.total = align256(ra_bytes(cols) * (size_t)n_x);
  return w;
}

struct FfnWs {
  size_t ra_x, h, ra_h, total;
};
static FfnWs ffn_ws(int hidden, int inter, int64_t n_x, int64_t n_pairs) {
  FfnWs w;
  w.ra_x = 0;
  w.h = align256(ra_bytes(hidden) * (size_t)n_x);
  w.ra_h = w.h + align256((size_t)4 * inter * n_pairs);
  w.total = w.ra_h + align256(ra_bytes(inter) * (size_t)n_pairs);
  return w;
}

struct MoeWs {
  size_t idx, w, offsets, perm, chunk, items, n_items, ra_x, h, ra_h, yp;   // decode / items
  size_t tiles, xt16, ht16;                                                 // grouped GEMM
  size_t sync;                                                              // one-launch decode (offset 0)
  size_t total;
};
// Upper bound on the work items of T tokens: every item holds at least one pair, and
// each expert's run of pairs ends in at most one partly filled item.
static int64_t moe_item_bound(int T, int E, int k, int slots) {
  const int64_t P = (int64_t)T * k;
  return std::min<int64_t>(P, std::min<int64_t>(E, P) + (P + slots - 1) / slots);
}
// The same for the GEMM tiles of kGemmBM pairs.
static int64_t moe_tile_bound(int T, int E, int k) {
  const int64_t P = (int64_t)T * k;
  return std::min<int64_t>(P, std::min<int64_t>(E, P) + (P + kGemmBM - 1) / kGemmBM);
}
enum MoePath { kDecode = 0, kGroupedItems = 1, kGroupedGemm = 2, kGroupedHybrid = 3 };
// Experts with at least this many pairs take the tile GEMM in the hybrid grouped path.
constexpr int kGemmMinPairs = 20;
// Row tiles per unit of the one-token layer kernel, (gate/up, down) as decimal digits.
constexpr int kDecodeLayerTiles = 32;
// Give-up time of a one-launch decode wait (100 MHz ticks): 10 ms, far beyond any healthy
// barrier (~2 us) and short enough that a launch whose workgroups are not all resident ends.
static int64_t decode_wait_ticks(uint32_t flags) { return (flags & GALE_SYNC_NO_WAIT) ? 0 : 1000000; }
static MoePath moe_path(int n_tok, uint32_t flags) {
  const bool grouped = (flags & GALE_PATH_GROUPED) || (!(flags & GALE_PATH_DECODE) && n_tok > GALE_MAX_DECODE_TOKENS);
  if (!grouped) return kDecode;
  if (flags & GALE_GROUPED_ITEMS) return kGroupedItems;
  if (flags & GALE_GROUPED_GEMM) return kGroupedGemm;
  return kGroupedHybrid;
}
static MoeWs moe_ws(int T, int E, int k, int hidden, int inter, MoePath path) {
  MoeWs w;
  memset(&w, 0, sizeof(w));
  const int64_t P = (int64_t)T * k;
  const int slots = pick_moe_slots(T, k, E, path != kDecode);
  size_t o = 0;
  w.sync = o; o += align256(kDecodeSyncBytes);   // first, at a fixed place (gale_sync_init / _status)
  w.idx = o; o += align256(4 * P);
  w.w = o; o += align256(4 * P);
  w.offsets = o; o += align256(4 * (size_t)(E + 1));
  w.perm = o; o += align256(4 * P);
  w.chunk = o; o += path != kDecode ? align256(route_chunk_count_bytes(T, E)) : 0;
  w.n_items = o; o += 256;
  w.h = o; o += align256((size_t)4 * inter * P);
  w.yp = o; o += align256((size_t)4 * hidden * P);
  if (path == kGroupedGemm || path == kGroupedHybrid) {
    w.tiles = o; o += align256(sizeof(GemmTile) * (size_t)moe_tile_bound(T, E, k));
    w.xt16 = o; o += align256((size_t)2 * hidden * T);
    w.ht16 = o; o += align256((size_t)2 * inter * P);
  }
  if (path != kGroupedGemm) {
    w.items = o; o += align256(sizeof(WorkItem) * (size_t)moe_item_bound(T, E, k, slots));
    w.ra_x = o; o += align256(ra_bytes(hidden) * (size_t)T);
    w.ra_h = o; o += align256(ra_bytes(inter) * (size_t)P);
  }
  w.total = o;
  return w;
}

}  // namespace gale

using namespace gale;

// ============================================================================
// errors and sizes
// ============================================================================
extern "C" const char* gale_status_str(int s) {
  switch (s) {
    case GALE_OK: return "ok";
    case GALE_ERR_NULL: return "null pointer";
    case GALE_ERR_SHAPE: return "bad shape";
    case GALE_ERR_DTYPE: return "bad dtype";
    case GALE_ERR_ALIGN: return "misaligned pointer";
    case GALE_ERR_WORKSPACE: return "workspace too small";
    case GALE_ERR_UNSUPPORTED: return "unsupported";
    case GALE_ERR_FORMAT: return "bad canonical format";
    case GALE_ERR_HIP: return "HIP runtime error";
    case GALE_ERR_SYNC: return "decode synchronisation words not valid";
    default: return "unknown status";
  }
}

extern "C" const char* gale_last_error(void) { return g_err; }

extern "C" int gale_packed_sizes(int32_t rows, int32_t cols, int64_t nnz, gale_sizes* out) {
  if (!out) { set_error("gale_packed_sizes: out is NULL"); return GALE_ERR_NULL; }
  int st = check_matrix_shape("gale_packed_sizes", rows, cols);
  if (st) return st;
  if (nnz < 0 || nnz > (int64_t)rows * cols) { set_error("gale_packed_sizes: bad nnz"); return GALE_ERR_SHAPE; }
  out->signs = (size_t)rows * cols / 8;
  out->block_scales = (size_t)rows * (cols / 128) * 2;
  out->row_scales = (size_t)rows * 2;
  out->row_ptr = (size_t)(rows + 1) * 4;
  out->out_cols = (size_t)nnz * 2;
  out->out_vals = (size_t)(nnz + 1) / 2;
  out->format_bytes = out->signs + out->block_scales + out->row_scales + out->out_cols + out->out_vals;
  return GALE_OK;
}

extern "C" int gale_check_canonical(int32_t rows, int32_t cols, const int32_t* row_ptr,
                                    const uint16_t* out_cols, int64_t nnz) {
  int st = check_matrix_shape("gale_check_canonical", rows, cols);
  if (st) return st;
  if (!row_ptr || (nnz > 0 && !out_cols)) { set_error("gale_check_canonical: NULL pointer"); return GALE_ERR_NULL; }
  if (row_ptr[0] != 0 || row_ptr[rows] != nnz) {
    set_error("gale_check_canonical: row_ptr must start at 0 and end at nnz=%lld", (long long)nnz);
    return GALE_ERR_FORMAT;
  }
  for (int n = 0; n < rows; ++n) {
    if (row_ptr[n + 1] < row_ptr[n]) { set_error("gale_check_canonical: row_ptr decreases at row %d", n); return GALE_ERR_FORMAT; }
    for (int p = row_ptr[n]; p < row_ptr[n + 1]; ++p) {
      if (out_cols[p] >= cols) { set_error("gale_check_canonical: column %d >= cols at row %d", out_cols[p], n); return GALE_ERR_FORMAT; }
      if (p > row_ptr[n] && out_cols[p] <= out_cols[p - 1]) {
        set_error("gale_check_canonical: columns not strictly ascending at row %d", n);
        return GALE_ERR_FORMAT;
      }
    }
  }
  return GALE_OK;
}

// ============================================================================
// packing and debug
// ============================================================================
extern "C" int gale_pack_device(int32_t rows, int32_t cols, int32_t n_mat, const uint32_t* canon_signs,
                                const uint16_t* canon_scales, uint32_t* dev_signs, uint16_t* dev_scales,
                                hipStream_t stream) {
  int st = check_matrix_shape("gale_pack_device", rows, cols);
  if (st) return st;
  if (n_mat < 1) { set_error("gale_pack_device: n_mat=%d", n_mat); return GALE_ERR_SHAPE; }
  if (!canon_signs || !canon_scales || !dev_signs || !dev_scales) { set_error("gale_pack_device: NULL pointer"); return GALE_ERR_NULL; }
  if (!aligned(dev_signs, 16) || !aligned(dev_scales, 16) || !aligned(canon_signs, 4) || !aligned(canon_scales, 2)) {
    set_error("gale_pack_device: misaligned pointer");
    return GALE_ERR_ALIGN;
  }
  return hip_status("gale_pack_device", launch_pack(rows, cols, n_mat, canon_signs, canon_scales, dev_signs, dev_scales, stream));
}

extern "C" int gale_debug_unpack_signs(int32_t rows, int32_t cols, const uint32_t* dev_signs,
                                       uint32_t* canon_signs, hipStream_t stream) {
  int st = check_matrix_shape("gale_debug_unpack_signs", rows, cols);
  if (st) return st;
  if (!dev_signs || !canon_signs) { set_error("gale_debug_unpack_signs: NULL pointer"); return GALE_ERR_NULL; }
  return hip_status("gale_debug_unpack_signs", launch_debug_unpack(rows, cols, dev_signs, canon_signs, stream));
}

extern "C" int gale_debug_unpack_outliers(int32_t rows, int64_t nnz, const gale_matrix* m_host,
                                          int32_t* out_row, int32_t* out_col, int32_t* out_val,
                                          hipStream_t stream) {
  if (!m_host) { set_error("gale_debug_unpack_outliers: NULL descriptor"); return GALE_ERR_NULL; }
  if (rows < 1 || nnz < 0) { set_error("gale_debug_unpack_outliers: bad shape"); return GALE_ERR_SHAPE; }
  if (nnz > 0 && (!m_host->row_ptr || !m_host->out_cols || !m_host->out_vals)) {
    set_error("gale_debug_unpack_outliers: NULL section");
    return GALE_ERR_NULL;
  }
  return hip_status("gale_debug_unpack_outliers", launch_debug_outliers(rows, nnz, *m_host, out_row, out_col, out_val, stream));
}

// ============================================================================
// FWHT
// ============================================================================
extern "C" int gale_fwht1024(const void* x, void* y, int64_t n_vec, int32_t len, int32_t in_dtype,
                             int32_t out_dtype, hipStream_t stream) {
  if (!x || !y) { set_error("gale_fwht1024: NULL pointer"); return GALE_ERR_NULL; }
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) { set_error("gale_fwht1024: bad dtype"); return GALE_ERR_DTYPE; }
  if (len < 1024 || len % 1024 || n_vec < 0) { set_error("gale_fwht1024: len=%d must be a positive multiple of 1024", len); return GALE_ERR_SHAPE; }
  if (x == y && in_dtype != out_dtype) { set_error("gale_fwht1024: in place needs equal dtypes"); return GALE_ERR_DTYPE; }
  if (!aligned(x, 16) || !aligned(y, 16)) { set_error("gale_fwht1024: x and y must be 16-byte aligned"); return GALE_ERR_ALIGN; }
  return hip_status("gale_fwht1024", launch_fwht(x, y, n_vec, len, in_dtype, out_dtype, stream));
}

// ============================================================================
// GEMV
// ============================================================================
extern "C" size_t gale_prepared_bytes(int32_t len) {
  if (len < 1024 || len % 1024) return 0;
  return ra_bytes(len);
}

extern "C" int gale_prepare_activations(const void* x, int32_t x_dtype, int64_t n_vec, int32_t len, uint32_t flags,
                                        void* out, size_t out_bytes, hipStream_t stream) {
  const char* fn = "gale_prepare_activations";
  if (!x || !out) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (!dtype_ok(x_dtype)) { set_error("%s: bad dtype", fn); return GALE_ERR_DTYPE; }
  if (len < 1024 || len % 1024 || len > GALE_MAX_COLS || n_vec < 0 || n_vec > (1 << 30)) {
    set_error("%s: len=%d n_vec=%lld", fn, len, (long long)n_vec);
    return GALE_ERR_SHAPE;
  }
  if (!aligned(x, 16) || !aligned(out, 256)) { set_error("%s: x needs 16-byte, out 256-byte alignment", fn); return GALE_ERR_ALIGN; }
  if (out_bytes < ra_bytes(len) * (size_t)n_vec) { set_error("%s: out %zu < %zu bytes", fn, out_bytes, ra_bytes(len) * (size_t)n_vec); return GALE_ERR_WORKSPACE; }
  return hip_status(fn, launch_prep(x, x_dtype, len, (int)n_vec, len, (flags & GALE_X_ROTATED) ? 1 : 0,
                                    reinterpret_cast<uint8_t*>(out), ra_bytes(len), stream));
}

extern "C" size_t gale_gemv_workspace_bytes(int32_t rows, int32_t cols, int32_t n_mat, int32_t n_tok,
                                            int32_t x_shared) {
  (void)rows;
  if (cols < 1024 || n_mat < 1 || n_tok < 1) return 0;
  return gemv_ws(cols, (int64_t)(x_shared ? 1 : n_mat) * n_tok).total;
}

extern "C" int gale_expert_gemv(int32_t rows, int32_t cols, const gale_matrix* mats_dev, int32_t n_mat,
                                const void* x, int32_t x_dtype, int32_t x_shared, int32_t n_tok,
                                void* y, int32_t y_dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                hipStream_t stream) {
  const char* fn = "gale_expert_gemv";
  int st = check_matrix_shape(fn, rows, cols);
  if (st) return st;
  if (n_mat < 1 || n_tok < 1) { set_error("%s: n_mat=%d n_tok=%d must be >= 1", fn, n_mat, n_tok); return GALE_ERR_SHAPE; }
  const bool prepared = (flags & GALE_X_PREPARED) != 0;
  if (!mats_dev || !x || !y || (!prepared && !ws)) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if ((!prepared && !dtype_ok(x_dtype)) || !dtype_ok(y_dtype)) { set_error("%s: bad dtype", fn); return GALE_ERR_DTYPE; }
  if (!aligned(x, prepared ? 256 : 16) || (!prepared && !aligned(ws, 256)) || !aligned(y, dsize(y_dtype)) ||
      !aligned(mats_dev, 8)) {
    set_error("%s: x needs 16-byte (prepared: 256-byte), ws 256-byte alignment", fn);
    return GALE_ERR_ALIGN;
  }
  const int64_t n_x = (int64_t)(x_shared ? 1 : n_mat) * n_tok;
  // one token per matrix, at most eight 1024-column chunks: the GEMV rotates and splits x
  // itself (one launch, no record in memory)
  const int slots = pick_slots(n_tok);
  const int out_chunks = pick_out_chunks(flags, slots, cols, 0, cols);
  const bool fused = !prepared && n_tok == 1 && raw_x_ok(cols, 0, flags, cols);
  const uint8_t* ra = nullptr;
  if (!prepared) {
    // the workspace contract does not depend on which path runs
    const GemvWs W = gemv_ws(cols, n_x);
    if (ws_bytes < W.total) { set_error("%s: workspace %zu < %zu bytes", fn, ws_bytes, W.total); return GALE_ERR_WORKSPACE; }
  }
  if (prepared) {
    ra = reinterpret_cast<const uint8_t*>(x);
  } else if (!fused) {
    const GemvWs W = gemv_ws(cols, n_x);
    uint8_t* raw = reinterpret_cast<uint8_t*>(ws) + W.ra;
    st = hip_status(fn, launch_prep(x, x_dtype, cols, (int)n_x, cols, (flags & GALE_X_ROTATED) ? 1 : 0, raw,
                                    ra_bytes(cols), stream));
    if (st) return st;
    ra = raw;
  }
  GemvParams P;
  memset(&P, 0, sizeof(P));
  P.table = mats_dev;
  P.mat_stride = 1;
  P.sel0 = P.sel1 = 0;
  P.rows = rows;
  P.cols = cols;
  P.ra = ra;
  P.ra_stride = ra_bytes(cols);
  P.implicit_items = 1;
  P.n_tok = n_tok;
  P.n_groups = (n_tok + slots - 1) / slots;
  P.x_shared = x_shared ? 1 : 0;
  P.n_items = n_mat * P.n_groups;
  P.ra_div = 1;
  P.y = y;
  P.y_dtype = y_dtype;
  P.y_stride = rows;
  P.gateup = 0;
  const int ntiles = rows / 16;
  P.out_chunks = out_chunks;
  const int R = pick_tiles(P.n_items, ntiles, cols, slots, P.out_chunks, flags);
  P.row_groups = (ntiles + R - 1) / R;
  P.stage_xt = stage_ok(cols, slots);
  if (fused) {
    P.x = x;
    P.x_dtype = x_dtype;
    P.x_rotated = (flags & GALE_X_ROTATED) ? 1 : 0;
    P.x_stride = cols;
  }
  return hip_status(fn, launch_gemv(P, slots, R, (int64_t)P.n_items * P.row_groups, stream));
}

// ============================================================================
// expert FFN
// ============================================================================
extern "C" size_t gale_ffn_workspace_bytes(int32_t hidden, int32_t inter, int32_t n_exp, int32_t n_tok,
                                           int32_t x_shared) {
  if (hidden < 1024 || inter < 1024 || n_exp < 1 || n_tok < 1) return 0;
  return ffn_ws(hidden, inter, (int64_t)(x_shared ? 1 : n_exp) * n_tok, (int64_t)n_exp * n_tok).total;
}

static int run_gemv_phase(const char* fn, const gale_matrix* table, int stride, int sel0, int sel1,
                          int rows, int cols, const uint8_t* ra, int implicit, int n_tok, int x_shared,
                          int n_items, const WorkItem* items, const int32_t* n_items_dev, int ra_div,
                          int item_bound, void* y, int y_dtype, int gateup, int slots, uint32_t flags,
                          hipStream_t s, int ref_cols, const void* raw_x = nullptr, int raw_dtype = 0) {
  GemvParams P;
  memset(&P, 0, sizeof(P));
  P.table = table;
  P.mat_stride = stride;
  P.sel0 = sel0;
  P.sel1 = sel1;
  P.rows = rows;
  P.cols = cols;
  P.ra = ra;
  P.ra_stride = ra_bytes(cols);
  P.implicit_items = implicit;
  P.n_tok = n_tok;
  P.n_groups = implicit ? (n_tok + slots - 1) / slots : 0;
  P.x_shared = x_shared;
  P.n_items = n_items;
  P.items = items;
  P.n_items_dev = n_items_dev;
  P.ra_div = ra_div;
  P.y = y;
  P.y_dtype = y_dtype;
  P.y_stride = rows;
  P.gateup = gateup;
  const int ntiles = rows / 16;
  const int64_t bound = implicit ? n_items : item_bound;
  P.out_chunks = pick_out_chunks(flags, slots, cols, gateup, ref_cols);
  const int R = pick_tiles(bound, ntiles, cols, slots, P.out_chunks, flags);
  P.row_groups = (ntiles + R - 1) / R;
  P.stage_xt = stage_ok(cols, slots);
  if (raw_x) {
    P.x = raw_x;
    P.x_dtype = raw_dtype;
    P.x_stride = cols;
  }
  return hip_status(fn, launch_gemv(P, slots, R, bound * P.row_groups, s));
}


extern "C" int gale_expert_ffn(int32_t hidden, int32_t inter, const gale_expert* experts_dev, int32_t n_exp,
                               const void* x, int32_t x_shared, int32_t n_tok, void* y, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  const char* fn = "gale_expert_ffn";
  int st = check_matrix_shape(fn, inter, hidden);
  if (st) return st;
  st = check_matrix_shape(fn, hidden, inter);
  if (st) return st;
  if (hidden > GALE_MAX_HIDDEN) {
    set_error("%s: hidden=%d above %d", fn, hidden, GALE_MAX_HIDDEN);
    return GALE_ERR_SHAPE;
  }
  if (n_exp < 1 || n_tok < 1) { set_error("%s: n_exp=%d n_tok=%d must be >= 1", fn, n_exp, n_tok); return GALE_ERR_SHAPE; }
  if (!experts_dev || !x || !y || !ws) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(y, 2)) { set_error("%s: misaligned pointer", fn); return GALE_ERR_ALIGN; }
  const int64_t n_x = (int64_t)(x_shared ? 1 : n_exp) * n_tok;
  const int64_t n_p = (int64_t)n_exp * n_tok;
  const FfnWs W = ffn_ws(hidden, inter, n_x, n_p);
  if (ws_bytes < W.total) { set_error("%s: workspace %zu < %zu bytes", fn, ws_bytes, W.total); return GALE_ERR_WORKSPACE; }
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint8_t* ra_x = base + W.ra_x;
  float* h = reinterpret_cast<float*>(base + W.h);
  uint8_t* ra_h = base + W.ra_h;
  const gale_matrix* table = reinterpret_cast<const gale_matrix*>(experts_dev);
  const int slots = pick_slots(n_tok);
  // one token per expert: each GEMV phase rotates and splits its input itself (same bits)
  const bool raw_up = n_tok == 1 && raw_x_ok(hidden, 1, 0, hidden);
  const bool raw_down = n_tok == 1 && raw_x_ok(inter, 0, 0, hidden);
  if (!raw_up) {
    st = hip_status(fn, launch_prep(x, GALE_F16, hidden, (int)n_x, hidden, 0, ra_x, ra_bytes(hidden), stream));
    if (st) return st;
  }
  const int n_groups = (n_tok + slots - 1) / slots;
  st = run_gemv_phase(fn, table, 3, 0, 1, inter, hidden, ra_x, 1, n_tok, x_shared ? 1 : 0, n_exp * n_groups,
                      nullptr, nullptr, 1, 0, h, GALE_F32, 1, slots, 0, stream, hidden, raw_up ? x : nullptr,
                      GALE_F16);
  if (st) return st;
  if (!raw_down) {
    st = hip_status(fn, launch_prep(h, GALE_F32, inter, (int)n_p, inter, 0, ra_h, ra_bytes(inter), stream));
    if (st) return st;
  }
  return run_gemv_phase(fn, table, 3, 2, 2, hidden, inter, ra_h, 1, n_tok, 0, n_exp * n_groups, nullptr,
                        nullptr, 1, 0, y, GALE_F16, 0, slots, 0, stream, hidden, raw_down ? h : nullptr, GALE_F32);
}

// ============================================================================
// routed layer
// ============================================================================
extern "C" size_t gale_moe_workspace_bytes(int32_t n_tok, int32_t n_experts, int32_t top_k, int32_t hidden,
                                           int32_t inter, uint32_t flags) {
  if (n_tok < 1 || n_experts < 1 || top_k < 1 || hidden < 1024 || inter < 1024) return 0;
  return moe_ws(n_tok, n_experts, top_k, hidden, inter, moe_path(n_tok, flags)).total;
}

static int moe_layer(const char* fn, int32_t hidden, int32_t inter, const gale_expert* experts_dev,
                     int32_t n_experts, const float* logits, const float* select_bias, const int32_t* fixed_idx,
                     int32_t top_k, const void* x, int32_t n_tok, void* y, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, uint32_t flags, hipStream_t stream) {
  int st = check_matrix_shape(fn, inter, hidden);
  if (st) return st;
  st = check_matrix_shape(fn, hidden, inter);
  if (st) return st;
  if (hidden > GALE_MAX_HIDDEN) {
    set_error("%s: hidden=%d above %d", fn, hidden, GALE_MAX_HIDDEN);
    return GALE_ERR_SHAPE;
  }
  if (n_experts < 1 || n_experts > GALE_MAX_EXPERTS || top_k < 1 || top_k > GALE_MAX_TOPK || top_k > n_experts) {
    set_error("%s: n_experts=%d top_k=%d out of range", fn, n_experts, top_k);
    return GALE_ERR_SHAPE;
  }
  if (n_tok < 1) { set_error("%s: n_tok=%d", fn, n_tok); return GALE_ERR_SHAPE; }
  if (!experts_dev || !logits || !x || !y || !ws) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(y, 2) || !aligned(logits, 4) || !aligned(select_bias, 4) ||
      !aligned(fixed_idx, 4)) {
    set_error("%s: misaligned pointer", fn);
    return GALE_ERR_ALIGN;
  }
  if (select_bias && fixed_idx) { set_error("%s: a selection bias and fixed experts exclude each other", fn); return GALE_ERR_SHAPE; }
  const RouteIn rin = {logits, select_bias, fixed_idx};
  if ((flags & GALE_PATH_DECODE) && (flags & GALE_PATH_GROUPED)) { set_error("%s: both paths forced", fn); return GALE_ERR_SHAPE; }
  const MoePath path = moe_path(n_tok, flags);
  if (path == kDecode && n_tok > GALE_MAX_DECODE_TOKENS) {
    set_error("%s: the decode path takes at most %d tokens", fn, GALE_MAX_DECODE_TOKENS);
    return GALE_ERR_SHAPE;
  }
  const MoeWs W = moe_ws(n_tok, n_experts, top_k, hidden, inter, path);
  if (ws_bytes < W.total) { set_error("%s: workspace %zu < %zu bytes", fn, ws_bytes, W.total); return GALE_ERR_WORKSPACE; }
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(base + W.idx);
  float* wts = topk_w ? topk_w : reinterpret_cast<float*>(base + W.w);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + W.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(base + W.perm);
  int32_t* n_items = reinterpret_cast<int32_t*>(base + W.n_items);
  float* h = reinterpret_cast<float*>(base + W.h);
  float* yp = reinterpret_cast<float*>(base + W.yp);
  const int P = n_tok * top_k;
  const int slots = pick_moe_slots(n_tok, top_k, n_experts, path != kDecode);
  const gale_matrix* table = reinterpret_cast<const gale_matrix*>(experts_dev);
  if (path != kDecode) {
    // chunked top-k and a stable sort of the pairs by expert
    st = hip_status(fn, launch_route_large(rin, n_tok, n_experts, top_k, idx, wts,
                                           reinterpret_cast<int32_t*>(base + W.chunk), offsets, perm, stream));
    if (st) return st;
  }
  const bool use_items = path != kGroupedGemm;
  const bool use_gemm = path == kGroupedGemm || path == kGroupedHybrid;
  WorkItem* items = reinterpret_cast<WorkItem*>(base + W.items);
  uint8_t* ra_x = base + W.ra_x;
  uint8_t* ra_h = base + W.ra_h;
  GemmTile* tiles = reinterpret_cast<GemmTile*>(base + W.tiles);
  int32_t* n_tiles = n_items + 16;
  uint16_t* xt16 = reinterpret_cast<uint16_t*>(base + W.xt16);
  uint16_t* ht16 = reinterpret_cast<uint16_t*>(base + W.ht16);
  const int max_tiles = use_gemm ? (int)moe_tile_bound(n_tok, n_experts, top_k) : 0;
  // hybrid: experts with at least kGemmMinPairs pairs run as GEMM tiles, the rest as items
  const int split = path == kGroupedHybrid ? kGemmMinPairs : (path == kGroupedGemm ? 1 : INT_MAX);
  // hybrid: each side rotates only the tokens and pairs it reads
  VecFilter tok_items, tok_gemm, pair_items, pair_gemm;
  if (path == kGroupedHybrid) {
    tok_items.idx = tok_gemm.idx = pair_items.idx = pair_gemm.idx = idx;
    tok_items.offsets = tok_gemm.offsets = pair_items.offsets = pair_gemm.offsets = offsets;
    tok_items.top_k = tok_gemm.top_k = top_k;
    tok_items.per_token = tok_gemm.per_token = 1;
    tok_items.split = tok_gemm.split = pair_items.split = pair_gemm.split = split;
    tok_items.items_side = pair_items.items_side = 1;
  }
  if (path == kDecode && n_tok == 1 && !(flags & GALE_DECODE_STAGED) && decode_layer_supported(hidden, inter, top_k)) {
    // one launch for the whole layer; its synchronisation words start the workspace
    gale_layer_io io;
    io.experts = experts_dev;
    io.logits = logits;
    io.select_bias = select_bias;
    io.fixed_idx = fixed_idx;
    io.x = x;
    io.y = y;
    io.topk_idx = topk_idx;
    io.topk_w = topk_w;
    const int forced = (int)((flags >> GALE_TILES_SHIFT) & 0xF);
    return hip_status(fn, launch_decode_stack(io, nullptr, 1, n_experts, top_k, hidden, inter, h, ra_h,
                                              reinterpret_cast<uint64_t*>(base + W.sync), forced,
                                              decode_wait_ticks(flags), stream));
  }
  // decode items of one vector: each GEMV phase rotates and splits its input itself (same bits)
  const bool raw_up = path == kDecode && slots == 1 && raw_x_ok(hidden, 1, flags, hidden);
  const bool raw_down = path == kDecode && slots == 1 && raw_x_ok(inter, 0, flags, hidden);
  if (path == kDecode) {
    st = hip_status(fn, launch_route_prep(rin, n_tok, n_experts, top_k, idx, wts, items, n_items, slots, x,
                                          GALE_F16, hidden, raw_up ? nullptr : ra_x, ra_bytes(hidden), stream));
    if (st) return st;
  } else {
    if (use_items) {
      st = hip_status(fn, launch_build_items(offsets, perm, n_experts, slots, split, items, n_items, stream));
      if (st) return st;
      st = hip_status(fn, launch_prep(x, GALE_F16, hidden, n_tok, hidden, 0, ra_x, ra_bytes(hidden), stream, tok_items));
      if (st) return st;
    }
    if (use_gemm) {
      st = hip_status(fn, launch_build_tiles(offsets, n_experts, split, tiles, n_tiles, stream));
      if (st) return st;
      st = hip_status(fn, launch_rotate_f16(x, GALE_F16, n_tok, hidden, xt16, stream, tok_gemm));
      if (st) return st;
    }
  }
  const int bound = (int)moe_item_bound(n_tok, n_experts, top_k, slots);
  // gate/up + SwiGLU: h[pair]
  if (use_items) {
    st = run_gemv_phase(fn, table, 3, 0, 1, inter, hidden, ra_x, 0, 0, 0, 0, items, n_items, top_k, bound, h,
                        GALE_F32, 1, slots, flags, stream, hidden, raw_up ? x : nullptr, GALE_F16);
    if (st) return st;
  }
  if (use_gemm) {
    st = hip_status(fn, launch_grouped_gemm(table, 1, inter, hidden, offsets, perm, top_k, tiles, n_tiles, max_tiles,
                                            xt16, h, inter, stream));
    if (st) return st;
  }
  // rotate h; down: yp[pair]
  if (use_items) {
    if (!raw_down) {
      st = hip_status(fn, launch_prep(h, GALE_F32, inter, P, inter, 0, ra_h, ra_bytes(inter), stream, pair_items));
      if (st) return st;
    }
    st = run_gemv_phase(fn, table, 3, 2, 2, hidden, inter, ra_h, 0, 0, 0, 0, items, n_items, 1, bound, yp,
                        GALE_F32, 0, slots, flags, stream, hidden, raw_down ? h : nullptr, GALE_F32);
    if (st) return st;
  }
  if (use_gemm) {
    st = hip_status(fn, launch_rotate_f16(h, GALE_F32, P, inter, ht16, stream, pair_gemm));
    if (st) return st;
    st = hip_status(fn, launch_grouped_gemm(table, 0, hidden, inter, offsets, perm, top_k, tiles, n_tiles,
                                            max_tiles, ht16, yp, hidden, stream));
    if (st) return st;
  }
  return hip_status(fn, launch_combine(yp, wts, n_tok, top_k, hidden, y, GALE_F16, stream));
}

extern "C" int gale_moe_layer_fwd(int32_t hidden, int32_t inter, const gale_expert* experts_dev,
                                  int32_t n_experts, const float* logits, int32_t top_k, const void* x,
                                  int32_t n_tok, void* y, int32_t* topk_idx, float* topk_w, void* ws,
                                  size_t ws_bytes, uint32_t flags, hipStream_t stream) {
  return moe_layer("gale_moe_layer_fwd", hidden, inter, experts_dev, n_experts, logits, nullptr, nullptr, top_k, x,
                   n_tok, y, topk_idx, topk_w, ws, ws_bytes, flags, stream);
}

extern "C" int gale_moe_layer_fwd_routed(int32_t hidden, int32_t inter, const gale_expert* experts_dev,
                                         int32_t n_experts, const float* logits, const float* select_bias,
                                         const int32_t* fixed_idx, int32_t top_k, const void* x, int32_t n_tok,
                                         void* y, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                                         uint32_t flags, hipStream_t stream) {
  return moe_layer("gale_moe_layer_fwd_routed", hidden, inter, experts_dev, n_experts, logits, select_bias, fixed_idx,
                   top_k, x, n_tok, y, topk_idx, topk_w, ws, ws_bytes, flags, stream);
}

extern "C" size_t gale_route_workspace_bytes(int32_t n_tok, int32_t n_experts) {
  if (n_tok < 1 || n_experts < 1) return 0;
  return align256(route_chunk_count_bytes(n_tok, n_experts));
}

extern "C" int gale_route_topk(const float* logits, int32_t n_tok, int32_t n_experts, int32_t top_k,
                               int32_t* topk_idx, float* topk_w, int32_t* offsets, int32_t* perm,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "gale_route_topk";
  if (!logits || !topk_idx || !topk_w) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (n_tok < 1 || n_experts < 1 || n_experts > GALE_MAX_EXPERTS || top_k < 1 || top_k > GALE_MAX_TOPK ||
      top_k > n_experts) {
    set_error("%s: bad sizes n_tok=%d n_experts=%d top_k=%d", fn, n_tok, n_experts, top_k);
    return GALE_ERR_SHAPE;
  }
  if ((offsets == nullptr) != (perm == nullptr)) { set_error("%s: offsets and perm go together", fn); return GALE_ERR_NULL; }
  if (!aligned(logits, 4)) { set_error("%s: misaligned logits", fn); return GALE_ERR_ALIGN; }
  if (offsets && n_tok > GALE_MAX_DECODE_TOKENS) {
    const size_t need = gale_route_workspace_bytes(n_tok, n_experts);
    if (!ws || ws_bytes < need) { set_error("%s: workspace %zu < %zu bytes", fn, ws_bytes, need); return GALE_ERR_WORKSPACE; }
    return hip_status(fn, launch_route_large(RouteIn{logits, nullptr, nullptr}, n_tok, n_experts, top_k, topk_idx,
                                             topk_w, reinterpret_cast<int32_t*>(ws), offsets, perm, stream));
  }
  if (n_tok <= GALE_MAX_DECODE_TOKENS)
    return hip_status(fn, launch_route_small(RouteIn{logits, nullptr, nullptr}, n_tok, n_experts, top_k, topk_idx,
                                             topk_w, offsets, perm, nullptr, nullptr, 1, stream));
  // top-k only, any number of tokens: the chunked kernel without grouping
  return hip_status(fn, launch_route_large(RouteIn{logits, nullptr, nullptr}, n_tok, n_experts, top_k, topk_idx,
                                           topk_w, nullptr, nullptr, nullptr, stream));
}

// ============================================================================
// one token through a stack of layers; the synchronisation words
// ============================================================================
extern "C" size_t gale_decode_stack_workspace_bytes(int32_t hidden, int32_t inter, int32_t top_k) {
  if (hidden < 1024 || inter < 1024 || top_k < 1 || top_k > GALE_MAX_TOPK) return 0;
  return align256(kDecodeSyncBytes) + align256(decode_stack_h_bytes(inter, top_k)) +
         align256(decode_stack_rec_bytes(inter, top_k));
}

// Host validation shared by the two stack entry points (ws == NULL is checked by the caller).
static int decode_stack_check(const char* fn, int32_t hidden, int32_t inter, int32_t n_experts, int32_t top_k,
                              int32_t n_layers, const gale_layer_io* layers_dev) {
  int st = check_matrix_shape(fn, inter, hidden);
  if (st) return st;
  st = check_matrix_shape(fn, hidden, inter);
  if (st) return st;
  if (n_layers < 1) { set_error("%s: n_layers=%d", fn, n_layers); return GALE_ERR_SHAPE; }
  if (n_experts < 1 || n_experts > GALE_MAX_EXPERTS || top_k < 1 || top_k > GALE_MAX_TOPK || top_k > n_experts) {
    set_error("%s: n_experts=%d top_k=%d out of range", fn, n_experts, top_k);
    return GALE_ERR_SHAPE;
  }
  if (!decode_layer_supported(hidden, inter, top_k)) {
    set_error("%s: hidden=%d inter=%d top_k=%d is not a shape of the one-launch decode", fn, hidden, inter, top_k);
    return GALE_ERR_UNSUPPORTED;
  }
  if (!layers_dev) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (!aligned(layers_dev, 8)) { set_error("%s: misaligned pointer", fn); return GALE_ERR_ALIGN; }
  return GALE_OK;
}

extern "C" int gale_moe_decode_stack(int32_t hidden, int32_t inter, int32_t n_experts, int32_t top_k,
                                     int32_t n_layers, const gale_layer_io* layers_dev, void* ws, size_t ws_bytes,
                                     uint32_t flags, hipStream_t stream) {
  const char* fn = "gale_moe_decode_stack";
  int st = decode_stack_check(fn, hidden, inter, n_experts, top_k, n_layers, layers_dev);
  if (st) return st;
  if (!ws) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (!aligned(ws, 256)) { set_error("%s: misaligned pointer", fn); return GALE_ERR_ALIGN; }
  const size_t need = gale_decode_stack_workspace_bytes(hidden, inter, top_k);
  if (ws_bytes < need) { set_error("%s: workspace %zu < %zu bytes", fn, ws_bytes, need); return GALE_ERR_WORKSPACE; }
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  float* h = reinterpret_cast<float*>(base + align256(kDecodeSyncBytes));
  uint8_t* rec = base + align256(kDecodeSyncBytes) + align256(decode_stack_h_bytes(inter, top_k));
  gale_layer_io none;
  memset(&none, 0, sizeof(none));
  const int forced = (int)((flags >> GALE_TILES_SHIFT) & 0xF);
  return hip_status(fn, launch_decode_stack(none, layers_dev, n_layers, n_experts, top_k, hidden, inter, h, rec,
                                            reinterpret_cast<uint64_t*>(base), forced, decode_wait_ticks(flags),
                                            stream));
}

extern "C" int gale_sync_init(void* ws, hipStream_t stream) {
  const char* fn = "gale_sync_init";
  if (!ws) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  if (!aligned(ws, 256)) { set_error("%s: misaligned workspace", fn); return GALE_ERR_ALIGN; }
  return hip_status(fn, launch_sync_init(ws, stream));
}

extern "C" int gale_sync_status(const void* ws, uint64_t* words_host) {
  const char* fn = "gale_sync_status";
  if (!ws) { set_error("%s: NULL pointer", fn); return GALE_ERR_NULL; }
  uint64_t w[3] = {0, 0, 0};
  const hipError_t e = hipMemcpy(w, ws, sizeof(w), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(fn, e);
  if (words_host) memcpy(words_host, w, sizeof(w));
  switch (sync_words_state(w)) {
    case 0: return GALE_OK;
    case 1:
      set_error("%s: the synchronisation words were never zeroed (gale_sync_init)", fn);
      return GALE_ERR_SYNC;
    default:
      set_error("%s: a cross-workgroup wait gave up in an earlier call (error bits 0x%llx); outputs of that "
                "call are unspecified, calls compute nothing until gale_sync_init", fn, (unsigned long long)w[2]);
      return GALE_ERR_SYNC;
  }
}

extern "C" int gale_moe_decode_stack_static(int32_t hidden, int32_t inter, int32_t n_experts, int32_t top_k,
                                            int32_t n_layers, const gale_layer_io* layers_dev, uint32_t flags,
                                            hipStream_t stream) {
  const char* fn = "gale_moe_decode_stack_static";
  int st = decode_stack_check(fn, hidden, inter, n_experts, top_k, n_layers, layers_dev);
  if (st) return st;
  const size_t need = gale_decode_stack_workspace_bytes(hidden, inter, top_k);
  if (need > (size_t)GALE_STATIC_SCRATCH_BYTES) {
    set_error("%s: hidden=%d inter=%d top_k=%d needs %zu workspace bytes, above the static array's %d", fn, hidden,
              inter, top_k, need, GALE_STATIC_SCRATCH_BYTES);
    return GALE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  st = hip_status(fn, static_scratch(&ws));
  if (st) return st;
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  // every call starts from zeroed synchronisation words (the array keeps the last call's)
  st = hip_status(fn, launch_sync_init(base, stream));
  if (st) return st;
  float* h = reinterpret_cast<float*>(base + align256(kDecodeSyncBytes));
  uint8_t* rec = base + align256(kDecodeSyncBytes) + align256(decode_stack_h_bytes(inter, top_k));
  gale_layer_io none;
  memset(&none, 0, sizeof(none));
  const int forced = (int)((flags >> GALE_TILES_SHIFT) & 0xF);
  return hip_status(fn, launch_decode_stack(none, layers_dev, n_layers, n_experts, top_k, hidden, inter, h, rec,
                                            reinterpret_cast<uint64_t*>(base), forced, decode_wait_ticks(flags),
                                            stream));
}
