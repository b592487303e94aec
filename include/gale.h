/*
 * gale.h - C ABI of libgale: the GALE 1-bit routed-expert matmul on one AMD
 * Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V4-Flash GALE 1-bit model card, "What is in the pack"):
 * every routed-expert matrix Wq [rows, cols] stores one sign bit per weight under
 * a blocked FWHT-1024 rotation of the input, an fp16 scale per 128-weight block,
 * and about 1 % outliers as int4 values with a per-row fp16 scale.  A product is
 *     y = Wq . (blockdiag(H_1024) . x),   H[i][j] = (-1)^popcount(i & j) / 32,
 * with Wq[n][k] = s[n][k/128] * (1 - 2 b[n][k]) + r[n] * q at each outlier (n, k).
 * The expert FFN (w1 gate, w3 up, w2 down; same card, "What is in the pack") is
 *     h = silu(w1 . H x) * (w3 . H x),   y = w2 . (H h),
 * and a routed layer sums the top-k experts of each token weighted by the softmax
 * of their router logits (same card, "Measured performance": 43 x 6 experts per token).
 * The decode kernels multiply straight out of the packed record, as the
 * DeepSeek-V4-Pro-671B-GALE-1bit-v4 page describes for its direct GEMV (serving
 * knobs paragraph, DSV4_DIRECT_GEMV) and its single-kernel Walsh-Hadamard
 * transform (DSV4_FWHT=butterfly).
 *
 * Conventions for every entry point
 *  - Pointers are device pointers unless a comment says "host".
 *  - The caller owns every buffer (weights, descriptor tables, activations,
 *    outputs, workspace).  The library never allocates or frees memory and keeps
 *    no state except a thread-local error message.
 *  - Compute calls enqueue on `stream` and return without synchronising.  They
 *    make no allocation, no synchronisation and no host<->device copy.
 *  - Arguments are validated on the host before anything is enqueued; a call that
 *    returns an error has enqueued nothing.  Launch failures return GALE_ERR_HIP.
 *    Device faults surface at the caller's next synchronisation.
 *  - Descriptor contents (pointers, CSR offsets) are trusted on the device; use
 *    gale_check_canonical() on the host to validate canonical data before packing.
 *  - fp16 values are IEEE binary16 bit patterns (uint16_t); fp16 outputs are
 *    rounded to nearest even; subnormal fp16 scales are honoured.
 */
#ifndef GALE_H
#define GALE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define GALE_OK               0
#define GALE_ERR_NULL        (-1)  /* a required pointer is NULL */
#define GALE_ERR_SHAPE       (-2)  /* a size is out of range or inconsistent */
#define GALE_ERR_DTYPE       (-3)  /* unknown dtype code */
#define GALE_ERR_ALIGN       (-4)  /* a pointer is not aligned as required */
#define GALE_ERR_WORKSPACE   (-5)  /* workspace missing or too small */
#define GALE_ERR_UNSUPPORTED (-6)  /* valid request the library does not implement */
#define GALE_ERR_FORMAT      (-7)  /* canonical data violates the format */
#define GALE_ERR_HIP         (-8)  /* a HIP runtime call failed */
#define GALE_ERR_SYNC        (-9)  /* gale_sync_status: the one-launch decode's synchronisation words
                                      were never zeroed, or a wait in an earlier call gave up */

/* ---- dtype codes and flags ---------------------------------------------- */
#define GALE_F16 1
#define GALE_F32 2

#define GALE_X_ROTATED    0x1u   /* x is already H.x (fp32 or fp16); skip the rotation */
#define GALE_X_PREPARED   0x2u   /* gale_expert_gemv: x holds records from gale_prepare_activations */
#define GALE_PATH_DECODE  0x10u  /* gale_moe_layer_fwd: force the per-expert GEMV path */
#define GALE_PATH_GROUPED 0x20u  /* gale_moe_layer_fwd: force the grouped (token-sorted) path */
#define GALE_GROUPED_ITEMS 0x40u /* gale_moe_layer_fwd grouped path: GEMV work items only */
#define GALE_GROUPED_GEMM  0x80u /* gale_moe_layer_fwd grouped path: fp16 MFMA tile GEMM only */
#define GALE_DECODE_STAGED 0x1000u /* gale_moe_layer_fwd, one token: the five-launch decode sequence
                                      instead of the one-launch layer kernel */
/* Tuning knob, bits 8..11: a value v != 0 fixes the row tiles (16 rows each) per work unit
 * instead of the built-in choice.  GEMV kernels: 2^(v-1) (capped where registers run out).
 * One-launch decode (one token): v = 1, 2 or 3 gate/up tiles per unit (at most hidden / 1024).
 * Results do not depend on it. */
#define GALE_TILES_SHIFT 8
/* Tuning knob, bits 14..15: outlier entries that a GEMV wavefront stages per work unit for
 * its 16 rows.  v = 0: 1024 (64 per row on average, the 1 % budget's 41 fit); 1: 2048;
 * 2: 4096 (one activation vector per item only; with more, as 1).  Entries past the staged
 * ones are read from HBM one by one, which is slow; a larger staging takes registers from the
 * row tiles per unit.  For budgets of 2 to 3 % take 1, from 4 % take 2.  In the expert FFN
 * and MoE layer the value describes w1/w3; the down phase stages half as many entries for
 * each halving of its columns (a budget is a share of each row).  The one-token layer
 * kernel ignores it.  Results do not depend on it. */
#define GALE_OUTLIER_STAGE_SHIFT 14
/* Test knob for the one-launch decode: every cross-workgroup wait gives up at once, as one whose
 * time budget ran out would (the call then records the give-up in its synchronisation words and
 * its outputs are unspecified).  Every kernel still ends normally. */
#define GALE_SYNC_NO_WAIT 0x10000u

/* ---- limits -------------------------------------------------------------- */
#define GALE_FWHT_N        1024   /* rotation block ("blocked FWHT-1024") */
#define GALE_SCALE_BLOCK    128   /* weights per fp16 block scale */
#define GALE_MAX_COLS     16384   /* cols: multiple of 1024, at most this */
#define GALE_MAX_ROWS   1048576   /* rows: multiple of 16, at most this */
#define GALE_MAX_HIDDEN    8192   /* expert FFN / MoE hidden size: the w1/w3 GEMV runs one wavefront
                                   per 1024 columns of each matrix in one workgroup of at most
                                   1024 threads */
#define GALE_MAX_TOPK         8
#define GALE_MAX_EXPERTS    512
#define GALE_MAX_DECODE_TOKENS 64 /* gale_moe_layer_fwd decode path limit */

/*
 * Device layout of one packed matrix (produced by gale_pack_*), rows % 16 == 0,
 * cols % 1024 == 0, C = cols / 1024:
 *  signs         uint32 [rows/16][C][2][64][4]   (rows*cols/32 words, 16-byte aligned)
 *      word (t, c, h, l, e) holds, for row n = 16 t + (l % 16), g = l / 16 and
 *      scale block d = 4 h + p (p in 0..3), bit (4 i + p) = b[n][1024 c + 128 d + kh],
 *      kh = 64 (g % 2) + 16 (g / 2) + 32 (e / 2) + 8 (e % 2) + i, i in 0..7
 *      (the element order of an fp4 operand of the 16x16x128 MFMA, so that one
 *      AND of a word yields one operand dword of block d).  One 2 KB tile =
 *      16 rows x 1024 columns, read by one wavefront as two fully coalesced 1 KB
 *      dwordx4 loads.
 *  block_scales  fp16 [rows/16][C][16][8]: s[16 t + r][8 c + d] (16-byte aligned)
 *  row_scales    fp16 [rows]                 (canonical)
 *  row_ptr       int32 [rows + 1]            (canonical CSR offsets)
 *  out_cols      uint16 [nnz]                (canonical, ascending within a row)
 *  out_vals      uint8 [ceil(nnz/2)]         (canonical int4, low nibble first)
 *  out_cols and out_vals start 16-byte aligned and stay readable up to the next
 *  16-byte boundary past their end (at least 16 bytes, even when nnz == 0): the
 *  kernels fetch them in whole 16-byte chunks.
 */
typedef struct gale_matrix {
    const uint32_t* signs;
    const uint16_t* block_scales;
    const uint16_t* row_scales;
    const int32_t*  row_ptr;
    const uint16_t* out_cols;
    const uint8_t*  out_vals;
} gale_matrix;

/* One routed expert: w1 (gate) and w3 (up) are [inter, hidden], w2 (down) is [hidden, inter]. */
typedef struct gale_expert {
    gale_matrix w1, w3, w2;
} gale_expert;

/* The inputs and outputs of one routed-expert layer for one token (gale_moe_decode_stack).
 * All pointers are device pointers. */
typedef struct gale_layer_io {
    const gale_expert* experts;  /* descriptor table of the layer's n_experts experts */
    const float* logits;         /* fp32 [n_experts] router logits */
    const float* select_bias;    /* fp32 [n_experts] selection bias, or NULL (as gale_moe_layer_fwd_routed) */
    const int32_t* fixed_idx;    /* int32 [top_k] given experts, or NULL (as gale_moe_layer_fwd_routed) */
    const void* x;               /* fp16 [hidden]; may be the previous layer's y */
    void* y;                     /* fp16 [hidden] */
    int32_t* topk_idx;           /* int32 [top_k], or NULL */
    float* topk_w;               /* fp32 [top_k], or NULL */
} gale_layer_io;

/* Bytes of each packed section of one matrix. */
typedef struct gale_sizes {
    size_t signs, block_scales, row_scales, row_ptr, out_cols, out_vals;
    size_t format_bytes;  /* signs + block scales + row scales + out_cols + out_vals (row_ptr excluded) */
} gale_sizes;

/* ---- errors ---------------------------------------------------------------- */
const char* gale_status_str(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* gale_last_error(void);

/* ---- format helpers (host only, no GPU needed) ----------------------------- */

/* Section sizes of a [rows, cols] matrix with nnz outliers.  out: host. */
int gale_packed_sizes(int32_t rows, int32_t cols, int64_t nnz, gale_sizes* out);

/* Validate canonical CSR outliers (host pointers): row_ptr monotone from 0 to nnz,
 * columns < cols and strictly ascending within each row.  GALE_ERR_FORMAT on violation. */
int gale_check_canonical(int32_t rows, int32_t cols, const int32_t* row_ptr,
                         const uint16_t* out_cols, int64_t nnz);

/* Canonical -> device layout for the sections that change (signs, block scales), on the
 * host.  canon_signs: uint32 [rows][cols/32], b[n][k] = bit (k % 32) of word k / 32;
 * canon_scales: fp16 [rows][cols/128].  All pointers host; outputs sized by
 * gale_packed_sizes.  Outliers and row scales are stored canonically (copy as is). */
int gale_pack_host(int32_t rows, int32_t cols, const uint32_t* canon_signs,
                   const uint16_t* canon_scales, uint32_t* dev_signs, uint16_t* dev_scales);

/* Inverse of gale_pack_host (host pointers). */
int gale_unpack_host(int32_t rows, int32_t cols, const uint32_t* dev_signs,
                     const uint16_t* dev_scales, uint32_t* canon_signs, uint16_t* canon_scales);

/* ---- packing and bit-exact checks on the GPU -------------------------------- */

/* gale_pack_host for n_mat matrices stored back to back, on the device. */
int gale_pack_device(int32_t rows, int32_t cols, int32_t n_mat, const uint32_t* canon_signs,
                     const uint16_t* canon_scales, uint32_t* dev_signs, uint16_t* dev_scales,
                     hipStream_t stream);

/* Device layout -> canonical sign words, decoding every bit with the same plane masks the
 * GEMV kernel applies.  dev_signs: one packed matrix; canon_signs: uint32 [rows][cols/32]. */
int gale_debug_unpack_signs(int32_t rows, int32_t cols, const uint32_t* dev_signs,
                            uint32_t* canon_signs, hipStream_t stream);

/* Decode the outliers of one matrix as the GEMV kernel does: for each CSR entry p, write its
 * row (int32), column (int32) and int4 value (int32, -8..7).  Any pointer may be NULL. */
int gale_debug_unpack_outliers(int32_t rows, int64_t nnz, const gale_matrix* m_host,
                               int32_t* out_row, int32_t* out_col, int32_t* out_val,
                               hipStream_t stream);

/* ---- compute -------------------------------------------------------------- */

/* Blocked Walsh-Hadamard transform (DeepSeek-V4-Pro GALE page, serving knobs: a single-kernel
 * butterfly, exact to 1e-8 of the matrix form): for every vector v and block beta,
 *   y[v][1024 beta + i] = sum_j H[i][j] x[v][1024 beta + j].
 * x, y: [n_vec][len], len % 1024 == 0, dtypes GALE_F16 / GALE_F32; fp32 arithmetic.
 * In place (x == y) is allowed when the dtypes match. */
int gale_fwht1024(const void* x, void* y, int64_t n_vec, int32_t len, int32_t in_dtype,
                  int32_t out_dtype, hipStream_t stream);

/* Bytes of one prepared activation record of length len (a multiple of 256). */
size_t gale_prepared_bytes(int32_t len);

/* Prepare activation vectors for the GEMV: x~ = blockdiag(H) x (skipped with GALE_X_ROTATED),
 * stored as fp32 plus the matrix-core operand form (four fp8 e4m3 terms per element with a
 * power-of-two scale per 1024-block).  x: [n_vec][len] (x_dtype); out: n_vec records of
 * gale_prepared_bytes(len) bytes, 256-byte aligned.  A record can feed any number of GEMVs
 * (the routed layer shares one per token across its experts' gate and up matrices). */
int gale_prepare_activations(const void* x, int32_t x_dtype, int64_t n_vec, int32_t len, uint32_t flags,
                             void* out, size_t out_bytes, hipStream_t stream);

/* Workspace bytes for gale_expert_gemv. */
size_t gale_gemv_workspace_bytes(int32_t rows, int32_t cols, int32_t n_mat, int32_t n_tok,
                                 int32_t x_shared);

/* Batched direct GEMV (DeepSeek-V4-Pro GALE page, serving knobs: a GEMV that multiplies
 * straight out of a packed record, with a batched mode over many matrices):
 *   y[m][t][:] = Wq_m . (H . x[m][t][:])   for m < n_mat, t < n_tok.
 * mats_dev: device array of n_mat gale_matrix descriptors, all [rows, cols].
 * x: [n_mat][n_tok][cols] (or [n_tok][cols] shared by all matrices when x_shared != 0),
 *    dtype x_dtype (GALE_F16 / GALE_F32); flags GALE_X_ROTATED means x is already H.x.
 * y: [n_mat][n_tok][rows], dtype y_dtype.  ws: gale_gemv_workspace_bytes(...) bytes,
 * 256-byte aligned.  With GALE_X_PREPARED, x holds the prepared records (same indexing,
 * x_dtype ignored) and ws may be NULL.  fp32 accumulation.
 * With n_tok == 1 and cols <= 8192 the rotation, the activation split and the GEMV run in one
 * kernel launch (ws is then left untouched, but its size is still checked); otherwise the
 * records are prepared in ws first.  Both give the same bits. */
int gale_expert_gemv(int32_t rows, int32_t cols, const gale_matrix* mats_dev, int32_t n_mat,
                     const void* x, int32_t x_dtype, int32_t x_shared, int32_t n_tok,
                     void* y, int32_t y_dtype, void* ws, size_t ws_bytes, uint32_t flags,
                     hipStream_t stream);

/* Workspace bytes for gale_expert_ffn. */
size_t gale_ffn_workspace_bytes(int32_t hidden, int32_t inter, int32_t n_exp, int32_t n_tok,
                                int32_t x_shared);

/* Expert FFN for n_exp experts (model card naming: w1 gate, w3 up, w2 down):
 *   y[e][t] = w2_e . H( silu(w1_e . H x) * (w3_e . H x) ),  x = x[e][t] (or x[t] if x_shared).
 * experts_dev: device array of n_exp gale_expert.  x, y fp16 [.. ][n_tok][hidden];
 * intermediate h and every sum in fp32.  hidden <= GALE_MAX_HIDDEN (else GALE_ERR_SHAPE). */
int gale_expert_ffn(int32_t hidden, int32_t inter, const gale_expert* experts_dev, int32_t n_exp,
                    const void* x, int32_t x_shared, int32_t n_tok, void* y,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for gale_moe_layer_fwd. */
size_t gale_moe_workspace_bytes(int32_t n_tok, int32_t n_experts, int32_t top_k,
                                int32_t hidden, int32_t inter, uint32_t flags);

/* One routed-expert layer:
 *   route: S_t = the top_k experts by (logit desc, expert index asc) of logits[t] (fp32
 *          [n_tok][n_experts]); w[t] = softmax of those k logits (fp32).
 *   y[t] = sum over slots j = 0..top_k-1, in order, of w[t][j] * FFN_{S_t[j]}(x[t]).
 * x, y: fp16 [n_tok][hidden].  topk_idx (int32 [n_tok][top_k]) and topk_w (fp32) are
 * written when non-NULL.  Two paths, same results bit for bit on any token:
 *   decode  (n_tok <= 64): one workgroup routes all tokens and lists the work items;
 *           with one token the whole layer is a single persistent launch (the
 *           DeepSeek-V4-Pro GALE page's batch-1 notes put the floor in launches), the
 *           layer of gale_moe_decode_stack: every workgroup routes the token itself,
 *           runs its gate/up units, and then owns 16 rows of y for all top_k experts,
 *           waiting only for the rotated 1024-blocks of h it reads.  This needs the workspace's synchronisation words (its first
 *           GALE_SYNC_BYTES bytes) zero-filled once before the first such call
 *           (gale_sync_init, or any zero fill) and calls sharing a workspace must not
 *           overlap in time (true of every workspace).  When the words are not valid
 *           the call computes nothing (y is left as it was); gale_sync_status() reports
 *           it.  GALE_DECODE_STAGED selects the five-launch sequence instead (same
 *           results bit for bit; it does not use the synchronisation words);
 *   grouped (n_tok > 64):  chunked top-k and a stable sort of the (token, slot) pairs
 *           by expert; then experts with many pairs run a tiled GEMM on the matrix
 *           cores (128 pairs x 128 weight rows per workgroup, the weights dequantized to
 *           fp16 in LDS -- sign times block scale, plus the outliers -- and the rotated
 *           activations in fp16: each rounding ~2^-12 relative, results within the
 *           rel-L2 bar, not bit-equal to the decode path), and the others run work
 *           items of up to 4 pairs of one expert through the decode GEMV (bit-equal to
 *           the decode path).  GALE_GROUPED_ITEMS / GALE_GROUPED_GEMM force one kind
 *           for every expert.
 * Flags GALE_PATH_DECODE / GALE_PATH_GROUPED force a path (decode takes at most 64
 * tokens).  The workspace depends on the path (gale_moe_workspace_bytes with the same
 * flags).  hidden <= GALE_MAX_HIDDEN (else GALE_ERR_SHAPE); the single-launch layer
 * takes hidden <= 4096 (whole 1024-column blocks; the down tasks of top_k x inter / 1024
 * must fit its wavefronts, true of every shape with inter <= 2 hidden), other shapes run
 * the five-launch sequence. */
int gale_moe_layer_fwd(int32_t hidden, int32_t inter, const gale_expert* experts_dev,
                       int32_t n_experts, const float* logits, int32_t top_k, const void* x,
                       int32_t n_tok, void* y, int32_t* topk_idx, float* topk_w,
                       void* ws, size_t ws_bytes, uint32_t flags, hipStream_t stream);

/* The same layer with two of DeepSeek's routing variants:
 *   select_bias (fp32 [n_experts], or NULL): a per-expert term added to the logits for the
 *          choice of the top_k experts only; the weights stay the softmax of the chosen
 *          experts' own logits (the aux-loss-free balancing bias, DeepSeek-V4-Pro GALE page,
 *          serving notes on the tier bias).  The choice compares fp32 sums logit + bias,
 *          ties to the lower expert index.
 *   fixed_idx (int32 [n_tok][top_k], or NULL): the experts of each token are given, in slot
 *          order (hash-routed layers that read a token-to-expert table, DeepSeek-V4-Flash
 *          180B REAP card); the weights are again the softmax of those experts' logits.
 *          Entries must be distinct experts in [0, n_experts); an entry outside that range
 *          is clamped into it (memory-safe, result unspecified).
 * At most one of the two may be given (GALE_ERR_SHAPE otherwise); with neither, the call is
 * gale_moe_layer_fwd.  Both pointers are device memory, 4-byte aligned.  Same workspace,
 * paths and flags as gale_moe_layer_fwd. */
int gale_moe_layer_fwd_routed(int32_t hidden, int32_t inter, const gale_expert* experts_dev,
                              int32_t n_experts, const float* logits, const float* select_bias,
                              const int32_t* fixed_idx, int32_t top_k, const void* x, int32_t n_tok,
                              void* y, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                              uint32_t flags, hipStream_t stream);

/* ---- one token through a stack of layers in one launch -------------------------- */

/* Bytes at the start of a one-launch decode workspace that hold its synchronisation words. */
#define GALE_SYNC_BYTES 40960

/* Workspace bytes for gale_moe_decode_stack (the synchronisation words, then fp32 h and the
 * rotated h's activation records). */
size_t gale_decode_stack_workspace_bytes(int32_t hidden, int32_t inter, int32_t top_k);

/* One decode token through n_layers routed-expert layers, in one persistent launch
 * (DeepSeek-V4-Flash GALE model card, "Measured performance": 43 layers x 6 routed experts
 * per token; the DeepSeek-V4-Pro GALE page's batch-1 notes put the floor in launches).
 * Layer l computes exactly gale_moe_layer_fwd of one token on layers_dev[l] (same results
 * bit for bit), and reads its x only after every row of layer l-1's y has been stored, as
 * separate launches in stream order would: x of layer l may be y of layer l-1.  Logits,
 * selection biases and fixed experts are inputs of the call: layer l's logits may be read
 * while layer l-1 runs, so they must not alias any layer's y.
 * layers_dev: device array of n_layers gale_layer_io (read by the kernel); at most one of
 * select_bias / fixed_idx per layer.  hidden and inter as the one-launch layer takes them
 * (gale_moe_layer_fwd); n_experts <= GALE_MAX_EXPERTS, top_k <= GALE_MAX_TOPK.
 * ws: gale_decode_stack_workspace_bytes() bytes, 256-byte aligned, whose first
 * GALE_SYNC_BYTES must have been zero-filled once (gale_sync_init) before the first call
 * on it; if they are not valid, or a wait in an earlier call gave up, the call computes
 * nothing and gale_sync_status() says why.  Every workgroup of the launch must be resident
 * at once (one per CU): a wait gives up after about 10 ms, records that in the words and
 * the kernel carries on, so it always ends.  flags: GALE_TILES_SHIFT, GALE_SYNC_NO_WAIT. */
int gale_moe_decode_stack(int32_t hidden, int32_t inter, int32_t n_experts, int32_t top_k, int32_t n_layers,
                          const gale_layer_io* layers_dev, void* ws, size_t ws_bytes, uint32_t flags,
                          hipStream_t stream);

/* For callers that cannot allocate -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc: gale_moe_decode_stack with its workspace in a device array
 * of GALE_STATIC_SCRATCH_BYTES that the library holds for each GPU it runs on, from its first
 * call on that GPU until the process ends.  The call allocates nothing and frees nothing.
 * Every call zeroes the array's synchronisation words before its kernel (a fill kernel on
 * `stream`), so each call starts clean and a wait that gave up in an earlier call does not
 * carry over (nor can it be queried: use gale_moe_decode_stack with gale_sync_status for
 * that).  Calls on one GPU share its array: calls that overlap in time on one GPU (two streams,
 * two threads) race and must not be made.  The arguments are those of gale_moe_decode_stack;
 * a shape whose workspace (gale_decode_stack_workspace_bytes) exceeds
 * GALE_STATIC_SCRATCH_BYTES returns GALE_ERR_WORKSPACE before anything is enqueued. */
#define GALE_STATIC_SCRATCH_BYTES (GALE_SYNC_BYTES + 196608)
int gale_moe_decode_stack_static(int32_t hidden, int32_t inter, int32_t n_experts, int32_t top_k,
                                 int32_t n_layers, const gale_layer_io* layers_dev, uint32_t flags,
                                 hipStream_t stream);

/* Zero the synchronisation words at the start of ws (GALE_SYNC_BYTES; a kernel on `stream`,
 * so it can be captured in a graph).  Needed once before the first one-launch decode call on
 * a workspace, and again after gale_sync_status() reported GALE_ERR_SYNC. */
int gale_sync_init(void* ws, hipStream_t stream);

/* State of the synchronisation words at the start of ws, for the caller to check after its
 * own synchronisation: copies the three header words to the host (a blocking copy, not for
 * graph capture).  GALE_OK: valid and no wait has given up.  GALE_ERR_SYNC: the words were
 * never zeroed, or a wait of an earlier call gave up (gale_last_error() says which); the
 * outputs of that call are unspecified and later calls compute nothing until gale_sync_init.
 * words_host (3 x uint64, may be NULL): generation, check word, error bits. */
int gale_sync_status(const void* ws, uint64_t* words_host);

/* Workspace bytes for gale_route_topk with grouping of more than GALE_MAX_DECODE_TOKENS tokens. */
size_t gale_route_workspace_bytes(int32_t n_tok, int32_t n_experts);

/* Routing alone (same rule as gale_moe_layer_fwd), plus the stable grouping of the
 * (token, slot) pairs p = t * top_k + j by expert: offsets int32 [n_experts + 1] and
 * perm int32 [n_tok * top_k] (pairs of expert e in ascending order at
 * perm[offsets[e] .. offsets[e+1])).  offsets and perm are both NULL (top-k only) or
 * both set; grouping more than GALE_MAX_DECODE_TOKENS tokens needs ws of
 * gale_route_workspace_bytes() bytes (otherwise ws may be NULL). */
int gale_route_topk(const float* logits, int32_t n_tok, int32_t n_experts, int32_t top_k,
                    int32_t* topk_idx, float* topk_w, int32_t* offsets, int32_t* perm,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Diagnostic, not a step of the method: reads `bytes` bytes at device pointer src (16-byte
 * aligned, a positive multiple of 16) once with a plain streaming kernel, 16 bytes per lane per
 * step, on `stream`, and writes one folded word per workgroup to the device array sink
 * (4-byte aligned, sink_words >= 1 words; the grid is at most sink_words workgroups).  Timed
 * by the caller, it gives the HBM read rate a trivial kernel reaches on this device, the
 * practical ceiling next to the 8 TB/s peak.  Errors: GALE_ERR_NULL, GALE_ERR_SHAPE,
 * GALE_ERR_ALIGN, GALE_ERR_HIP (a launch failure). */
int gale_read_stream(const void* src, size_t bytes, uint32_t* sink, int32_t sink_words, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GALE_H */
