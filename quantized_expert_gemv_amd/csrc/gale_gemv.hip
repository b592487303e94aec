// Direct GEMV out of the packed GALE record on the MI355X matrix cores.
//
// What it computes (DeepSeek-V4-Flash GALE 1-bit model card, "What is in the
// pack"): y[n] = sum_k Wq[n][k] x~[k], x~ = blockdiag(H_1024) x, with
//   Wq[n][k] = s[n][k/128] (1 - 2 b[n][k]) + r[n] q at the row's int4 outliers.
// The DeepSeek-V4-Pro GALE page (serving options, the direct GEMV) multiplies
// straight out of the packed record with signs, block scales and outliers decoded
// in registers; this kernel keeps that idea and re-plans it for gfx950.
//
// gfx950 plan.  A 1-bit GEMV has ~1 VALU op per weight of budget at HBM speed,
// too little for a per-bit select-and-add.  Instead each sign bit becomes one
// 4-bit element of an fp4 (e2m1) MFMA operand with a single AND:
//   * the device layout puts eight columns of scale block d at bit position
//     d % 4 of the eight nibbles of a word, so (w & 0x11111111 << d % 4) is an
//     fp4 operand dword whose elements are b * 2^(d % 4 - 1) (b = sign bit), and
//     the MFMA's E8M0 B-scale 2^(2 - d % 4) makes them exactly 2 b; blocks 3 and
//     7 use the sign form (w & 0x88888888) | 0x22222222 = (1 - 2 b) * 1.0;
//   * the activation enters as A = four fp8 e4m3 terms of X = x~ 2^p (rows of
//     A), up to four tokens sharing the weights (so M = 4 terms x 4 tokens);
//   * the block sums S = sum_k X (one MFMA against an all -1.0 operand when the
//     activation changes) turn the 0/1 planes into signs: block d adds
//     s[n][d] (S - 2 sum_k b X).
// One v_mfma_scale_f32_16x16x128_f8f6f4 therefore consumes one scale block of
// 16 rows: 2048 weights for 4 ANDs (8 in sign form) and two FMAs per token.
//
// Work split.  A unit is R row tiles (16 rows each) of one work item (a matrix,
// or the w1/w3 pair of an expert, with up to four activation vectors).  A
// workgroup has one wavefront per 1024-column chunk of each matrix (split-K);
// the partial sums meet in LDS, in a fixed order.  Workgroups are persistent:
// each streams a contiguous run of units, tracking its position incrementally
// and reloading a work item's descriptors only when the item changes.
//
// Memory pipeline.  Vector-memory completions are counted in issue order, so a
// wait for any load also waits for every older one.  Each unit therefore
// consumes only data issued one unit earlier: at the top of unit u the
// workgroup issues the whole of unit u+1 (sign words, block scales, the outlier
// entries of its rows as 16-byte chunks, row scales) and the CSR offsets of
// unit u+2, then computes unit u from registers and LDS.  Descriptors are read
// with scalar loads; nothing is loaded conditionally (addresses are clamped);
// every global load is a uniform base plus a 32-bit lane offset.
//
// Outliers: each wavefront serves 16 rows of the unit.  Their CSR entries are a
// contiguous range, fetched as coalesced 16-byte chunks and staged in the
// wavefront's own LDS slice; four lanes per row then walk the row in CSR order
// and gather x~ from an LDS copy of the activation.
#include "gale_internal.h"
#include "gale_decode.h"
#include "gale_gemv_core.h"
#include "gale_rotate.h"

namespace gale {

// Item of a unit, decoded without dynamically indexed arrays.
struct Item {
  int mat, nslots;
  int ra0, ra1, ra2, ra3;
  int out0, out1, out2, out3;
};

template <int NS>
__device__ __forceinline__ Item decode_item(const GemvParams& P, int item) {
  Item it;
  if (P.implicit_items) {
    const int mat = item / P.n_groups;
    const int grp = item - mat * P.n_groups;
    it.mat = mat;
    const int ns = P.n_tok - grp * NS;
    it.nslots = ns < NS ? ns : NS;
    const int base_ra = (P.x_shared ? 0 : mat * P.n_tok) + grp * NS;
    const int base_out = mat * P.n_tok + grp * NS;
    it.ra0 = base_ra;
    it.ra1 = base_ra + (1 < it.nslots ? 1 : 0);
    it.ra2 = base_ra + (2 < it.nslots ? 2 : 0);
    it.ra3 = base_ra + (3 < it.nslots ? 3 : 0);
    it.out0 = base_out;
    it.out1 = base_out + (1 < it.nslots ? 1 : 0);
    it.out2 = base_out + (2 < it.nslots ? 2 : 0);
    it.out3 = base_out + (3 < it.nslots ? 3 : 0);
  } else {
    const auto* w = as_const(P.items) + item;
    it.mat = uni(w->expert);
    const int ns = uni(w->n_slots);
    it.nslots = ns < NS ? ns : NS;
    const int p0 = uni(w->pair[0]), p1 = uni(w->pair[1]), p2 = uni(w->pair[2]), p3 = uni(w->pair[3]);
    it.out0 = p0;
    it.out1 = 1 < it.nslots ? p1 : p0;
    it.out2 = 2 < it.nslots ? p2 : p0;
    it.out3 = 3 < it.nslots ? p3 : p0;
    it.ra0 = it.out0 / P.ra_div;
    it.ra1 = it.out1 / P.ra_div;
    it.ra2 = it.out2 / P.ra_div;
    it.ra3 = it.out3 / P.ra_div;
  }
  return it;
}

// Descriptor-table index of an item's matrix group.
__device__ __forceinline__ int item_mat(const GemvParams& P, int item) {
  if (P.implicit_items) return uni(item / P.n_groups);
  return uni(as_const(P.items)[item].expert);
}

struct Geo {
  int K, C, tid, lane, wave, half, c, g, nl, ntiles, RG;
  int ohalf, orow0, wr, sub;   // outlier role: rows orow0 + wr of half ohalf, lane sub of four
  bool orole;
  uint32_t sw_lane, sc_lane;   // lane's byte offsets inside one row tile's sign words / scales
  uint32_t sw_tile, sc_tile;   // bytes per row tile (all chunks)
};

// The sections of one work item that this wavefront reads: the matrix of its half
// (signs, block scales) and the matrix whose outliers it serves.
struct Desc {
  const char* signs;
  const char* scales;
  const char* rsc;
  const int32_t* rptr;
  const char* ocols;
  const char* ovals;
};

__device__ __forceinline__ Desc load_desc(const GemvParams& P, const Geo& G, int mat) {
  const auto* t = as_const(P.table);
  const int iw = uni(mat * P.mat_stride + (G.half ? P.sel1 : P.sel0));
  const int io = uni(mat * P.mat_stride + (G.ohalf ? P.sel1 : P.sel0));
  Desc d;
  d.signs = reinterpret_cast<const char*>(t[iw].signs);
  d.scales = reinterpret_cast<const char*>(t[iw].block_scales);
  d.rsc = reinterpret_cast<const char*>(t[io].row_scales);
  d.rptr = t[io].row_ptr;
  d.ocols = reinterpret_cast<const char*>(t[io].out_cols);
  d.ovals = reinterpret_cast<const char*>(t[io].out_vals);
  return d;
}

// Position of a unit: index, work item, row group.
struct Pos {
  int u, item, rg;
};

// The unit after p, or p itself at the end of the workgroup's range.
__device__ __forceinline__ Pos pos_next(const Pos& p, int u1, int RG) {
  if (p.u + 1 >= u1) return p;
  Pos q;
  q.u = p.u + 1;
  q.rg = p.rg + 1;
  q.item = p.item;
  if (q.rg == RG) {
    q.rg = 0;
    q.item = p.item + 1;
  }
  return q;
}

// Row served by this thread's outlier role in row group rg, clamped to [0, rows].
template <int R>
__device__ __forceinline__ int outlier_row(const GemvParams& P, const Geo& G, int rg, bool* valid) {
  const int n = rg * R * 16 + G.orow0 + G.wr;
  *valid = G.orole && n < P.rows;
  return n < P.rows ? n : P.rows;
}

// Issue the loads of unit v (descriptors dv) into b.  rp0/rp1 of v must already be in
// b (from the previous unit's np0/np1).  Also fetches the CSR offsets of unit vn.
template <int R, int OC>
__device__ __forceinline__ void issue_unit(const GemvParams& P, const Geo& G, const Pos& v, const Desc& dv,
                                           const Pos& vn, const Desc& dn, UnitBuf<R, OC>& b) {
  const int t0 = v.rg * R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int tile = t0 + r;
    tile = tile < G.ntiles ? tile : G.ntiles - 1;
    const uint32_t o = (uint32_t)tile * G.sw_tile + G.sw_lane;
    const uint4 lo = ld16_stream(dv.signs, o);
    const uint4 hi = ld16_stream(dv.signs, o + 1024u);
    b.sw[r][0] = lo.x; b.sw[r][1] = lo.y; b.sw[r][2] = lo.z; b.sw[r][3] = lo.w;
    b.sw[r][4] = hi.x; b.sw[r][5] = hi.y; b.sw[r][6] = hi.z; b.sw[r][7] = hi.w;
    const uint4 sc = ld16_stream(dv.scales, (uint32_t)tile * G.sc_tile + G.sc_lane);
    b.sc[r][0] = sc.x; b.sc[r][1] = sc.y; b.sc[r][2] = sc.z; b.sc[r][3] = sc.w;
  }
  // outlier entries of the wave's 16 rows: CSR range [e0, e1) from lanes 0 (first row) and 60 (last row)
  const int e0 = uni(__builtin_amdgcn_readlane(b.rp0, 0));
  const int e1 = uni(__builtin_amdgcn_readlane(b.rp1, 60));
  // 16-byte chunks holding the uint16 columns and the packed int4 values of [e0, e1); an
  // empty range reads chunk 0 (the sections are padded to, and readable in, whole 16-byte chunks)
  const bool any = e1 > e0;
  const int cf = any ? (2 * e0) >> 4 : 0;
  const int cl = any ? (2 * e1 - 1) >> 4 : 0;
  const int vf = any ? (e0 >> 1) >> 4 : 0;
  const int vl = any ? ((e1 - 1) >> 1) >> 4 : 0;
  b.ocf = cf;
  b.ovf = vf;
#pragma unroll
  for (int k = 0; k < OC; ++k) {
    int ch = cf + 64 * k + G.lane;
    ch = ch < cl ? ch : cl;
    b.oc[k] = ld16_stream(dv.ocols, (uint32_t)ch * 16u);
  }
#pragma unroll
  for (int k = 0; k < val_chunks(OC); ++k) {
    int ch = vf + 64 * k + G.lane;
    ch = ch < vl ? ch : vl;
    b.ov[k] = ld16_stream(dv.ovals, (uint32_t)ch * 16u);
  }
  bool ok;
  const int n = outlier_row<R>(P, G, v.rg, &ok);
  b.rsc = *reinterpret_cast<const uint16_t*>(dv.rsc + 2u * (uint32_t)(n < P.rows ? n : P.rows - 1));
  // CSR offsets of the next unit's row
  const int n2 = outlier_row<R>(P, G, vn.rg, &ok);
  b.np0 = dn.rptr[n2];
  b.np1 = dn.rptr[n2 + (n2 < P.rows ? 1 : 0)];
}

template <int NS>
__device__ __forceinline__ void load_activation(const GemvParams& P, const Geo& G, const Item& it, Act& a) {
  const int term = G.nl >> 2, slot = G.nl & 3;
  const int ra = sel4(slot < it.nslots ? slot : 0, it.ra0, it.ra1, it.ra2, it.ra3);
  const uint8_t* tb = P.ra + (size_t)ra * P.ra_stride + ra_terms_off(G.K) + ((size_t)G.c * 4 + term) * 1024 + 32 * G.g;
  // lanes of empty slots load nothing (their rows of A are zero)
  const bool live = slot < it.nslots;
#pragma unroll
  for (int d = 0; d < 8; ++d) a.A[d] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(tb + 128 * d);
      const uint4 a1 = *reinterpret_cast<const uint4*>(tb + 128 * d + 16);
      a.A[d] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int rai = sel4(i < it.nslots ? i : 0, it.ra0, it.ra1, it.ra2, it.ra3);
    const int pv = reinterpret_cast<const int32_t*>(P.ra + (size_t)rai * P.ra_stride + ra_p_off(G.K))[G.c];
    a.pexp[i] = i < it.nslots ? pv : 0;
  }
}

// fp32 x~ of the item's vectors into LDS for the outlier gather (when it fits); with several
// vectors, interleaved by column (xt[NS col + i]) so one gather reads every vector's value
template <int NS>
__device__ __forceinline__ void stage_activation(const GemvParams& P, const Geo& G, const Item& it, lds_f32* xt) {
  if (!P.stage_xt) return;
  for (int i = 0; i < NS; ++i) {
    if (i >= it.nslots) break;
    const int ra = sel4(i, it.ra0, it.ra1, it.ra2, it.ra3);
    const u32x4* src = reinterpret_cast<const u32x4*>(P.ra + (size_t)ra * P.ra_stride);
    if constexpr (NS == 1) {
      lds_v4* dst = reinterpret_cast<lds_v4*>(xt);
      for (int q = G.tid; q < (G.K >> 2); q += (int)blockDim.x) dst[q] = src[q];
    } else {
      for (int q = G.tid; q < (G.K >> 2); q += (int)blockDim.x) {
        const u32x4 v = src[q];
        xt[NS * (4 * q + 0) + i] = __uint_as_float(v.x);
        xt[NS * (4 * q + 1) + i] = __uint_as_float(v.y);
        xt[NS * (4 * q + 2) + i] = __uint_as_float(v.z);
        xt[NS * (4 * q + 3) + i] = __uint_as_float(v.w);
      }
    }
  }
}

// Every vector's x~ at column col from the staged copy (one LDS read)
template <int NS>
__device__ __forceinline__ void xs_at(const lds_f32* xt, int col, float* x) {
  if constexpr (NS == 1) {
    x[0] = xt[col];
  } else if constexpr (NS == 2) {
    typedef float v2f_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) const v2f_t lds_v2f;
    const v2f_t v = *reinterpret_cast<lds_v2f*>(xt + 2 * col);
    x[0] = v[0]; x[1] = v[1];
  } else {
    typedef __attribute__((address_space(3))) const v4f lds_v4f;
    const v4f v = *reinterpret_cast<lds_v4f*>(xt + 4 * col);
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  }
}

// Raw activations (FX): wavefront c rotates and splits chunk c of an item's x into the
// workgroup's LDS record with the same code and layout as a prepared record, so every
// product equals the one from a record prepared by prep_kernel.  The first item's x comes
// with plain loads; every later item's x is copied global-to-LDS one unit ahead, with the
// loads of the unit that starts it, so it costs no registers while in flight.
__device__ __forceinline__ const char* x_chunk(const GemvParams& P, const Geo& G, int v) {
  const int64_t isz = P.x_dtype == GALE_F16 ? 2 : 4;
  return reinterpret_cast<const char*>(P.x) + ((int64_t)v * P.x_stride + (int64_t)G.c * 1024) * isz;
}

__device__ __forceinline__ void issue_x_copy(const GemvParams& P, const Geo& G, int v, lds_u8* xstage) {
  const int isz = P.x_dtype == GALE_F16 ? 2 : 4;
  const char* src = x_chunk(P, G, v) + 16 * G.lane;
  lds_u8* dst = xstage + G.c * 1024 * isz;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < isz) __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) uint8_t*)(src + 1024 * j),
                                                  dst + 1024 * j, 16, 0, 0);
}

// Chunk c of the record of x (16 values of this lane, in the coalesced layout of x's dtype).
__device__ __forceinline__ void prep_x_record(const GemvParams& P, const Geo& G, const float f[16], uint8_t* lrec) {
  PrepLane o;
  prep_lane(f, G.lane, !P.x_rotated, o);
  store_record_chunk(o, P.x_dtype, lrec, G.K, G.c, G.lane);
}

template <int NS, int R, bool GATEUP, int OC, bool FX>
__device__ __forceinline__ void process_unit(const GemvParams& P, const Geo& G, const Pos& cur_pos, Item& it,
                                             UnitBuf<R, OC>& cur, UnitBuf<R, OC>& nxt, const Pos& p1, const Desc& d1,
                                             const Pos& p2, const Desc& d2, int& act_item, Act& act,
                                             lds_f32* red, lds_f32* ored, lds_f32* xt, lds_u8* wout,
                                             uint8_t* lrec, uint8_t* xstage) {
  constexpr int HALVES = GATEUP ? 2 : 1;
  constexpr int RR = R * 16;
  const int item = cur_pos.item;
  const int rg = cur_pos.rg;

  // 1. activation of a new item (A operands, block sums, x~ in LDS); issued before the
  //    next unit's loads so that waiting for it never waits for them
  if (item != act_item) {
    it = decode_item<NS>(P, item);
    if constexpr (FX) {
      // the w1 (or only) wavefront of chunk c builds the chunk's record; its copy of the
      // item's x chunk (issued a unit ago) has landed
      if (G.half == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        float f[16];
        load_block_coalesced(xstage + G.c * 1024 * (P.x_dtype == GALE_F16 ? 2 : 4), P.x_dtype, G.lane, f);
        prep_x_record(P, G, f, lrec);
      }
      __syncthreads();
      record_activation(lrec, G.K, G.c, G.lane, act);
    } else {
      load_activation<NS>(P, G, it, act);
      stage_activation<NS>(P, G, it, xt);
      __syncthreads();
    }
    block_sums<NS>(act);
    act_item = item;
  }

  // 2. stage this unit's outlier chunks in the wave's LDS slice
  {
    lds_v4* oc = reinterpret_cast<lds_v4*>(wout);
#pragma unroll
    for (int k = 0; k < OC; ++k) oc[64 * k + G.lane] = to_v4(cur.oc[k]);
#pragma unroll
    for (int k = 0; k < val_chunks(OC); ++k) oc[64 * (OC + k) + G.lane] = to_v4(cur.ov[k]);
  }

  // 3. issue unit u+1 (and the CSR offsets of u+2) behind this unit's arithmetic
  nxt.rp0 = cur.np0;
  nxt.rp1 = cur.np1;
  issue_unit<R, OC>(P, G, p1, d1, p2, d2, nxt);
  if constexpr (FX) {
    // the next unit starts another item (at the end of the range p1 is this unit): its x
    if (p1.item != item && G.half == 0) issue_x_copy(P, G, decode_item<NS>(P, p1.item).ra0, (lds_u8*)xstage);
  }

  // 4. sign pass over the wave's R tiles
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc[NS];
    sign_tile<NS>(act, cur.sw[r], cur.sc[r], acc);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float v = term_sum(ldexpf(acc[i], -act.pexp[i]));   // undo 2^p, sum the four terms
      if (G.lane < 16) red[((G.half * G.C + G.c) * RR + r * 16 + G.lane) * NS + i] = v;
    }
  }

  // 5. outliers: four lanes per row in CSR order, entries and x~ from LDS
  {
    bool valid;
    (void)outlier_row<R>(P, G, rg, &valid);
    const lds_u16* lc = reinterpret_cast<const lds_u16*>(wout);
    const lds_u8* lv = wout + 64 * 16 * OC;
    float o[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) o[i] = 0.f;
    const int cbase = 8 * cur.ocf, vbase = 16 * cur.ovf;
    const int p_begin = cur.rp0 + G.sub, p_end = valid ? cur.rp1 : p_begin;
    // entries p < p_cap are in the staged chunks
    const int p_cap = min(cbase + 64 * 8 * OC, 2 * (vbase + 64 * 16 * val_chunks(OC)));
    const int p_mid = min(p_end, p_cap);
    int p = p_begin;
    if (P.stage_xt) {
      // eight entries per step: all their LDS reads issue before the first FMA waits
      for (; p + 28 < p_mid; p += 32) {
        int col[8], by[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) { col[j] = lc[p + 4 * j - cbase]; by[j] = lv[((p + 4 * j) >> 1) - vbase]; }
        // every vector's values (slots past the item's vectors compute into sums never stored)
        float x[8][NS];
#pragma unroll
        for (int j = 0; j < 8; ++j) xs_at<NS>(xt, col[j], x[j]);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
#pragma unroll
          for (int j = 0; j < 8; ++j) o[i] = fmaf(nibble_value(by[j], p), x[j][i], o[i]);
        }
      }
      for (; p + 12 < p_mid; p += 16) {
        const int col0 = lc[p - cbase], col1 = lc[p + 4 - cbase], col2 = lc[p + 8 - cbase], col3 = lc[p + 12 - cbase];
        const int by0 = lv[(p >> 1) - vbase], by1 = lv[((p + 4) >> 1) - vbase];
        const int by2 = lv[((p + 8) >> 1) - vbase], by3 = lv[((p + 12) >> 1) - vbase];
        float x0[NS], x1[NS], x2[NS], x3[NS];
        xs_at<NS>(xt, col0, x0);
        xs_at<NS>(xt, col1, x1);
        xs_at<NS>(xt, col2, x2);
        xs_at<NS>(xt, col3, x3);
#pragma unroll
        for (int i = 0; i < NS; ++i)
          o[i] = fmaf(nibble_value(by3, p), x3[i], fmaf(nibble_value(by2, p), x2[i],
                 fmaf(nibble_value(by1, p), x1[i], fmaf(nibble_value(by0, p), x0[i], o[i]))));
      }
      for (; p + 4 < p_mid; p += 8) {
        const int col0 = lc[p - cbase], col1 = lc[p + 4 - cbase];
        const float q0 = nibble_value(lv[(p >> 1) - vbase], p);
        const float q1 = nibble_value(lv[((p + 4) >> 1) - vbase], p + 4);
        float x0[NS], x1[NS];
        xs_at<NS>(xt, col0, x0);
        xs_at<NS>(xt, col1, x1);
#pragma unroll
        for (int i = 0; i < NS; ++i) o[i] = fmaf(q1, x1[i], fmaf(q0, x0[i], o[i]));
      }
      for (; p < p_mid; p += 4) {
        const int col = lc[p - cbase];
        const float q = nibble_value(lv[(p >> 1) - vbase], p);
        float x0[NS];
        xs_at<NS>(xt, col, x0);
#pragma unroll
        for (int i = 0; i < NS; ++i) o[i] = fmaf(q, x0[i], o[i]);
      }
    } else {
      for (; p < p_mid; p += 4) {
        const int col = lc[p - cbase];
        const float q = nibble_value(lv[(p >> 1) - vbase], p);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (i < it.nslots) {
            const int ra = sel4(i, it.ra0, it.ra1, it.ra2, it.ra3);
            o[i] = fmaf(q, reinterpret_cast<const float*>(P.ra + (size_t)ra * P.ra_stride)[col], o[i]);
          }
        }
      }
    }
    // rows whose entries run past the staged chunks (more than 64 per row on average over
    // the wave's 16 rows): the rest straight from memory, eight entries of the lane per
    // step with all their loads issued before the first use
    if (p < p_end) {
      const gale_matrix* Mo = P.table + it.mat * P.mat_stride + (G.ohalf ? P.sel1 : P.sel0);
      for (; p < p_end; p += 32) {
        int col[8];
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pj = min(p + 4 * j, p_end - 1);
          col[j] = Mo->out_cols[pj];
          q[j] = p + 4 * j < p_end ? (float)outlier_value(Mo->out_vals, pj) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (i < it.nslots) {
            const int ra = sel4(i, it.ra0, it.ra1, it.ra2, it.ra3);
            const float* xg = reinterpret_cast<const float*>(P.ra + (size_t)ra * P.ra_stride);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[i] = fmaf(q[j], P.stage_xt ? xt[NS * col[j] + i] : xg[col[j]], o[i]);
          }
        }
      }
    }
    const float rscale = half_bits_to_float(cur.rsc);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      o[i] += __shfl_xor(o[i], 1, 64);
      o[i] += __shfl_xor(o[i], 2, 64);
      if (G.orole && G.sub == 0) ored[(G.ohalf * RR + G.orow0 + G.wr) * NS + i] = o[i] * rscale;
    }
  }
  // every wave's partials of this unit are in LDS; the buffers alternate between
  // units, so the next unit's writes never meet this unit's reads
  __syncthreads();

  // 6. sum the split-K partials in a fixed order, add the outliers, store
  for (int e = G.tid; e < RR * NS; e += (int)blockDim.x) {
    const int rr = e / NS, i = e - rr * NS;
    const int n = rg * RR + rr;
    if (n >= P.rows || i >= it.nslots) continue;
    float v[HALVES];
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
      float a = 0.f;
      for (int q = 0; q < G.C; ++q) a += red[((hf * G.C + q) * RR + rr) * NS + i];
      v[hf] = a + ored[(hf * RR + rr) * NS + i];
    }
    const int64_t off = (int64_t)sel4(i, it.out0, it.out1, it.out2, it.out3) * P.y_stride + n;
    if (GATEUP) {
      reinterpret_cast<float*>(P.y)[off] = silu_f(v[0]) * v[HALVES - 1];
    } else if (P.y_dtype == GALE_F16) {
      reinterpret_cast<__half*>(P.y)[off] = __float2half_rn(v[0]);
    } else {
      reinterpret_cast<float*>(P.y)[off] = v[0];
    }
  }
}

// NS: activation vectors per item (1, 2 or 4); R: row tiles per unit (R <= chunks);
// GATEUP: two matrices (w1, w3) and a SwiGLU epilogue.  blockDim.x = 64 * C * (GATEUP ? 2 : 1)
// <= MAXT: 512 for up to eight wavefronts, 1024 (half the registers per lane) beyond.
// FX: raw activations (one vector per item): the record is built in LDS (by the w1 half's
// wavefronts when the item is a gate/up pair; both halves read it).
template <int NS, int R, bool GATEUP, int MAXT, int OC, bool FX>
__global__ void __launch_bounds__(MAXT) gemv_kernel(const GemvParams P) {
  static_assert(!FX || NS == 1, "raw activations: one vector per item");
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int HALVES = GATEUP ? 2 : 1;
  constexpr int RR = R * 16;
  Geo G;
  G.K = P.cols;
  G.C = P.cols >> 10;
  G.tid = threadIdx.x;
  G.lane = G.tid & 63;
  G.wave = uni(G.tid >> 6);
  G.half = uni(GATEUP ? (G.wave >= G.C ? 1 : 0) : 0);
  G.c = uni(G.wave - G.half * G.C);
  G.g = G.lane >> 4;
  G.nl = G.lane & 15;
  G.ntiles = P.rows >> 4;
  G.RG = P.row_groups;
  // outlier role: wave w serves unit rows 16 w .. 16 w + 15 (across the halves)
  G.orole = G.wave < HALVES * R;
  G.ohalf = uni(G.orole ? (16 * G.wave) / RR : 0);
  G.orow0 = uni(G.orole ? 16 * G.wave - G.ohalf * RR : 0);
  G.wr = G.lane >> 2;
  G.sub = G.lane & 3;
  // sign words of tile t, chunk c, lane l: byte 2048 (t C + c) + 16 l (and + 1024 for the
  // second half); block scales: byte 256 (t C + c) + 16 (l % 16)
  G.sw_tile = (uint32_t)G.C * 2048u;
  G.sc_tile = (uint32_t)G.C * 256u;
  G.sw_lane = (uint32_t)G.c * 2048u + 16u * (uint32_t)G.lane;
  G.sc_lane = (uint32_t)G.c * 256u + 16u * (uint32_t)G.nl;

  // LDS: two alternating sets of partial sums, the waves' outlier slices, x~
  lds_u8* base = (lds_u8*)smem;
  const int red_n = HALVES * G.C * RR * NS, ored_n = HALVES * RR * NS;
  lds_f32* red0 = reinterpret_cast<lds_f32*>(base);            // [2][HALVES][C][RR][NS]
  lds_f32* ored0 = red0 + 2 * red_n;                            // [2][HALVES][RR][NS]
  lds_u8* wbase = reinterpret_cast<lds_u8*>(ored0 + 2 * ored_n);
  lds_u8* wout = wbase + G.wave * wave_out_bytes(OC);          // this wave's outlier staging slice
  lds_f32* xt = reinterpret_cast<lds_f32*>(wbase + (size_t)HALVES * G.C * wave_out_bytes(OC));   // [NS][K] when staged
  // FX: the item's whole record from xt on (x~ is its first part), then the x copies
  const size_t lrec_off = (size_t)4 * (red_n * 2 + ored_n * 2) + (size_t)HALVES * G.C * wave_out_bytes(OC);
  uint8_t* lrec = smem + lrec_off;
  uint8_t* xstage = smem + lrec_off + ra_bytes(G.K);

  const int n_items = P.implicit_items ? P.n_items : uni(*as_const(P.n_items_dev));
  const int total = n_items * G.RG;
  const int u0 = uni((int)((int64_t)total * blockIdx.x / gridDim.x));
  const int u1 = uni((int)((int64_t)total * (blockIdx.x + 1) / gridDim.x));
  if (u0 >= u1) return;

  UnitBuf<R, OC> b0, b1;
  Act act;
  int act_item;
  Item it;
  Pos pc, p1, p2;
  Desc d1, d2;
  {
    // prologue: the first item's activation operands (independent of the weight
    // descriptors, so their latency overlaps the descriptor and CSR loads), the CSR
    // offsets of u0, the whole of u0 (with the offsets of u0 + 1), then x~ into LDS
    pc.u = u0;
    pc.item = uni(u0 / G.RG);
    pc.rg = uni(u0 - pc.item * G.RG);
    it = decode_item<NS>(P, pc.item);
    float xf[16];
    if constexpr (FX) {
      if (G.half == 0) load_block_coalesced(x_chunk(P, G, it.ra0), P.x_dtype, G.lane, xf);
    } else {
      load_activation<NS>(P, G, it, act);
    }
    const Desc d0 = load_desc(P, G, uni(it.mat));
    p1 = pos_next(pc, u1, G.RG);
    d1 = p1.item == pc.item ? d0 : load_desc(P, G, item_mat(P, p1.item));
    bool ok;
    const int n = outlier_row<R>(P, G, pc.rg, &ok);
    b0.rp0 = d0.rptr[n];
    b0.rp1 = d0.rptr[n + (n < P.rows ? 1 : 0)];
    issue_unit<R, OC>(P, G, pc, d0, p1, d1, b0);
    if constexpr (FX) {
      if (G.half == 0) prep_x_record(P, G, xf, lrec);
      __syncthreads();
      record_activation(lrec, G.K, G.c, G.lane, act);
    } else {
      stage_activation<NS>(P, G, it, xt);
      __syncthreads();
    }
    block_sums<NS>(act);
    act_item = pc.item;
    p2 = pos_next(p1, u1, G.RG);
    d2 = p2.item == p1.item ? d1 : load_desc(P, G, item_mat(P, p2.item));
  }
  for (;;) {
    process_unit<NS, R, GATEUP, OC, FX>(P, G, pc, it, b0, b1, p1, d1, p2, d2, act_item, act, red0, ored0, xt, wout,
                                        lrec, xstage);
    if (pc.u + 1 >= u1) break;
    pc = p1;
    p1 = p2;
    d1 = d2;
    p2 = pos_next(p2, u1, G.RG);
    d2 = p2.item == p1.item ? d1 : load_desc(P, G, item_mat(P, p2.item));
    process_unit<NS, R, GATEUP, OC, FX>(P, G, pc, it, b1, b0, p1, d1, p2, d2, act_item, act, red0 + red_n,
                                        ored0 + ored_n, xt, wout, lrec, xstage);
    if (pc.u + 1 >= u1) break;
    pc = p1;
    p1 = p2;
    d1 = d2;
    p2 = pos_next(p2, u1, G.RG);
    d2 = p2.item == p1.item ? d1 : load_desc(P, G, item_mat(P, p2.item));
  }
}

size_t gemv_smem_bytes(int cols, int slots, int tiles, int gateup, int stage_xt, int out_chunks, int fused) {
  const int halves = gateup ? 2 : 1;
  const int C = cols >> 10;
  const size_t f = 2 * ((size_t)halves * C * tiles * 16 * slots + (size_t)halves * tiles * 16 * slots);
  size_t b = f * 4 + (size_t)halves * C * (size_t)(64 * 16 * (out_chunks + out_chunks / 4 + 1));
  if (fused) return b + ra_bytes(cols) + (size_t)cols * 4;   // the record, then x copies of either dtype
  if (stage_xt) b += (size_t)slots * cols * 4;
  return b;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int NS, int R, bool G, int MAXT, int OC, bool FX>
static hipError_t launch_b(const GemvParams& p, int block, int64_t max_units, hipStream_t s) {
  const size_t smem = gemv_smem_bytes(p.cols, NS, R, G, p.stage_xt, OC, FX ? 1 : 0);
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_kernel<NS, R, G, MAXT, OC, FX>, block, smem) !=
          hipSuccess || occ < 1)
    occ = 1;
  const int64_t grid = std::min<int64_t>(max_units, (int64_t)device_cu_count() * occ);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemv_kernel<NS, R, G, MAXT, OC, FX>), dim3((unsigned)grid), dim3(block), smem, s, p);
  return hipGetLastError();
}

template <int NS, int R, bool G, int OC, bool FX = false>
static hipError_t launch_t(const GemvParams& p, int64_t max_units, hipStream_t s) {
  const int block = 64 * (p.cols >> 10) * (G ? 2 : 1);
  if (block > kGemvMaxThreads) return hipErrorInvalidConfiguration;   // the host checks first
  if constexpr (FX) {
    if (block > 512) return hipErrorInvalidConfiguration;           // the host checks first
    return launch_b<NS, R, G, 512, OC, true>(p, block, max_units, s);
  } else {
    if (block <= 512) return launch_b<NS, R, G, 512, OC, false>(p, block, max_units, s);
    return launch_b<NS, R, G, 1024, OC, false>(p, block, max_units, s);
  }
}

// Raw activations, one vector per item: the staging and tile counts the host picks for one
// vector (two chunks: up to four tiles, four: up to three, eight: up to two).
template <bool G, int OC>
static hipError_t launch_fx(const GemvParams& p, int tiles, int64_t max_units, hipStream_t s) {
  switch (tiles) {
    case 1: return launch_t<1, 1, G, OC, true>(p, max_units, s);
    case 2: return launch_t<1, 2, G, OC, true>(p, max_units, s);
    case 3:
      if constexpr (OC <= 4) return launch_t<1, 3, G, OC, true>(p, max_units, s);
      else return hipErrorInvalidValue;
    case 4:
      if constexpr (OC == 2) return launch_t<1, 4, G, OC, true>(p, max_units, s);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// Row tiles per unit by outlier staging.  One chunk (the down phase of a layer whose
// intermediate size is at most half the hidden size): as four chunks.  Two chunks: four
// tiles for items of up to two
// vectors, three for four vectors (four would spill).  Four chunks (twice the staged
// entries): three tiles for up to two vectors, two for four.  Eight chunks: one vector,
// up to two tiles (two spill a few registers, and still stream 1.4x faster than one).
// The host's row groups are counted with the same tile count, so no other value is taken.
template <int NS, bool G, int OC>
static hipError_t launch_r(const GemvParams& p, int tiles, int64_t max_units, hipStream_t s) {
  if constexpr (OC == 8) {
    if (NS == 1 && tiles == 1) return launch_t<1, 1, G, 8>(p, max_units, s);
    if (NS == 1 && tiles == 2) return launch_t<1, 2, G, 8>(p, max_units, s);
    return hipErrorInvalidValue;
  } else {
    constexpr int kMax = OC == 2 ? (NS <= 2 ? 4 : 3) : (NS <= 2 ? 3 : 2);
    switch (tiles) {
      case 1: return launch_t<NS, 1, G, OC>(p, max_units, s);
      case 2: return launch_t<NS, 2, G, OC>(p, max_units, s);
      case 3:
        if constexpr (kMax >= 3) return launch_t<NS, 3, G, OC>(p, max_units, s);
        else return hipErrorInvalidValue;
      case 4:
        if constexpr (kMax >= 4) return launch_t<NS, 4, G, OC>(p, max_units, s);
        else return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
}

template <bool G, int OC>
static hipError_t launch_s(const GemvParams& p, int slots, int tiles, int64_t max_units, hipStream_t s) {
  if (slots == 1) return launch_r<1, G, OC>(p, tiles, max_units, s);
  if (slots == 2) return launch_r<2, G, OC>(p, tiles, max_units, s);
  return launch_r<4, G, OC>(p, tiles, max_units, s);
}

template <bool G>
static hipError_t launch_o(const GemvParams& p, int slots, int tiles, int64_t max_units, hipStream_t s) {
  if constexpr (!G) {
    if (p.out_chunks == 1) return launch_s<G, 1>(p, slots, tiles, max_units, s);
  }
  if (p.out_chunks == 8) return launch_s<G, 8>(p, slots, tiles, max_units, s);
  if (p.out_chunks == 4) return launch_s<G, 4>(p, slots, tiles, max_units, s);
  if (p.out_chunks == 2) return launch_s<G, 2>(p, slots, tiles, max_units, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemvParams& p, int slots, int tiles_per_unit, int64_t max_units, hipStream_t s) {
  if (max_units <= 0) return hipSuccess;
  if (p.x) {
    if (slots != 1) return hipErrorInvalidValue;   // the host checks first
    if (p.gateup) {
      if (p.out_chunks == 4) return launch_fx<true, 4>(p, tiles_per_unit, max_units, s);
      if (p.out_chunks == 2) return launch_fx<true, 2>(p, tiles_per_unit, max_units, s);
      return hipErrorInvalidValue;
    }
    if (p.out_chunks == 8) return launch_fx<false, 8>(p, tiles_per_unit, max_units, s);
    if (p.out_chunks == 4) return launch_fx<false, 4>(p, tiles_per_unit, max_units, s);
    if (p.out_chunks == 2) return launch_fx<false, 2>(p, tiles_per_unit, max_units, s);
    if (p.out_chunks == 1) return launch_fx<false, 1>(p, tiles_per_unit, max_units, s);
    return hipErrorInvalidValue;
  }
  if (p.gateup) return launch_o<true>(p, slots, tiles_per_unit, max_units, s);
  return launch_o<false>(p, slots, tiles_per_unit, max_units, s);
}

}  // namespace gale
