"""Plain fp64 CPU oracle for the GALE 1-bit routed-expert matmul.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the GPU library: it never loads it, and the GPU library never loads this.  The
one thing both sides use is the seeded input generator (package ``synth``),
which holds none of the method's arithmetic.

Everything here is written for a reader to check against the pages by eye:
explicit dense Hadamard matrix, explicit dense dequantized weight matrix, then a
matrix-vector product (numpy ``@`` as the one library primitive), all in fp64.

Sources (cited by page title and section):
  [Flash]  "DeepSeek-V4-Flash - GALE 1-bit experts" model card, section "What is
           in the pack": routed experts w1/w3 [2048,4096] and w2 [4096,2048]; a
           sign bit per weight under a blocked FWHT-1024 rotation; an fp16 scale
           per 128-weight block; 1 % outliers as int4 with a per-row fp16 scale;
           1.329 bits/weight; 46.0 GB; 277.0 B parameters in 33,024 matrices.
  [Flash-perf] same card, "Measured performance": 258 = 43 x 6 experts per token.
  [Pro]    "DeepSeek-V4-Pro-671B-GALE-1bit-v4" page, serving-knobs paragraph on
           DSV4_DIRECT_GEMV / DSV4_FWHT: a GEMV straight out of the packed record
           (signs, block scales, int4 outliers decoded in registers) and a
           single-kernel Walsh-Hadamard transform exact to 1e-8 of the matmul form.
           Same page, serving notes on the tier bias: a per-expert selection bias
           (DeepSeek's aux-loss-free balancing term) changes which experts are chosen,
           never the routing weights.
  [REAP]   DeepSeek-V4-Flash 180B REAP W4A16 card, lineage notes: layers 0-2 route
           by hash, reading the experts of each token from a token-to-expert table.

Readings taken where the pages are silent (each also listed in the design notes):
  * H is the Sylvester-ordered Walsh-Hadamard matrix normalised by 1/sqrt(1024)
    (orthonormal, symmetric, H.H = I); no random sign diagonal.
  * The rotation acts on the input side: y = Wq . (blockdiag(H) . x).
  * A scale block is 128 consecutive input columns of one row.
  * Sign bit 1 means negative: w = s * (1 - 2 b).
  * Outliers are additive: Wq[n, c] += r[n] * q at each listed (n, c).
  * FFN: h = silu(w1 x~) * (w3 x~), y = w2 . (blockdiag(H) . h), silu(a) = a / (1 + e^-a).
  * Routing: top-k by (logit descending, expert index ascending); weights are the
    softmax of the k selected logits.
  * Selection bias: added to the fp32 logits (an fp32 sum) for the ordering only.
  * Hash routing: the pages give the token-to-expert table but not the weights; they
    are taken as the softmax of the given experts' logits, as on the other layers.
"""
from __future__ import annotations

import sys
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

assert sys.byteorder == "little", "canonical sign words are read as little-endian bytes"

FWHT_N = 1024          # [Flash] "blocked FWHT-1024 rotation"
SCALE_BLOCK = 128      # [Flash] "fp16 scale per 128-weight block"


# --------------------------------------------------------------------------
# O1, O2: Hadamard matrix and blocked rotation
# --------------------------------------------------------------------------
def popcount(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.uint64)
    c = np.zeros(v.shape, dtype=np.int64)
    while np.any(v):
        c += (v & np.uint64(1)).astype(np.int64)
        v = v >> np.uint64(1)
    return c


_H_CACHE: Dict[Tuple[int, bool], np.ndarray] = {}


def hadamard(n: int = FWHT_N, normalized: bool = True) -> np.ndarray:
    """Explicit dense Walsh-Hadamard matrix H[i, j] = (-1)^popcount(i AND j) (/ sqrt(n))."""
    key = (n, normalized)
    if key not in _H_CACHE:
        i = np.arange(n, dtype=np.uint64)
        sign = 1.0 - 2.0 * (popcount(i[:, None] & i[None, :]) & 1)
        H = sign.astype(np.float64)
        if normalized:
            H = H / np.sqrt(float(n))
        _H_CACHE[key] = H
    return _H_CACHE[key]


def rotate(x: np.ndarray, n: int = FWHT_N) -> np.ndarray:
    """x~ = blockdiag(H_n, ..., H_n) . x along the last axis (length a multiple of n)."""
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-1]
    if L % n:
        raise ValueError("length must be a multiple of the FWHT block")
    H = hadamard(n)
    xb = x.reshape(x.shape[:-1] + (L // n, n))
    return (xb @ H.T).reshape(x.shape)


# --------------------------------------------------------------------------
# O3: dequantize a canonical GALE matrix into a dense fp64 matrix
# --------------------------------------------------------------------------
def unpack_signs(words: np.ndarray, cols: int) -> np.ndarray:
    """uint32 [N, K/32] -> uint8 [N, K]; b[n, k] = bit (k % 32) of word k // 32."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    by = w.view(np.uint8).reshape(w.shape[0], -1)
    b = np.unpackbits(by, axis=1, bitorder="little")
    assert b.shape[1] == cols
    return b


def decode_int4(packed: np.ndarray, nnz: int) -> np.ndarray:
    """uint8 [ceil(nnz/2)] -> int64 [nnz]; entry j is the low nibble of byte j//2 when j is even."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    nib = np.empty(2 * p.shape[0], dtype=np.int64)
    nib[0::2] = p & 0xF
    nib[1::2] = p >> 4
    nib = nib[:nnz]
    return np.where(nib >= 8, nib - 16, nib)          # two's complement


def outlier_triplets(m: Dict) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(row, column, int4 value) of every outlier, in CSR order."""
    rp = np.asarray(m["row_ptr"], dtype=np.int64)
    nnz = int(rp[-1])
    rows = np.repeat(np.arange(m["rows"], dtype=np.int64), np.diff(rp))
    cols = np.asarray(m["out_cols"], dtype=np.uint16).astype(np.int64)[:nnz]
    vals = decode_int4(m["out_vals"], nnz)
    return rows, cols, vals


def dequantize(m: Dict) -> np.ndarray:
    """Dense fp64 Wq [N, K]: Wq = s[n, k//128] * (1 - 2 b[n, k]) + sum of r[n] * q at outliers."""
    N, K = m["rows"], m["cols"]
    b = unpack_signs(m["signs"], K).astype(np.float64)
    s = np.asarray(m["block_scales"], dtype=np.float16).astype(np.float64)      # [N, K/128]
    W = np.repeat(s, SCALE_BLOCK, axis=1) * (1.0 - 2.0 * b)
    rows, cols, vals = outlier_triplets(m)
    r = np.asarray(m["row_scales"], dtype=np.float16).astype(np.float64)
    np.add.at(W, (rows, cols), r[rows] * vals.astype(np.float64))
    return W


# --------------------------------------------------------------------------
# O4: GEMV  y = Wq . (blockdiag(H) . x)
# --------------------------------------------------------------------------
def gemv(m: Dict, x: np.ndarray, pre_rotated: bool = False) -> np.ndarray:
    """x [T, K] (any float dtype) -> y [T, N] fp64."""
    x = np.atleast_2d(np.asarray(x).astype(np.float64))
    xt = x if pre_rotated else rotate(x)
    return xt @ dequantize(m).T


# --------------------------------------------------------------------------
# O5: expert FFN
# --------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def ffn(w1: Dict, w3: Dict, w2: Dict, x: np.ndarray) -> np.ndarray:
    """y = w2 . H(silu(w1 . H x) * (w3 . H x)); x [T, hidden] -> y [T, hidden] fp64."""
    x = np.atleast_2d(np.asarray(x).astype(np.float64))
    xt = rotate(x)
    a = xt @ dequantize(w1).T
    g = xt @ dequantize(w3).T
    h = silu(a) * g
    return rotate(h) @ dequantize(w2).T


# --------------------------------------------------------------------------
# O6, O7: routing and combine
# --------------------------------------------------------------------------
def route(logits: np.ndarray, k: int, select_bias: Optional[np.ndarray] = None,
          fixed_idx: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token ordered by (logit desc, index asc); softmax over the k chosen logits.

    logits: fp32 [T, E].  Returns idx int64 [T, k] and weights fp64 [T, k].

    Routing variants ([Pro] serving notes on the tier bias; [REAP] hash-routed layers):
      select_bias fp32 [E]: DeepSeek's balancing term, added to the logits for the choice of
        the k experts only -- the order is taken on the fp32 sums logit + bias (same ties
        rule) and the weights remain the softmax of the chosen experts' own logits.
      fixed_idx [T, k]: the experts come from a token-to-expert table (hash routing), in slot
        order; the weights are the softmax of those experts' logits.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    ar = np.arange(E)
    score = lg if select_bias is None else lg + np.asarray(select_bias, dtype=np.float32)[None, :]   # fp32 sums
    for t in range(T):
        if fixed_idx is not None:
            sel = np.asarray(fixed_idx[t], dtype=np.int64)
        else:
            order = np.lexsort((ar, -score[t].astype(np.float64)))   # primary: -score, secondary: index
            sel = order[:k]
        idx[t] = sel
        v = lg[t, sel].astype(np.float64)
        e = np.exp(v - v.max())
        w[t] = e / e.sum()
    return idx, w


def moe(expert_of, logits: np.ndarray, x: np.ndarray, k: int = 6, select_bias: Optional[np.ndarray] = None,
        fixed_idx: Optional[np.ndarray] = None, map_fn=map):
    """y_t = sum over the k routed experts e of w[t, e] * FFN_e(x_t).

    ``expert_of(e)`` returns the canonical (w1, w3, w2) of expert e.  Returns
    (y fp64 [T, hidden], idx, weights).  select_bias / fixed_idx: the routing variants of
    ``route``.  ``map_fn`` evaluates the per-expert FFNs (each an independent call of
    ``ffn`` on that expert's tokens); a thread pool's map runs them side by side without
    changing any result.
    """
    x = np.atleast_2d(np.asarray(x).astype(np.float64))
    idx, w = route(logits, k, select_bias, fixed_idx)
    y = np.zeros_like(x)
    experts = [int(e) for e in np.unique(idx)]
    toks_of = {e: np.nonzero((idx == e).any(axis=1))[0] for e in experts}

    def expert_ffn(e):
        w1, w3, w2 = expert_of(e)
        return ffn(w1, w3, w2, x[toks_of[e]])

    for e, ye in zip(experts, map_fn(expert_ffn, experts)):
        for j, t in enumerate(toks_of[e]):
            slot = int(np.nonzero(idx[t] == e)[0][0])
            y[t] += w[t, slot] * ye[j]
    return y, idx, w


def group_by_expert(idx: np.ndarray, n_experts: int) -> Tuple[np.ndarray, np.ndarray]:
    """Stable grouping of the (token, slot) pairs by expert: offsets [E+1] and pair list [T*k].

    Pairs are numbered t*k + slot; within an expert they stay in ascending order.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(flat, kind="stable")
    return offsets, perm


# --------------------------------------------------------------------------
# format accounting ([Flash] table: 1.329 bits/weight, 46.0 GB)
# --------------------------------------------------------------------------
def packed_bytes(N: int, K: int, nnz: int) -> Dict[str, int]:
    """Bytes of each section of one matrix: signs, fp16 block scales, uint16 outlier
    columns, int4 outlier values, fp16 row scales.  CSR row offsets are an index,
    not counted."""
    return {
        "signs": N * K // 8,
        "block_scales": 2 * N * (K // SCALE_BLOCK),
        "out_cols": 2 * nnz,
        "out_vals": (nnz + 1) // 2,
        "row_scales": 2 * N,
    }


def bits_per_weight(N: int, K: int, nnz: int) -> float:
    return 8.0 * sum(packed_bytes(N, K, nnz).values()) / (N * K)


def bits_per_weight_closed_form(outlier_frac: float, K: int) -> float:
    """1 + 16/128 + frac * (16 + 4) + 16/K: sign, block scale, outlier (uint16 col + int4), row scale."""
    return 1.0 + 16.0 / SCALE_BLOCK + outlier_frac * (16 + 4) + 16.0 / K


# --------------------------------------------------------------------------
# comparison metric
# --------------------------------------------------------------------------
def rel_l2(y: np.ndarray, ref: np.ndarray, axis: int = -1) -> np.ndarray:
    """||y - ref|| / ||ref|| per vector along ``axis`` (fp64)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(y - ref, axis=axis)
    den = np.linalg.norm(ref, axis=axis)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
