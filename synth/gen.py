"""Seeded synthetic inputs for the GALE 1-bit expert format.

This module is shared by the fp64 oracle and by the GPU harness.  It holds no
part of the method's arithmetic: it only draws random numbers and stores them in
the *canonical* interchange format described below.  Everything is built from a
counter-based generator (the SplitMix64 output function of Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014) evaluated with
int64 tensor ops, so the same call returns bit-identical tensors on the CPU and
on a GPU: integer ops are exact, and the only float ops used (table lookups and
single IEEE add/sub/mul in fp32) are correctly rounded on both.

Canonical format of one matrix with ``N`` rows (outputs) and ``K`` columns
(inputs), K a multiple of 1024 (DeepSeek-V4-Flash GALE model card, "What is in
the pack": one sign bit per weight under a blocked FWHT-1024 rotation, an fp16
scale per 128-weight block, 1 % int4 outliers with a per-row fp16 scale):

  signs        int32 [N, K/32]   bit (k % 32) of word k // 32 is b[n, k]; b = 1 means negative
  block_scales int16 [N, K/128]  fp16 bit patterns, block j covers columns 128j..128j+127
  row_scales   int16 [N]         fp16 bit patterns (outlier scale)
  row_ptr      int32 [N+1]       CSR offsets
  out_cols     int16 [nnz]       uint16 column indices, ascending within a row
  out_vals     uint8 [ceil(nnz/2)] int4 two's complement, entry j in byte j//2, low nibble if j even

Distributions (one 2048x4096 matrix, one token): signs Bernoulli(1/2); block
scales fp16(|z| * 0.02); round(0.01 K) distinct uniform outlier columns per row
with int4 values uniform in [-8, 7] and row scale fp16(0.05); x ~ fp16(z) with
round(0.001 K) distinct positions per token set to fp16(20 z); router logits
fp32 z; prefill logits log p_r + Gumbel with p_r ~ r^-1.1 (Zipf(1.1)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "GOLDEN", "mix64_int", "stream_key", "bits64", "CanonicalMatrix",
    "gen_matrix", "gen_matrices", "gen_matrix_bank", "gen_x", "gen_logits_normal", "gen_logits_zipf",
    "config_seed", "MAT_W1", "MAT_W3", "MAT_W2", "n_outliers",
]

_M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB

MAT_W1, MAT_W3, MAT_W2 = 0, 1, 2

# section tags used in stream keys
_SEC_SIGNS, _SEC_SCALES, _SEC_OCOLS, _SEC_OVALS = 1, 2, 3, 4
_SEC_X, _SEC_XSPIKE, _SEC_LOGITS, _SEC_ZIPF_PERM, _SEC_GUMBEL = 5, 6, 7, 8, 9


def config_seed(i: int) -> int:
    """Base seed of workload i: the ASCII bytes 'GALE' in the high word, i in the low word."""
    return 0x47414C45_00000000 + int(i)


def _s64(v: int) -> int:
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference for the tensor version)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def stream_key(seed: int, *ids: int) -> int:
    """Key of one random stream, derived from the base seed and a path of small ids."""
    k = mix64_int(seed)
    for i in ids:
        k = mix64_int(k ^ ((int(i) + 1) * GOLDEN & _M64))
    return k


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    # logical right shift on int64 (torch's >> is arithmetic)
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_C1)
    z = (z ^ _lsr(z, 27)) * _s64(_C2)
    return z ^ _lsr(z, 31)


def bits64(key, idx: torch.Tensor) -> torch.Tensor:
    """64 random bits (as int64) for element indices ``idx`` of stream ``key``.

    ``key`` is a Python int or an int64 tensor broadcastable against ``idx``.
    """
    if isinstance(key, int):
        key = _s64(key)
    return _mix64((idx + 1) * _s64(GOLDEN) + key)


def _hi16(b: torch.Tensor) -> torch.Tensor:
    return _lsr(b, 48)


def _lo32(b: torch.Tensor) -> torch.Tensor:
    return b & 0xFFFFFFFF


# --------------------------------------------------------------------------
# value tables: inverse normal CDF at the 65536 midpoints, built once in fp64
# --------------------------------------------------------------------------
_TABLES: Dict[str, np.ndarray] = {}


def _tables() -> Dict[str, np.ndarray]:
    if not _TABLES:
        from scipy.special import ndtri
        u = (np.arange(65537, dtype=np.float64) + 0.5) / 65536.0
        u[-1] = min(u[-1], 1.0 - 0.25 / 65536.0)
        z = ndtri(u)                                   # Phi^-1 at midpoints (+1 guard entry)
        _TABLES["z32"] = z.astype(np.float32)          # fp32 normal, for interpolation
        _TABLES["x16"] = z[:65536].astype(np.float16).view(np.int16)
        _TABLES["spike16"] = (20.0 * z[:65536]).astype(np.float16).view(np.int16)
        _TABLES["scale16"] = (np.abs(z[:65536]) * 0.02).astype(np.float16).view(np.int16)
        g = -np.log(-np.log(u))                        # Gumbel(0,1) inverse CDF
        _TABLES["gumbel32"] = g.astype(np.float32)
    return _TABLES


def _table(name: str, device) -> torch.Tensor:
    return torch.from_numpy(_tables()[name]).to(device)


def _interp32(name: str, b: torch.Tensor) -> torch.Tensor:
    """fp32 value from 32 random bits: table at the high 16 bits, linear step by the low 16."""
    t = _table(name, b.device)
    hi = _lsr(b, 48)
    lo = (_lsr(b, 32) & 0xFFFF).to(torch.float32) * (1.0 / 65536.0)
    t0 = t[hi]
    t1 = t[hi + 1]
    return t0 + lo * (t1 - t0)


def _distinct_uniform(key_rows: torch.Tensor, count: int, n: int) -> torch.Tensor:
    """``count`` distinct integers uniform in [0, n) per row, sorted ascending.

    Draw all, then repeatedly redraw the later copy of each duplicate; the
    procedure is symmetric under relabelling [0, n), so every subset of size
    ``count`` is equally likely.  ``key_rows``: int64 [R] stream keys, one per row.
    """
    R = key_rows.shape[0]
    dev = key_rows.device
    slot = torch.arange(count, device=dev, dtype=torch.int64)
    kr = key_rows[:, None]

    def draw(rnd: int, pos: torch.Tensor) -> torch.Tensor:
        b = bits64(kr, pos + rnd * count)
        return (_lsr(b, 32) * n) >> 32               # multiply-high: uniform in [0, n)

    vals = torch.sort(draw(0, slot.expand(R, count)), dim=1).values
    rnd = 1
    while True:
        dup = torch.zeros_like(vals, dtype=torch.bool)
        dup[:, 1:] = vals[:, 1:] == vals[:, :-1]
        if not bool(dup.any()):
            return vals
        fresh = draw(rnd, slot.expand(R, count))
        vals = torch.sort(torch.where(dup, fresh, vals), dim=1).values
        rnd += 1
        if rnd > 1000:
            raise RuntimeError("outlier column sampling did not converge")


# --------------------------------------------------------------------------
# matrices
# --------------------------------------------------------------------------
def n_outliers(K: int, frac: float = 0.01) -> int:
    """Outliers per row: round(frac * K) (41 for K=4096, 20 for K=2048 at 1 %)."""
    return int(math.floor(frac * K + 0.5))


@dataclass
class CanonicalMatrix:
    rows: int
    cols: int
    signs: torch.Tensor         # int32 [N, K/32]
    block_scales: torch.Tensor  # int16 [N, K/128] (fp16 bits)
    row_scales: torch.Tensor    # int16 [N] (fp16 bits)
    row_ptr: torch.Tensor       # int32 [N+1]
    out_cols: torch.Tensor      # int16 [nnz] (uint16 values)
    out_vals: torch.Tensor      # uint8 [ceil(nnz/2)]

    @property
    def nnz(self) -> int:
        return int(self.out_cols.shape[0])

    def to(self, device) -> "CanonicalMatrix":
        return CanonicalMatrix(self.rows, self.cols, *[getattr(self, f).to(device) for f in
                               ("signs", "block_scales", "row_scales", "row_ptr", "out_cols", "out_vals")])

    def numpy(self) -> Dict[str, np.ndarray]:
        """Host copies with the canonical numpy dtypes (uint32 / float16 / uint16 / uint8)."""
        return {
            "rows": self.rows, "cols": self.cols,
            "signs": self.signs.cpu().numpy().view(np.uint32),
            "block_scales": self.block_scales.cpu().numpy().view(np.float16),
            "row_scales": self.row_scales.cpu().numpy().view(np.float16),
            "row_ptr": self.row_ptr.cpu().numpy().astype(np.int64),
            "out_cols": self.out_cols.cpu().numpy().view(np.uint16),
            "out_vals": self.out_vals.cpu().numpy(),
        }


def gen_matrix_bank(seed: int, ids: Sequence[Sequence[int]], rows: int, cols: int,
                    outlier_frac: float = 0.01, row_scale: float = 0.05, device="cpu") -> Dict[str, torch.Tensor]:
    """Canonical sections of several same-shape matrices as stacked tensors; matrix i is keyed
    by (seed, *ids[i]):

      signs [M, N, K/32] int32, block_scales [M, N, K/128] int16, out_cols [M, N*cnt] int16,
      out_vals [M, ceil(N*cnt/2)] uint8, and, shared by all M (fixed count per row, fixed
      scale), row_ptr [N+1] int32 and row_scales [N] int16.
    """
    if cols % 1024 != 0:
        raise ValueError("cols must be a multiple of 1024")
    M = len(ids)
    N, K = rows, cols
    dev = torch.device(device)
    keys = {sec: torch.tensor([_s64(stream_key(seed, *p, sec)) for p in ids],
                              dtype=torch.int64, device=dev)
            for sec in (_SEC_SIGNS, _SEC_SCALES, _SEC_OCOLS, _SEC_OVALS)}
    nw = N * (K // 32)
    words = _lo32(bits64(keys[_SEC_SIGNS][:, None], torch.arange(nw, device=dev, dtype=torch.int64)[None, :]))
    words = words.to(torch.int32).view(M, N, K // 32)   # low 32 bits, two's complement
    nb = N * (K // 128)
    sb = bits64(keys[_SEC_SCALES][:, None], torch.arange(nb, device=dev, dtype=torch.int64)[None, :])
    scales = _table("scale16", dev)[_hi16(sb)].view(M, N, K // 128)
    del sb
    rs_bits = int(np.array([row_scale], dtype=np.float16).view(np.int16)[0])
    cnt = n_outliers(K, outlier_frac)
    if cnt > 0:
        row_idx = torch.arange(N, device=dev, dtype=torch.int64)
        row_keys = bits64(keys[_SEC_OCOLS][:, None], row_idx[None, :]).reshape(-1)
        cols_all = _distinct_uniform(row_keys, cnt, K).view(M, N * cnt).to(torch.int32).to(torch.int16)
        vb = bits64(keys[_SEC_OVALS][:, None], torch.arange(N * cnt, device=dev, dtype=torch.int64)[None, :])
        nib = _lsr(vb, 60)                                      # 4 random bits = int4 two's complement
        if (N * cnt) % 2:
            nib = torch.cat([nib, torch.zeros(M, 1, dtype=nib.dtype, device=dev)], dim=1)
        nib = nib.view(M, -1, 2)
        vals_all = (nib[:, :, 0] | (nib[:, :, 1] << 4)).to(torch.uint8)
    else:
        cols_all = torch.zeros(M, 0, dtype=torch.int16, device=dev)
        vals_all = torch.zeros(M, 0, dtype=torch.uint8, device=dev)
    return {
        "signs": words, "block_scales": scales, "out_cols": cols_all, "out_vals": vals_all,
        "row_ptr": (torch.arange(N + 1, device=dev, dtype=torch.int64) * cnt).to(torch.int32),
        "row_scales": torch.full((N,), rs_bits, dtype=torch.int16, device=dev),
    }


def gen_matrices(seed: int, ids: Sequence[Sequence[int]], rows: int, cols: int,
                 outlier_frac: float = 0.01, row_scale: float = 0.05,
                 device="cpu") -> list:
    """Generate several matrices at once; matrix i is keyed by (seed, *ids[i]).

    The result for one id path does not depend on which other ids are requested,
    so any single matrix can be regenerated on its own (e.g. by the oracle).
    """
    b = gen_matrix_bank(seed, ids, rows, cols, outlier_frac, row_scale, device)
    out = []
    for m in range(len(ids)):
        out.append(CanonicalMatrix(
            rows=rows, cols=cols,
            signs=b["signs"][m].contiguous(),
            block_scales=b["block_scales"][m].contiguous(),
            row_scales=b["row_scales"].clone(),
            row_ptr=b["row_ptr"].clone(),
            out_cols=b["out_cols"][m].contiguous(),
            out_vals=b["out_vals"][m].contiguous(),
        ))
    return out


def gen_matrix(seed: int, ids: Sequence[int], rows: int, cols: int, **kw) -> CanonicalMatrix:
    return gen_matrices(seed, [tuple(ids)], rows, cols, **kw)[0]


# --------------------------------------------------------------------------
# activations and router logits
# --------------------------------------------------------------------------
def gen_x(seed: int, ids: Sequence[int], n_tok: int, K: int, spike_frac: float = 0.001,
          device="cpu") -> torch.Tensor:
    """fp16 [n_tok, K] activations: N(0,1) with round(spike_frac*K) distinct entries x20 per token."""
    dev = torch.device(device)
    kx = stream_key(seed, *ids, _SEC_X)
    b = bits64(kx, torch.arange(n_tok * K, device=dev, dtype=torch.int64)).view(n_tok, K)
    x = _table("x16", dev)[_hi16(b)]
    ns = int(math.floor(spike_frac * K + 0.5))
    if ns > 0:
        ks = torch.tensor([_s64(stream_key(seed, *ids, _SEC_XSPIKE, t)) for t in range(n_tok)],
                          dtype=torch.int64, device=dev)
        pos = _distinct_uniform(ks, ns, K)
        spike = _table("spike16", dev)[_hi16(b)]
        x = x.scatter(1, pos, torch.gather(spike, 1, pos))
    return x.view(torch.float16)


def gen_logits_normal(seed: int, ids: Sequence[int], n_tok: int, n_exp: int, device="cpu") -> torch.Tensor:
    """fp32 [n_tok, n_exp] router logits ~ N(0,1)."""
    dev = torch.device(device)
    k = stream_key(seed, *ids, _SEC_LOGITS)
    b = bits64(k, torch.arange(n_tok * n_exp, device=dev, dtype=torch.int64))
    return _interp32("z32", b).view(n_tok, n_exp)


def gen_logits_zipf(seed: int, ids: Sequence[int], n_tok: int, n_exp: int, s: float = 1.1,
                    device="cpu") -> torch.Tensor:
    """fp32 [n_tok, n_exp] logits log p_rank(e) + Gumbel(0,1), p_r ~ r^-s, rank->expert by a seeded permutation.

    Taking the top-k of these logits draws k experts without replacement with
    probability proportional to p (the Gumbel-top-k identity), so the routing is
    Zipf-skewed across experts.
    """
    dev = torch.device(device)
    r = np.arange(1, n_exp + 1, dtype=np.float64)
    p = r ** (-s)
    logp = np.log(p / p.sum()).astype(np.float32)
    kp = stream_key(seed, *ids, _SEC_ZIPF_PERM)
    perm_keys = bits64(kp, torch.arange(n_exp, dtype=torch.int64))
    rank_of_expert = torch.argsort(perm_keys, stable=True)      # expert e has rank rank_of_expert[e]
    lp = torch.from_numpy(logp)[rank_of_expert].to(dev)
    kg = stream_key(seed, *ids, _SEC_GUMBEL)
    b = bits64(kg, torch.arange(n_tok * n_exp, device=dev, dtype=torch.int64))
    g = _interp32("gumbel32", b).view(n_tok, n_exp)
    return lp[None, :] + g
