"""ctypes binding of libgale (include/gale.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  torch supplies device memory and the current stream; nothing here
computes the method, and there is no fallback: if libgale.so is missing or the
GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgale.so")

GALE_OK = 0
GALE_F16, GALE_F32 = 1, 2
GALE_X_ROTATED = 0x1
GALE_X_PREPARED = 0x2
GALE_PATH_DECODE = 0x10
GALE_PATH_GROUPED = 0x20
GALE_GROUPED_ITEMS = 0x40
GALE_GROUPED_GEMM = 0x80
GALE_DECODE_STAGED = 0x1000
GALE_SYNC_NO_WAIT = 0x10000
GALE_SYNC_BYTES = 40960
GALE_STATIC_SCRATCH_BYTES = GALE_SYNC_BYTES + 196608
GALE_ERR_SYNC = -9
STATUS = {0: "GALE_OK", -1: "GALE_ERR_NULL", -2: "GALE_ERR_SHAPE", -3: "GALE_ERR_DTYPE", -4: "GALE_ERR_ALIGN",
          -5: "GALE_ERR_WORKSPACE", -6: "GALE_ERR_UNSUPPORTED", -7: "GALE_ERR_FORMAT", -8: "GALE_ERR_HIP",
          -9: "GALE_ERR_SYNC"}


def gale_tiles_flag(r: int) -> int:
    """flags bits 8..11 force the GEMV kernels' row tiles per unit (1, 2, 4 or 8)."""
    return ((r.bit_length()) & 0xF) << 8


GALE_OUTLIER_STAGE_SHIFT = 14


def gale_outlier_stage_flag(per_row: float) -> int:
    """flags bits 14..15 for a mean outlier count per row: the GEMV staging (1024, 2048 or
    4096 entries per 16-row group) that holds a 16-row group's entries.  Measured on
    [2048, 4096]: 1 % (41 per row) streams fastest with 1024, 2 and 3 % (82, 123) with 2048,
    5 % (205) with 4096."""
    v = 0 if per_row <= 48 else (1 if per_row <= 128 else 2)
    return v << GALE_OUTLIER_STAGE_SHIFT


def _with_stage(flags: int, table: "DescriptorTable") -> int:
    """flags with the outlier staging of the table's densest matrix, unless the caller set it."""
    if (flags >> GALE_OUTLIER_STAGE_SHIFT) & 3:
        return flags
    return flags | gale_outlier_stage_flag(table.outliers_per_row)


def gale_layer_tiles_flag(gate_up: int) -> int:
    """flags bits 8..11 for the one-launch decode: row tiles per gate/up unit (1, 2 or 3)."""
    if gate_up not in (1, 2, 3):
        raise ValueError("the one-launch decode takes 1, 2 or 3 gate/up tiles per unit")
    return gate_up << 8


class GaleError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {detail}")
        self.status = status


class gale_matrix(ctypes.Structure):
    _fields_ = [("signs", ctypes.c_void_p), ("block_scales", ctypes.c_void_p), ("row_scales", ctypes.c_void_p),
                ("row_ptr", ctypes.c_void_p), ("out_cols", ctypes.c_void_p), ("out_vals", ctypes.c_void_p)]


class gale_expert(ctypes.Structure):
    _fields_ = [("w1", gale_matrix), ("w3", gale_matrix), ("w2", gale_matrix)]


class gale_layer_io(ctypes.Structure):
    _fields_ = [("experts", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("select_bias", ctypes.c_void_p),
                ("fixed_idx", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p)]


class gale_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("signs", "block_scales", "row_scales", "row_ptr", "out_cols", "out_vals", "format_bytes")]


_I32, _I64, _U32, _SZ, _P = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes)
_SIGS = {
    "gale_status_str": (ctypes.c_char_p, [_I32]),
    "gale_last_error": (ctypes.c_char_p, []),
    "gale_packed_sizes": (_I32, [_I32, _I32, _I64, ctypes.POINTER(gale_sizes)]),
    "gale_check_canonical": (_I32, [_I32, _I32, _P, _P, _I64]),
    "gale_pack_host": (_I32, [_I32, _I32, _P, _P, _P, _P]),
    "gale_unpack_host": (_I32, [_I32, _I32, _P, _P, _P, _P]),
    "gale_pack_device": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "gale_debug_unpack_signs": (_I32, [_I32, _I32, _P, _P, _P]),
    "gale_debug_unpack_outliers": (_I32, [_I32, _I64, ctypes.POINTER(gale_matrix), _P, _P, _P, _P]),
    "gale_fwht1024": (_I32, [_P, _P, _I64, _I32, _I32, _I32, _P]),
    "gale_prepared_bytes": (_SZ, [_I32]),
    "gale_prepare_activations": (_I32, [_P, _I32, _I64, _I32, _U32, _P, _SZ, _P]),
    "gale_gemv_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "gale_expert_gemv": (_I32, [_I32, _I32, _P, _I32, _P, _I32, _I32, _I32, _P, _I32, _P, _SZ, _U32, _P]),
    "gale_ffn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "gale_expert_ffn": (_I32, [_I32, _I32, _P, _I32, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "gale_moe_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _U32]),
    "gale_moe_layer_fwd": (_I32, [_I32, _I32, _P, _I32, _P, _I32, _P, _I32, _P, _P, _P, _P, _SZ, _U32, _P]),
    "gale_moe_layer_fwd_routed": (_I32, [_I32, _I32, _P, _I32, _P, _P, _P, _I32, _P, _I32, _P, _P, _P, _P, _SZ, _U32,
                                         _P]),
    "gale_route_workspace_bytes": (_SZ, [_I32, _I32]),
    "gale_route_topk": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "gale_decode_stack_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "gale_moe_decode_stack": (_I32, [_I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _U32, _P]),
    "gale_moe_decode_stack_static": (_I32, [_I32, _I32, _I32, _I32, _I32, _P, _U32, _P]),
    "gale_sync_init": (_I32, [_P, _P]),
    "gale_read_stream": (_I32, [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P]),
    "gale_sync_status": (_I32, [_P, ctypes.POINTER(ctypes.c_uint64)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgale.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgale.so not found at {LIB_PATH}; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols() -> List[str]:
    return list(_SIGS)


def _check(fn: str, status: int) -> None:
    if status != GALE_OK:
        raise GaleError(fn, status, lib().gale_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _require_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libgale compute calls take device (cuda) tensors")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return GALE_F16
    if t.dtype == torch.float32:
        return GALE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _tdt(code: int) -> torch.dtype:
    return torch.float16 if code == GALE_F16 else torch.float32


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator hands out 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def moe_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace for gale_moe_layer_fwd / gale_moe_decode_stack whose synchronisation words
    (its first GALE_SYNC_BYTES) are zeroed, as the one-launch decode needs before its first call."""
    ws = _workspace(max(int(nbytes), GALE_SYNC_BYTES), device)
    sync_init(ws)
    return ws


# ----------------------------------------------------------------------------
# format
# ----------------------------------------------------------------------------
def packed_sizes(rows: int, cols: int, nnz: int) -> dict:
    s = gale_sizes()
    _check("gale_packed_sizes", lib().gale_packed_sizes(rows, cols, nnz, ctypes.byref(s)))
    return {n: getattr(s, n) for n, _ in gale_sizes._fields_}


def check_canonical(rows: int, cols: int, row_ptr, out_cols) -> None:
    """Validate canonical CSR arrays (host numpy/torch CPU)."""
    rp = torch.as_tensor(row_ptr, dtype=torch.int32).contiguous()
    oc = torch.as_tensor(out_cols).view(torch.int16).contiguous() if torch.is_tensor(out_cols) else \
        torch.from_numpy(out_cols.view("int16")).contiguous()
    _check("gale_check_canonical", lib().gale_check_canonical(rows, cols, rp.data_ptr(),
                                                               oc.data_ptr() if oc.numel() else None, oc.numel()))


def pack_host(rows: int, cols: int, signs: torch.Tensor, scales: torch.Tensor):
    """Canonical -> device layout on the host (CPU tensors int32 [N, K/32], int16 [N, K/128])."""
    s = signs.contiguous()
    sc = scales.contiguous()
    ds = torch.empty_like(s)
    dsc = torch.empty_like(sc)
    _check("gale_pack_host", lib().gale_pack_host(rows, cols, s.data_ptr(), sc.data_ptr(), ds.data_ptr(), dsc.data_ptr()))
    return ds, dsc


def unpack_host(rows: int, cols: int, dev_signs: torch.Tensor, dev_scales: torch.Tensor):
    cs = torch.empty_like(dev_signs)
    csc = torch.empty_like(dev_scales)
    _check("gale_unpack_host", lib().gale_unpack_host(rows, cols, dev_signs.data_ptr(), dev_scales.data_ptr(),
                                                       cs.data_ptr(), csc.data_ptr()))
    return cs, csc


@dataclass
class PackedMatrix:
    """One matrix in the device layout (all tensors on one GPU).

    out_cols / out_vals are the section buffers, which may extend past the nnz
    entries (whole 16-byte chunks, at least one): the kernels read them in chunks."""
    rows: int
    cols: int
    signs: torch.Tensor
    block_scales: torch.Tensor
    row_scales: torch.Tensor
    row_ptr: torch.Tensor
    out_cols: torch.Tensor
    out_vals: torch.Tensor
    nnz: int = -1

    def __post_init__(self):
        if self.nnz < 0:
            self.nnz = int(self.out_cols.numel())

    def descriptor(self) -> gale_matrix:
        d = gale_matrix()
        d.signs, d.block_scales, d.row_scales = _ptr(self.signs), _ptr(self.block_scales), _ptr(self.row_scales)
        d.row_ptr, d.out_cols, d.out_vals = _ptr(self.row_ptr), _ptr(self.out_cols), _ptr(self.out_vals)
        for name, _ in gale_matrix._fields_:
            if not getattr(d, name):
                raise ValueError(f"PackedMatrix section {name} has no storage (NULL pointer); every section, "
                                 "outliers included, needs a readable buffer")
        return d


def pack_device(rows: int, cols: int, n_mat: int, canon_signs: torch.Tensor, canon_scales: torch.Tensor,
                out_signs: Optional[torch.Tensor] = None, out_scales: Optional[torch.Tensor] = None):
    """n_mat canonical matrices stored back to back (device) -> device layout."""
    _require_cuda(canon_signs, canon_scales)
    if out_signs is None:
        out_signs = torch.empty(n_mat * rows * cols // 32, dtype=torch.int32, device=canon_signs.device)
    if out_scales is None:
        out_scales = torch.empty(n_mat * rows * cols // 128, dtype=torch.int16, device=canon_signs.device)
    _check("gale_pack_device", lib().gale_pack_device(rows, cols, n_mat, canon_signs.data_ptr(), canon_scales.data_ptr(),
                                                       out_signs.data_ptr(), out_scales.data_ptr(), _stream()))
    return out_signs, out_scales


def _padded16(t: torch.Tensor) -> torch.Tensor:
    """Copy a 1-D section into a fresh buffer padded to whole 16-byte chunks (at least one)."""
    nbytes = t.numel() * t.element_size()
    n = max(16, (nbytes + 15) // 16 * 16)
    out = torch.zeros(n, dtype=torch.uint8, device=t.device)
    if nbytes:
        out[:nbytes] = t.reshape(-1).contiguous().view(torch.uint8)
    return out


def pack_matrix(cm) -> PackedMatrix:
    """synth.CanonicalMatrix (on a GPU) -> PackedMatrix.  Signs and block scales are re-laid out;
    outliers and row scales keep the canonical format (outlier sections padded to 16 bytes)."""
    ds, dsc = pack_device(cm.rows, cm.cols, 1, cm.signs, cm.block_scales)
    # the padded buffers themselves (an empty slice would have a NULL data pointer)
    return PackedMatrix(cm.rows, cm.cols, ds, dsc, cm.row_scales, cm.row_ptr.contiguous(),
                        _padded16(cm.out_cols).view(torch.int16), _padded16(cm.out_vals), nnz=cm.nnz)


class DescriptorTable:
    """A device array of gale_matrix or gale_expert descriptors, keeping the matrices alive."""

    def __init__(self, structs: Sequence[ctypes.Structure], keep: Sequence, device, outliers_per_row: float = 0.0):
        self.outliers_per_row = outliers_per_row   # mean outliers per row of the densest matrix
        n = len(structs)
        size = ctypes.sizeof(structs[0]) if n else 8
        raw = (ctypes.c_uint8 * (size * max(n, 1)))()
        for i, s in enumerate(structs):
            ctypes.memmove(ctypes.addressof(raw) + i * size, ctypes.addressof(s), size)
        host = torch.frombuffer(bytearray(raw), dtype=torch.uint8)
        self.tensor = host.to(device)
        self.count = n
        self.keep = list(keep)

    def ptr(self) -> int:
        return self.tensor.data_ptr()


def matrix_table(mats: Sequence[PackedMatrix], device=None) -> DescriptorTable:
    device = device or mats[0].signs.device
    return DescriptorTable([m.descriptor() for m in mats], mats, device,
                           max((m.nnz / m.rows for m in mats), default=0.0))


def expert_table(experts: Sequence[Sequence[PackedMatrix]], device=None) -> DescriptorTable:
    device = device or experts[0][0].signs.device
    structs = []
    for w1, w3, w2 in experts:
        e = gale_expert()
        e.w1, e.w3, e.w2 = w1.descriptor(), w3.descriptor(), w2.descriptor()
        structs.append(e)
    return DescriptorTable(structs, experts, device,
                           max((m.nnz / m.rows for ex in experts for m in ex), default=0.0))


# ----------------------------------------------------------------------------
# debug exports
# ----------------------------------------------------------------------------
def debug_unpack_signs(pm: PackedMatrix) -> torch.Tensor:
    out = torch.empty(pm.rows, pm.cols // 32, dtype=torch.int32, device=pm.signs.device)
    _check("gale_debug_unpack_signs", lib().gale_debug_unpack_signs(pm.rows, pm.cols, pm.signs.data_ptr(),
                                                                     out.data_ptr(), _stream()))
    return out


def debug_unpack_outliers(pm: PackedMatrix):
    n = pm.nnz
    dev = pm.signs.device
    r = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    c = torch.empty_like(r)
    v = torch.empty_like(r)
    d = pm.descriptor()
    _check("gale_debug_unpack_outliers", lib().gale_debug_unpack_outliers(pm.rows, n, ctypes.byref(d), r.data_ptr(),
                                                                           c.data_ptr(), v.data_ptr(), _stream()))
    return r[:n], c[:n], v[:n]


# ----------------------------------------------------------------------------
# compute
# ----------------------------------------------------------------------------
def fwht1024(x: torch.Tensor, out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None):
    _require_cuda(x)
    x = x.contiguous()
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    L = x.shape[-1]
    nv = x.numel() // L
    _check("gale_fwht1024", lib().gale_fwht1024(x.data_ptr(), out.data_ptr(), nv, L, _dt(x), _dt(out), _stream()))
    return out


def prepared_bytes(length: int) -> int:
    return int(lib().gale_prepared_bytes(length))


def prepare_activations(x: torch.Tensor, rotated: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [..., len] -> uint8 [n_vec, prepared_bytes(len)] records for GALE_X_PREPARED GEMVs."""
    _require_cuda(x)
    x = x.contiguous()
    L = x.shape[-1]
    nv = x.numel() // L
    rb = prepared_bytes(L)
    if out is None:
        out = torch.empty(nv, rb, dtype=torch.uint8, device=x.device)
    _check("gale_prepare_activations", lib().gale_prepare_activations(
        x.data_ptr(), _dt(x), nv, L, GALE_X_ROTATED if rotated else 0, out.data_ptr(), out.numel(), _stream()))
    return out


def gemv_workspace_bytes(rows, cols, n_mat, n_tok, x_shared) -> int:
    return int(lib().gale_gemv_workspace_bytes(rows, cols, n_mat, n_tok, int(bool(x_shared))))


def expert_gemv(table: DescriptorTable, rows: int, cols: int, x: torch.Tensor, n_mat: Optional[int] = None,
                x_shared: bool = False, y_dtype=torch.float16, flags: int = 0, y: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[m, t] = Wq_m . H x[m, t]; x [n_mat, n_tok, cols] (or [n_tok, cols] with x_shared)."""
    _require_cuda(x)
    n_mat = n_mat or table.count
    prepared = bool(flags & GALE_X_PREPARED)
    if prepared:
        # x: uint8 records [n_x, prepared_bytes(cols)], n_x = (1 if x_shared else n_mat) * n_tok
        n_tok = x.shape[0] // (1 if x_shared else n_mat)
    else:
        n_tok = x.shape[-2]
    if y is None:
        y = torch.empty(n_mat, n_tok, rows, dtype=y_dtype, device=x.device)
    if ws is None and not prepared:
        ws = _workspace(gemv_workspace_bytes(rows, cols, n_mat, n_tok, x_shared), x.device)
    flags = _with_stage(flags, table)
    _check("gale_expert_gemv", lib().gale_expert_gemv(rows, cols, table.ptr(), n_mat, x.data_ptr(),
                                                       GALE_F16 if prepared else _dt(x), int(bool(x_shared)), n_tok,
                                                       y.data_ptr(), _dt(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                                       flags, _stream()))
    return y


def ffn_workspace_bytes(hidden, inter, n_exp, n_tok, x_shared) -> int:
    return int(lib().gale_ffn_workspace_bytes(hidden, inter, n_exp, n_tok, int(bool(x_shared))))


def expert_ffn(table: DescriptorTable, hidden: int, inter: int, x: torch.Tensor, n_exp: Optional[int] = None,
               x_shared: bool = False, y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    _require_cuda(x)
    n_exp = n_exp or table.count
    n_tok = x.shape[-2]
    if y is None:
        y = torch.empty(n_exp, n_tok, hidden, dtype=torch.float16, device=x.device)
    if ws is None:
        ws = _workspace(ffn_workspace_bytes(hidden, inter, n_exp, n_tok, x_shared), x.device)
    _check("gale_expert_ffn", lib().gale_expert_ffn(hidden, inter, table.ptr(), n_exp, x.data_ptr(),
                                                     int(bool(x_shared)), n_tok, y.data_ptr(), ws.data_ptr(),
                                                     ws.numel(), _stream()))
    return y


def moe_workspace_bytes(n_tok, n_experts, top_k, hidden, inter, flags=0) -> int:
    return int(lib().gale_moe_workspace_bytes(n_tok, n_experts, top_k, hidden, inter, flags))


def moe_layer_fwd(table: DescriptorTable, hidden: int, inter: int, logits: torch.Tensor, x: torch.Tensor,
                  top_k: int = 6, flags: int = 0, y: Optional[torch.Tensor] = None,
                  topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, select_bias: Optional[torch.Tensor] = None,
                  fixed_idx: Optional[torch.Tensor] = None):
    """One routed-expert layer; select_bias (fp32 [E]) or fixed_idx (int32 [T, top_k]) select the
    routing variants of gale_moe_layer_fwd_routed."""
    _require_cuda(x, logits)
    n_tok = x.shape[0]
    E = logits.shape[1]
    if y is None:
        y = torch.empty(n_tok, hidden, dtype=torch.float16, device=x.device)
    if topk_idx is None:
        topk_idx = torch.empty(n_tok, top_k, dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty(n_tok, top_k, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = moe_workspace(moe_workspace_bytes(n_tok, E, top_k, hidden, inter, flags), x.device)
    flags = _with_stage(flags, table)
    if select_bias is None and fixed_idx is None:
        _check("gale_moe_layer_fwd", lib().gale_moe_layer_fwd(hidden, inter, table.ptr(), E, logits.data_ptr(), top_k,
                                                               x.data_ptr(), n_tok, y.data_ptr(), topk_idx.data_ptr(),
                                                               topk_w.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                                                               _stream()))
        return y, topk_idx, topk_w
    if select_bias is not None:
        _require_cuda(select_bias)
        if select_bias.dtype != torch.float32 or select_bias.numel() != E or not select_bias.is_contiguous():
            raise ValueError("select_bias must be a contiguous fp32 tensor of n_experts entries")
    if fixed_idx is not None:
        _require_cuda(fixed_idx)
        if fixed_idx.dtype != torch.int32 or tuple(fixed_idx.shape) != (n_tok, top_k) or not fixed_idx.is_contiguous():
            raise ValueError("fixed_idx must be a contiguous int32 tensor [n_tok, top_k]")
    _check("gale_moe_layer_fwd_routed", lib().gale_moe_layer_fwd_routed(
        hidden, inter, table.ptr(), E, logits.data_ptr(), None if select_bias is None else select_bias.data_ptr(),
        None if fixed_idx is None else fixed_idx.data_ptr(), top_k, x.data_ptr(), n_tok, y.data_ptr(),
        topk_idx.data_ptr(), topk_w.data_ptr(), ws.data_ptr(), ws.numel(), flags, _stream()))
    return y, topk_idx, topk_w


def route_topk(logits: torch.Tensor, top_k: int, group: bool = False):
    _require_cuda(logits)
    T, E = logits.shape
    dev = logits.device
    idx = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    offsets = perm = ws = None
    if group:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(T * top_k, dtype=torch.int32, device=dev)
        ws = _workspace(lib().gale_route_workspace_bytes(T, E), dev)
    _check("gale_route_topk", lib().gale_route_topk(logits.contiguous().data_ptr(), T, E, top_k, idx.data_ptr(),
                                                     w.data_ptr(), _ptr(offsets), _ptr(perm), _ptr(ws),
                                                     0 if ws is None else ws.numel(), _stream()))
    return (idx, w, offsets, perm) if group else (idx, w)


# ----------------------------------------------------------------------------
# one token through a stack of layers; synchronisation words
# ----------------------------------------------------------------------------
def sync_init(ws: torch.Tensor) -> None:
    """Zero the synchronisation words at the start of ws (a kernel on the current stream)."""
    _require_cuda(ws)
    _check("gale_sync_init", lib().gale_sync_init(ws.data_ptr(), _stream()))


def sync_status(ws: torch.Tensor):
    """(status, (generation, check, error bits), detail) of the synchronisation words of ws.
    Blocking: call after the stream's work is done."""
    _require_cuda(ws)
    words = (ctypes.c_uint64 * 3)()
    st = lib().gale_sync_status(ws.data_ptr(), words)
    detail = lib().gale_last_error().decode() if st != GALE_OK else ""
    if st not in (GALE_OK, GALE_ERR_SYNC):
        raise GaleError("gale_sync_status", st, detail)
    return st, (words[0], words[1], words[2]), detail


def decode_stack_workspace_bytes(hidden: int, inter: int, top_k: int) -> int:
    return int(lib().gale_decode_stack_workspace_bytes(hidden, inter, top_k))


class LayerTable:
    """Device array of gale_layer_io records for gale_moe_decode_stack (keeps the tensors alive)."""

    def __init__(self, records: Sequence[dict], device):
        self.keep = records
        arr = (gale_layer_io * len(records))()
        for i, r in enumerate(records):
            arr[i] = gale_layer_io(*[_ptr(r.get(n)) for n, _ in gale_layer_io._fields_])
        host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
        self.dev = host.to(device)
        self.n = len(records)

    def ptr(self) -> int:
        return self.dev.data_ptr()


def layer_table(layers: Sequence[dict], device=None) -> LayerTable:
    """layers: per layer a dict of tensors with keys experts (DescriptorTable), logits, x, y and
    optionally select_bias, fixed_idx, topk_idx, topk_w."""
    recs = []
    for r in layers:
        d = dict(r)
        d["experts"] = r["experts"].tensor if isinstance(r["experts"], DescriptorTable) else r["experts"]
        recs.append(d)
    dev = device if device is not None else recs[0]["x"].device
    return LayerTable(recs, dev)


def moe_decode_stack(hidden: int, inter: int, n_experts: int, top_k: int, layers: LayerTable,
                     ws: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """One token through the layers of `layers` in one launch; returns the workspace used."""
    if ws is None:
        ws = moe_workspace(decode_stack_workspace_bytes(hidden, inter, top_k), layers.dev.device)
    _check("gale_moe_decode_stack", lib().gale_moe_decode_stack(hidden, inter, n_experts, top_k, layers.n,
                                                                 layers.ptr(), ws.data_ptr(), ws.numel(), flags,
                                                                 _stream()))
    return ws
