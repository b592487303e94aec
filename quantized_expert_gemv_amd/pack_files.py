"""GALE pack files and their manifest: expert matrices on disk, loaded into the device layout.

The GALE packs described on the "DeepSeek-V4-Flash - GALE 1-bit experts" model card
("Files") and the "DeepSeek-V4-Pro-671B-GALE-1bit-v4" page (the paragraph listing the
pack's files) keep one pack file per layer and a JSONL manifest with one record per
tensor: its kind, shape, sections, outlier count, pack file and byte offset.  Neither
page publishes the byte layout of a record's sections, so this module defines its own
(format "gale-pack", version 1), writes it, and loads it:

  manifest.jsonl   one JSON object per line.  An optional first record
                   {"kind": "format", "name": "gale-pack", "version": 1} names the
                   format.  A GALE matrix record:
                     {"kind": "gale", "name": "layers.L.experts.E.w1", "layer": L,
                      "expert": E, "proj": "w1" | "w3" | "w2", "shape": [rows, cols],
                      "outliers": nnz, "file": "layer_LLL.h0.pack", "offset": B,
                      "nbytes": n, "sections": {name: [offset within the record, nbytes]}}
                   A non-expert tensor (router weights, selection biases, ...):
                     {"kind": "dense", "name": ..., "dtype": "float16" | "float32" |
                      "int32" | ..., "shape": [...], "file": ..., "offset": B, "nbytes": n}
  layer_LLL.h0.pack   the GALE records of layer L, each starting on a 256-byte boundary.
  misc.pack           the dense records.

The sections of a GALE record are the canonical format of the model card's "What is in
the pack" section, little-endian, each starting on a 256-byte boundary of the record:
  signs         uint32 [rows, cols/32]   bit j of word w is column 32 w + j; 1 = negative
  block_scales  fp16   [rows, cols/128]  one scale per 128 consecutive columns of a row
  row_scales    fp16   [rows]            the scale of the row's int4 outliers
  row_ptr       int32  [rows + 1]        CSR offsets of each row's outliers (0 .. nnz)
  out_cols      uint16 [nnz]             outlier columns, ascending within a row
  out_vals      uint8  [ceil(nnz / 2)]   int4 outlier values, two's complement, entry 2i in
                                         the low nibble of byte i

Loading is input/output and argument marshalling: sections are gathered per layer on the
host into pinned banks, copied to the device, and laid out for the kernels by the
library's device packer (gale_pack_device); outliers and row scales keep the canonical
format.  Every record is validated on the host first (bounds within its file, section
sizes against shape and outlier count, the CSR arrays through gale_check_canonical), and
a bad pack raises ValueError naming the record.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Mapping, Optional, Sequence, Tuple

import numpy as np
import torch

from . import binding as _b

FORMAT_NAME = "gale-pack"
FORMAT_VERSION = 1
ALIGN = 256
MANIFEST = "manifest.jsonl"
PROJS = ("w1", "w3", "w2")

# canonical section: (numpy dtype, shape as a function of (rows, cols, nnz))
SECTIONS: Dict[str, Tuple[np.dtype, callable]] = {
    "signs": (np.dtype("<u4"), lambda n, k, z: (n, k // 32)),
    "block_scales": (np.dtype("<f2"), lambda n, k, z: (n, k // 128)),
    "row_scales": (np.dtype("<f2"), lambda n, k, z: (n,)),
    "row_ptr": (np.dtype("<i4"), lambda n, k, z: (n + 1,)),
    "out_cols": (np.dtype("<u2"), lambda n, k, z: (z,)),
    "out_vals": (np.dtype("u1"), lambda n, k, z: ((z + 1) // 2,)),
}
DENSE_DTYPES = {"float16": np.float16, "float32": np.float32, "bfloat16": None, "int32": np.int32,
                "int64": np.int64, "uint8": np.uint8, "int16": np.int16}


def _up(n: int, a: int = ALIGN) -> int:
    return (n + a - 1) // a * a


def layer_file(layer: int) -> str:
    return f"layer_{layer:03d}.h0.pack"


def matrix_name(layer: int, expert: int, proj: str) -> str:
    return f"layers.{layer}.experts.{expert}.{proj}"


def section_shape(name: str, rows: int, cols: int, nnz: int) -> Tuple[int, ...]:
    return SECTIONS[name][1](rows, cols, nnz)


def section_nbytes(name: str, rows: int, cols: int, nnz: int) -> int:
    return int(np.prod(section_shape(name, rows, cols, nnz), dtype=np.int64)) * SECTIONS[name][0].itemsize


def record_layout(rows: int, cols: int, nnz: int) -> Tuple[Dict[str, List[int]], int]:
    """Section offsets within a GALE record and the record's size (a multiple of 256)."""
    off, secs = 0, {}
    for name in SECTIONS:
        nb = section_nbytes(name, rows, cols, nnz)
        secs[name] = [off, nb]
        off = _up(off + max(nb, 1))
    return secs, off


# ----------------------------------------------------------------------------
# writer
# ----------------------------------------------------------------------------
class PackWriter:
    """Writes GALE matrices (canonical sections) and dense tensors into a pack directory.

    Use as a context manager, or call close(): the manifest is written at the end."""

    def __init__(self, directory: str):
        self.dir = directory
        os.makedirs(directory, exist_ok=True)
        self.records: List[dict] = [{"kind": "format", "name": FORMAT_NAME, "version": FORMAT_VERSION}]
        self._files: Dict[str, object] = {}
        self._names = set()

    def _file(self, fname: str):
        f = self._files.get(fname)
        if f is None:
            f = open(os.path.join(self.dir, fname), "wb")
            self._files[fname] = f
        return f

    def _append(self, fname: str, payload: bytes) -> int:
        f = self._file(fname)
        off = _up(f.tell())
        if off > f.tell():
            f.write(b"\0" * (off - f.tell()))
        f.write(payload)
        return off

    def _claim(self, name: str) -> None:
        if name in self._names:
            raise ValueError(f"duplicate tensor name {name!r}")
        self._names.add(name)

    def add_gale(self, layer: int, expert: int, proj: str, m: Mapping[str, np.ndarray]) -> dict:
        """m: canonical sections (keys of SECTIONS plus rows, cols), numpy arrays of any
        dtype with the right item size (they are written as their bytes)."""
        if proj not in PROJS:
            raise ValueError(f"proj must be one of {PROJS}, got {proj!r}")
        rows, cols = int(m["rows"]), int(m["cols"])
        nnz = int(np.asarray(m["out_cols"]).size)
        name = matrix_name(layer, expert, proj)
        self._claim(name)
        secs, size = record_layout(rows, cols, nnz)
        buf = bytearray(size)
        for s, (off, nb) in secs.items():
            a = np.ascontiguousarray(np.asarray(m[s]))
            if s == "row_ptr":
                a = a.astype("<i4")
            raw = a.tobytes()
            if len(raw) != nb:
                raise ValueError(f"{name}: section {s} holds {len(raw)} bytes, expected {nb}")
            buf[off:off + nb] = raw
        fname = layer_file(layer)
        off = self._append(fname, bytes(buf))
        rec = {"kind": "gale", "name": name, "layer": int(layer), "expert": int(expert), "proj": proj,
               "shape": [rows, cols], "outliers": nnz, "file": fname, "offset": off, "nbytes": size,
               "sections": secs}
        self.records.append(rec)
        return rec

    def add_dense(self, name: str, a: np.ndarray, dtype: Optional[str] = None, fname: str = "misc.pack") -> dict:
        self._claim(name)
        a = np.ascontiguousarray(a)
        dt = dtype or str(a.dtype)
        if dt not in DENSE_DTYPES:
            raise ValueError(f"{name}: dense dtype {dt!r} not supported")
        raw = a.tobytes()
        off = self._append(fname, raw)
        rec = {"kind": "dense", "name": name, "dtype": dt, "shape": list(a.shape), "file": fname,
               "offset": off, "nbytes": len(raw)}
        self.records.append(rec)
        return rec

    def close(self) -> None:
        for f in self._files.values():
            f.close()
        self._files = {}
        with open(os.path.join(self.dir, MANIFEST), "w") as f:
            for r in self.records:
                f.write(json.dumps(r, separators=(",", ":")) + "\n")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if exc[0] is None:
            self.close()
        else:
            for f in self._files.values():
                f.close()


# ----------------------------------------------------------------------------
# manifest and host reads
# ----------------------------------------------------------------------------
def _need(rec: dict, key: str, typ, where: str):
    if key not in rec:
        raise ValueError(f"{where}: missing field {key!r}")
    v = rec[key]
    if not isinstance(v, typ) or isinstance(v, bool):
        raise ValueError(f"{where}: field {key!r} has type {type(v).__name__}")
    return v


def read_manifest(directory: str) -> List[dict]:
    """Parse and check the manifest's records (not the pack files)."""
    path = os.path.join(directory, MANIFEST)
    out = []
    with open(path) as f:
        for i, line in enumerate(f, 1):
            if not line.strip():
                continue
            where = f"{MANIFEST} line {i}"
            try:
                rec = json.loads(line)
            except json.JSONDecodeError as e:
                raise ValueError(f"{where}: not JSON ({e})") from None
            if not isinstance(rec, dict):
                raise ValueError(f"{where}: not an object")
            kind = _need(rec, "kind", str, where)
            if kind == "format":
                if rec.get("name") != FORMAT_NAME or rec.get("version") != FORMAT_VERSION:
                    raise ValueError(f"{where}: format {rec.get('name')!r} version {rec.get('version')!r}, "
                                     f"this loader reads {FORMAT_NAME!r} version {FORMAT_VERSION}")
                continue
            name = _need(rec, "name", str, where)
            where = f"{where} ({name})"
            _need(rec, "file", str, where)
            if os.path.isabs(rec["file"]) or os.path.normpath(rec["file"]).startswith(".."):
                raise ValueError(f"{where}: pack file must be a path inside the pack directory")
            if _need(rec, "offset", int, where) < 0 or _need(rec, "nbytes", int, where) < 0:
                raise ValueError(f"{where}: negative offset or size")
            shape = _need(rec, "shape", list, where)
            if not all(isinstance(d, int) and not isinstance(d, bool) and d >= 0 for d in shape):
                raise ValueError(f"{where}: bad shape {shape}")
            if kind == "gale":
                _check_gale_record(rec, where)
            elif kind == "dense":
                dt = _need(rec, "dtype", str, where)
                if dt not in DENSE_DTYPES:
                    raise ValueError(f"{where}: dense dtype {dt!r} not supported")
                isz = 2 if dt == "bfloat16" else np.dtype(DENSE_DTYPES[dt]).itemsize
                if int(np.prod(shape, dtype=np.int64)) * isz != rec["nbytes"]:
                    raise ValueError(f"{where}: {rec['nbytes']} bytes for shape {shape} of {dt}")
            else:
                raise ValueError(f"{where}: unknown kind {kind!r}")
            out.append(rec)
    names = [r["name"] for r in out]
    if len(set(names)) != len(names):
        raise ValueError(f"{MANIFEST}: duplicate tensor names")
    return out


def _check_gale_record(rec: dict, where: str) -> None:
    if len(rec["shape"]) != 2:
        raise ValueError(f"{where}: a GALE matrix has a 2-d shape")
    rows, cols = rec["shape"]
    if rows < 1 or cols < 1024 or cols % 1024:
        raise ValueError(f"{where}: shape {rec['shape']} (columns must be a positive multiple of 1024)")
    for key in ("layer", "expert", "outliers"):
        if _need(rec, key, int, where) < 0:
            raise ValueError(f"{where}: negative {key}")
    if _need(rec, "proj", str, where) not in PROJS:
        raise ValueError(f"{where}: proj {rec['proj']!r}")
    secs = _need(rec, "sections", dict, where)
    nnz = rec["outliers"]
    for s in SECTIONS:
        if s not in secs:
            raise ValueError(f"{where}: missing section {s!r}")
        v = secs[s]
        if (not isinstance(v, list) or len(v) != 2 or
                not all(isinstance(t, int) and not isinstance(t, bool) and t >= 0 for t in v)):
            raise ValueError(f"{where}: section {s} must be [offset, nbytes]")
        off, nb = v
        want = section_nbytes(s, rows, cols, nnz)
        if nb != want:
            raise ValueError(f"{where}: section {s} has {nb} bytes, shape and outlier count give {want}")
        if off + nb > rec["nbytes"]:
            raise ValueError(f"{where}: section {s} ends past the record")
        if (rec["offset"] + off) % SECTIONS[s][0].itemsize:
            raise ValueError(f"{where}: section {s} is not aligned to its element size")


class Pack:
    """A pack directory: its manifest, indexed, and memory-mapped reads of its files."""

    def __init__(self, directory: str):
        self.dir = directory
        self.records = read_manifest(directory)
        self.by_name = {r["name"]: r for r in self.records}
        self._maps: Dict[str, np.memmap] = {}
        self.gale: Dict[int, Dict[Tuple[int, str], dict]] = {}
        for r in self.records:
            if r["kind"] == "gale":
                key = (r["expert"], r["proj"])
                lay = self.gale.setdefault(r["layer"], {})
                if key in lay:
                    raise ValueError(f"{MANIFEST}: layer {r['layer']} lists expert {key[0]} {key[1]} twice")
                lay[key] = r
        for r in self.records:
            self._bytes(r)   # bounds of every record against its file

    def _map(self, fname: str) -> np.memmap:
        m = self._maps.get(fname)
        if m is None:
            path = os.path.join(self.dir, fname)
            if not os.path.isfile(path):
                raise ValueError(f"pack file {fname!r} is missing")
            if os.path.getsize(path) == 0:
                m = np.zeros(0, dtype=np.uint8)
            else:
                m = np.memmap(path, dtype=np.uint8, mode="r")
            self._maps[fname] = m
        return m

    def _bytes(self, rec: dict) -> np.ndarray:
        m = self._map(rec["file"])
        end = rec["offset"] + rec["nbytes"]
        if end > m.size:
            raise ValueError(f"{rec['name']}: record [{rec['offset']}, {end}) runs past the end of "
                             f"{rec['file']} ({m.size} bytes)")
        return m[rec["offset"]:end]

    def layers(self) -> List[int]:
        return sorted(self.gale)

    def layer_geometry(self, layer: int) -> Tuple[int, int, int]:
        """(experts, hidden, inter) of a layer; every expert needs w1, w3 [inter, hidden] and
        w2 [hidden, inter]."""
        lay = self.gale.get(layer)
        if not lay:
            raise ValueError(f"no GALE records for layer {layer}")
        experts = sorted({e for e, _ in lay})
        if experts != list(range(len(experts))):
            raise ValueError(f"layer {layer}: experts are not numbered 0..{len(experts) - 1}")
        w1 = lay.get((0, "w1"))
        if w1 is None:
            raise ValueError(f"layer {layer}: expert 0 has no w1")
        inter, hidden = w1["shape"]
        want = {"w1": [inter, hidden], "w3": [inter, hidden], "w2": [hidden, inter]}
        for e in experts:
            for p in PROJS:
                r = lay.get((e, p))
                if r is None:
                    raise ValueError(f"layer {layer}: expert {e} has no {p}")
                if r["shape"] != want[p]:
                    raise ValueError(f"{r['name']}: shape {r['shape']}, the layer needs {want[p]}")
        return len(experts), hidden, inter

    def read_gale(self, rec_or_name, check: bool = True) -> Dict[str, np.ndarray]:
        """One GALE matrix as canonical numpy sections (the arrays view the mapped file)."""
        rec = self.by_name[rec_or_name] if isinstance(rec_or_name, str) else rec_or_name
        raw = self._bytes(rec)
        rows, cols = rec["shape"]
        nnz = rec["outliers"]
        out: Dict[str, np.ndarray] = {"rows": rows, "cols": cols}
        for s, (dt, shp) in SECTIONS.items():
            off, nb = rec["sections"][s]
            out[s] = raw[off:off + nb].view(dt).reshape(shp(rows, cols, nnz))
        if check:
            if out["row_ptr"][-1] != nnz:
                raise ValueError(f"{rec['name']}: row_ptr ends at {int(out['row_ptr'][-1])}, outliers = {nnz}")
            try:
                _b.check_canonical(rows, cols, np.array(out["row_ptr"]), np.array(out["out_cols"]))
            except _b.GaleError as e:
                raise ValueError(f"{rec['name']}: {e}") from None
        return out

    def read_dense(self, name: str) -> np.ndarray:
        rec = self.by_name[name]
        if rec["kind"] != "dense":
            raise ValueError(f"{name} is a {rec['kind']} record")
        raw = self._bytes(rec)
        if rec["dtype"] == "bfloat16":
            return raw.view(np.uint16).reshape(rec["shape"])
        return raw.view(DENSE_DTYPES[rec["dtype"]]).reshape(rec["shape"])


# ----------------------------------------------------------------------------
# device load
# ----------------------------------------------------------------------------
@dataclass
class LoadedStack:
    """The GALE experts of a pack, resident on one GPU in the kernels' layout."""
    hidden: int
    inter: int
    experts: int
    layer_ids: List[int]
    tables: List[_b.DescriptorTable]            # per layer: expert descriptors (w1, w3, w2)
    matrices: List[List[Tuple[_b.PackedMatrix, ...]]]
    dense: Dict[str, torch.Tensor] = field(default_factory=dict)
    keep: List[torch.Tensor] = field(default_factory=list)


def _pinned(nbytes: int) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, pin_memory=True)


def load_stack(directory: str, device, layers: Optional[Sequence[int]] = None,
               dense: bool = True) -> LoadedStack:
    """Load the GALE experts of `layers` (default: every layer in the pack) onto `device`.

    Per layer: the w1/w3 and the w2 signs and block scales are gathered on the host into
    two pinned banks each, copied to the device and laid out by gale_pack_device (one call
    per bank); row scales, CSR offsets and outlier sections go in one pinned buffer, each
    on a 256-byte boundary and padded to whole 16-byte chunks (the kernels read outliers
    in 16-byte chunks), and are copied as they are.  Dense records are copied to the
    device as tensors of their dtype when `dense` is set."""
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError("load_stack places the experts on a GPU (device must be cuda)")
    pack = Pack(directory)
    ids = list(layers) if layers is not None else pack.layers()
    if not ids:
        raise ValueError("the pack has no GALE layers")
    geo = {l: pack.layer_geometry(l) for l in ids}
    E, H, I = geo[ids[0]]
    for l in ids:
        if geo[l] != (E, H, I):
            raise ValueError(f"layer {l}: {geo[l]} (experts, hidden, inter) differs from layer {ids[0]}'s "
                             f"{(E, H, I)}")
    nw13, ns13 = I * H // 32, I * H // 128       # words and scales per w1/w3 matrix
    nw2, ns2 = H * I // 32, H * I // 128
    # host staging reused across layers
    hs13 = _pinned(2 * E * nw13 * 4).view(torch.int32)
    hc13 = _pinned(2 * E * ns13 * 2).view(torch.int16)
    hs2 = _pinned(E * nw2 * 4).view(torch.int32)
    hc2 = _pinned(E * ns2 * 2).view(torch.int16)
    dcs13 = torch.empty(2 * E * nw13, dtype=torch.int32, device=dev)
    dcc13 = torch.empty(2 * E * ns13, dtype=torch.int16, device=dev)
    dcs2 = torch.empty(E * nw2, dtype=torch.int32, device=dev)
    dcc2 = torch.empty(E * ns2, dtype=torch.int16, device=dev)
    tables, mats, keep = [], [], []
    for l in ids:
        lay = pack.gale[l]
        reads = {(e, p): pack.read_gale(lay[(e, p)]) for e in range(E) for p in PROJS}
        n_s13 = hs13.numpy().reshape(2 * E, nw13)
        n_c13 = hc13.numpy().reshape(2 * E, ns13)
        n_s2 = hs2.numpy().reshape(E, nw2)
        n_c2 = hc2.numpy().reshape(E, ns2)
        for e in range(E):
            for j, p in enumerate(("w1", "w3")):
                m = reads[(e, p)]
                n_s13[2 * e + j] = m["signs"].reshape(-1).view(np.int32)
                n_c13[2 * e + j] = m["block_scales"].reshape(-1).view(np.int16)
            m = reads[(e, "w2")]
            n_s2[e] = m["signs"].reshape(-1).view(np.int32)
            n_c2[e] = m["block_scales"].reshape(-1).view(np.int16)
        # row scales, CSR offsets and outliers: one buffer, 256-byte aligned pieces
        layout, total = {}, 0
        for key, m in reads.items():
            for s in ("row_scales", "row_ptr", "out_cols", "out_vals"):
                nb = m[s].nbytes
                layout[(key, s)] = (total, nb)
                total = _up(total + max(16, (nb + 15) // 16 * 16))
        hmisc = _pinned(total)
        nm = hmisc.numpy()
        nm[:] = 0
        for (key, s), (off, nb) in layout.items():
            if nb:
                nm[off:off + nb] = reads[key][s].reshape(-1).view(np.uint8)
        dcs13.copy_(hs13, non_blocking=True)
        dcc13.copy_(hc13, non_blocking=True)
        dcs2.copy_(hs2, non_blocking=True)
        dcc2.copy_(hc2, non_blocking=True)
        dmisc = hmisc.to(dev, non_blocking=True)
        s13, c13 = _b.pack_device(I, H, 2 * E, dcs13, dcc13)
        s2, c2 = _b.pack_device(H, I, E, dcs2, dcc2)
        s13 = s13.view(2 * E, nw13)
        c13 = c13.view(2 * E, ns13)
        s2 = s2.view(E, nw2)
        c2 = c2.view(E, ns2)

        def piece(key, s, dtype):
            off, nb = layout[(key, s)]
            n = max(16, (nb + 15) // 16 * 16)
            return dmisc[off:off + n].view(dtype)

        experts = []
        for e in range(E):
            trio = []
            for j, p in enumerate(PROJS):
                if p == "w2":
                    sg, sc, rows, cols = s2[e], c2[e], H, I
                else:
                    sg, sc, rows, cols = s13[2 * e + j], c13[2 * e + j], I, H
                key = (e, p)
                trio.append(_b.PackedMatrix(
                    rows, cols, sg, sc,
                    piece(key, "row_scales", torch.int16)[:rows],
                    piece(key, "row_ptr", torch.int32)[:rows + 1],
                    piece(key, "out_cols", torch.int16),
                    piece(key, "out_vals", torch.uint8),
                    nnz=lay[key]["outliers"]))
            experts.append(tuple(trio))
        # the host banks are reused by the next layer: wait for this layer's copies
        torch.cuda.current_stream(dev).synchronize()
        tables.append(_b.expert_table(experts, dev))
        mats.append(experts)
        keep += [s13, c13, s2, c2, dmisc]
    dense_t = {}
    if dense:
        for r in pack.records:
            if r["kind"] == "dense":
                a = np.array(pack.read_dense(r["name"]))
                if r["dtype"] == "bfloat16":
                    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
                else:
                    t = torch.from_numpy(a)
                dense_t[r["name"]] = t.to(dev)
    return LoadedStack(H, I, E, ids, tables, mats, dense_t, keep)


def gale_record_count(layers: int, experts: int) -> int:
    """GALE records of a stack: three matrices (w1, w3, w2) per routed expert per layer."""
    return layers * experts * len(PROJS)
