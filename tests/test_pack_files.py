"""Pack files and manifest (host side, no GPU): what the writer stores, the loader's reads
give back bit for bit, and every malformed pack is refused with ValueError.

The record fields follow the "DeepSeek-V4-Flash - GALE 1-bit experts" card ("Files": kind,
shape, sections, outlier count, pack file, byte offset).  The section byte layout is this
library's own (the pages do not publish one), so nothing here is pinned to the real pack.
"""
import json
import os

import numpy as np
import pytest

from quantized_expert_gemv_amd import pack_files as PF
from synth import gen_matrices

HIDDEN, INTER, EXPERTS, LAYERS = 2048, 1024, 3, 2


def _stack(seed=7, frac=0.01):
    """canonical numpy sections of a small stack: [layer][expert] = (w1, w3, w2)."""
    out = []
    for l in range(LAYERS):
        w13 = gen_matrices(seed, [(l, e, m) for e in range(EXPERTS) for m in (0, 1)], INTER, HIDDEN,
                           outlier_frac=frac)
        w2 = gen_matrices(seed, [(l, e, 2) for e in range(EXPERTS)], HIDDEN, INTER, outlier_frac=frac)
        out.append([(w13[2 * e].numpy(), w13[2 * e + 1].numpy(), w2[e].numpy()) for e in range(EXPERTS)])
    return out


def _write(d, stack, dense=True):
    with PF.PackWriter(str(d)) as w:
        for l, layer in enumerate(stack):
            for e, trio in enumerate(layer):
                for p, m in zip(PF.PROJS, trio):
                    w.add_gale(l, e, p, m)
        if dense:
            w.add_dense("layers.0.gate.bias", np.linspace(-1, 1, EXPERTS).astype(np.float32))
            w.add_dense("layers.0.gate.weight", np.arange(EXPERTS * 8, dtype=np.float16).reshape(EXPERTS, 8))
            w.add_dense("layers.0.hash_table", np.arange(12, dtype=np.int32).reshape(4, 3))
    return str(d)


@pytest.fixture(scope="module")
def stack():
    return _stack()


@pytest.fixture()
def packdir(tmp_path, stack):
    return _write(tmp_path / "pack", stack)


def test_round_trip_bit_exact(packdir, stack):
    pk = PF.Pack(packdir)
    assert pk.layers() == list(range(LAYERS))
    assert pk.layer_geometry(0) == (EXPERTS, HIDDEN, INTER)
    for l in range(LAYERS):
        for e in range(EXPERTS):
            for p, m in zip(PF.PROJS, stack[l][e]):
                got = pk.read_gale(PF.matrix_name(l, e, p))
                assert got["rows"] == m["rows"] and got["cols"] == m["cols"]
                for s in PF.SECTIONS:
                    a = np.ascontiguousarray(got[s]).view(np.uint8)
                    b = np.ascontiguousarray(np.asarray(m[s], dtype=got[s].dtype)).view(np.uint8)
                    assert a.tobytes() == b.tobytes(), (l, e, p, s)
    np.testing.assert_array_equal(pk.read_dense("layers.0.gate.bias"), np.linspace(-1, 1, EXPERTS).astype(np.float32))
    assert pk.read_dense("layers.0.gate.weight").dtype == np.float16
    assert pk.read_dense("layers.0.hash_table").shape == (4, 3)


def test_manifest_fields(packdir, stack):
    recs = PF.read_manifest(packdir)
    gale = [r for r in recs if r["kind"] == "gale"]
    assert len(gale) == PF.gale_record_count(LAYERS, EXPERTS)
    # the card's full stack: 43 layers x 256 experts x 3 matrices = 33,024 expert records
    assert PF.gale_record_count(43, 256) == 33024
    for r in gale:
        assert r["file"] == PF.layer_file(r["layer"])
        assert r["offset"] % PF.ALIGN == 0
        m = stack[r["layer"]][r["expert"]][PF.PROJS.index(r["proj"])]
        assert r["outliers"] == m["out_cols"].size
        assert r["shape"] == [m["rows"], m["cols"]]
        for s, (off, nb) in r["sections"].items():
            assert off % PF.ALIGN == 0 and off + nb <= r["nbytes"]
    # records of one file do not overlap
    for f in {r["file"] for r in gale}:
        spans = sorted((r["offset"], r["offset"] + r["nbytes"]) for r in gale if r["file"] == f)
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert spans[-1][1] == os.path.getsize(os.path.join(packdir, f))


def test_bits_per_weight_of_a_record():
    # [2048, 4096] at 1 % outliers (41 per row): 1 sign bit + 16/128 scale bits + 41 x (16 + 4)
    # bits of outliers per 4096 weights + a row scale and a CSR offset per row
    secs, size = PF.record_layout(2048, 4096, 2048 * 41)
    payload = sum(nb for _, nb in secs.values())
    bpw = payload * 8 / (2048 * 4096)
    want = 1 + 16 / 128 + 41 * 20 / 4096 + (16 + 32) / 4096 + 32 / (2048 * 4096)
    assert abs(bpw - want) < 1e-9
    assert size - payload < 6 * PF.ALIGN


def _rewrite_manifest(d, fn):
    path = os.path.join(d, PF.MANIFEST)
    recs = [json.loads(l) for l in open(path)]
    recs = fn(recs)
    with open(path, "w") as f:
        for r in recs:
            f.write(json.dumps(r) + "\n")


def _first_gale(recs):
    return next(r for r in recs if r["kind"] == "gale")


@pytest.mark.parametrize("case", ["section_size", "section_past_record", "negative_offset", "bad_proj",
                                  "cols_not_1024", "bad_version", "path_escape", "not_json", "duplicate",
                                  "unknown_kind", "dense_size"])
def test_manifest_refusals(packdir, case):
    def edit(recs):
        g = _first_gale(recs)
        if case == "section_size":
            g["sections"]["out_cols"][1] += 2
        elif case == "section_past_record":
            g["sections"]["out_vals"][0] = g["nbytes"]
        elif case == "negative_offset":
            g["offset"] = -256
        elif case == "bad_proj":
            g["proj"] = "w4"
        elif case == "cols_not_1024":
            g["shape"] = [g["shape"][0], 1000]
        elif case == "bad_version":
            recs[0]["version"] = 2
        elif case == "path_escape":
            g["file"] = "../outside.pack"
        elif case == "duplicate":
            recs.append(dict(g))
        elif case == "unknown_kind":
            g["kind"] = "fp8"
        elif case == "dense_size":
            next(r for r in recs if r["kind"] == "dense")["nbytes"] += 4
        return recs

    if case == "not_json":
        with open(os.path.join(packdir, PF.MANIFEST), "a") as f:
            f.write("{not json\n")
    else:
        _rewrite_manifest(packdir, edit)
    with pytest.raises(ValueError):
        PF.read_manifest(packdir)


def test_truncated_file_refused(packdir):
    f = os.path.join(packdir, PF.layer_file(1))
    size = os.path.getsize(f)
    with open(f, "r+b") as fh:
        fh.truncate(size - 100)
    with pytest.raises(ValueError, match="runs past the end"):
        PF.Pack(packdir)


def test_missing_file_refused(packdir):
    os.remove(os.path.join(packdir, PF.layer_file(0)))
    with pytest.raises(ValueError, match="missing"):
        PF.Pack(packdir)


def _patch_section(d, name, section, fn):
    pk = PF.Pack(d)
    r = pk.by_name[name]
    off, nb = r["sections"][section]
    path = os.path.join(d, r["file"])
    with open(path, "r+b") as fh:
        fh.seek(r["offset"] + off)
        raw = bytearray(fh.read(nb))
        raw = fn(raw)
        fh.seek(r["offset"] + off)
        fh.write(raw)


def test_bad_csr_refused(packdir):
    name = PF.matrix_name(0, 1, "w3")

    def swap(raw):   # row_ptr[1] > row_ptr[2]: not monotone
        a = np.frombuffer(bytes(raw), dtype="<i4").copy()
        a[1], a[2] = a[2] + 5, a[1]
        return bytearray(a.tobytes())
    _patch_section(packdir, name, "row_ptr", swap)
    with pytest.raises(ValueError, match="layers.0.experts.1.w3"):
        PF.Pack(packdir).read_gale(name)


def test_outlier_column_out_of_range_refused(packdir):
    name = PF.matrix_name(1, 2, "w2")

    def bump(raw):
        a = np.frombuffer(bytes(raw), dtype="<u2").copy()
        a[0] = INTER   # == cols
        return bytearray(a.tobytes())
    _patch_section(packdir, name, "out_cols", bump)
    with pytest.raises(ValueError):
        PF.Pack(packdir).read_gale(name)


def test_incomplete_layer_refused(tmp_path, stack):
    with PF.PackWriter(str(tmp_path / "p")) as w:
        for e, trio in enumerate(stack[0]):
            for p, m in zip(PF.PROJS, trio):
                if (e, p) != (2, "w2"):
                    w.add_gale(0, e, p, m)
    with pytest.raises(ValueError, match="expert 2 has no w2"):
        PF.Pack(str(tmp_path / "p")).layer_geometry(0)


def test_wrong_layer_shape_refused(tmp_path, stack):
    with PF.PackWriter(str(tmp_path / "p")) as w:
        for e, (w1, w3, w2) in enumerate(stack[0]):
            w.add_gale(0, e, "w1", w1)
            w.add_gale(0, e, "w3", w3)
            w.add_gale(0, e, "w2", w1 if e == 1 else w2)   # [inter, hidden] where w2 must be [hidden, inter]
    with pytest.raises(ValueError, match="shape"):
        PF.Pack(str(tmp_path / "p")).layer_geometry(0)


def test_writer_refuses_duplicates_and_short_sections(tmp_path, stack):
    w = PF.PackWriter(str(tmp_path / "p"))
    m = stack[0][0][0]
    w.add_gale(0, 0, "w1", m)
    with pytest.raises(ValueError, match="duplicate"):
        w.add_gale(0, 0, "w1", m)
    bad = dict(m)
    bad["block_scales"] = m["block_scales"][:-1]
    with pytest.raises(ValueError, match="block_scales"):
        w.add_gale(0, 0, "w3", bad)
    w.close()


def test_no_outliers_and_empty_rows(tmp_path, stack):
    m = dict(stack[0][0][0])
    m["row_ptr"] = np.zeros(m["rows"] + 1, dtype=np.int64)
    m["out_cols"] = np.zeros(0, dtype=np.uint16)
    m["out_vals"] = np.zeros(0, dtype=np.uint8)
    with PF.PackWriter(str(tmp_path / "p")) as w:
        r = w.add_gale(0, 0, "w1", m)
    assert r["outliers"] == 0 and r["sections"]["out_cols"][1] == 0
    got = PF.Pack(str(tmp_path / "p")).read_gale(r["name"])
    assert got["out_cols"].size == 0 and got["out_vals"].size == 0
    assert np.array_equal(got["signs"], m["signs"])
