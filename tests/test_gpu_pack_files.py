"""Experts loaded from pack files (MI355X): a stack written to disk by the pack writer and
loaded by load_stack gives the same device layout, bit for bit, as the same matrices packed
straight from memory, the same MoE outputs bit for bit on the decode, one-launch and grouped
paths, and the oracle's outputs within the parity bar.

Inputs: seeded synthetic experts at the "DeepSeek-V4-Flash - GALE 1-bit experts" card's
shapes (w1/w3 [2048, 4096], w2 [4096, 2048], 1 % outliers), 16 experts per layer, two
layers, and a per-layer selection bias stored as a dense record.  The byte layout of the
pack is this library's own: parity against the published pack stays unpinned.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config_seed, gen_logits_normal, gen_matrix_bank, gen_x

pytestmark = pytest.mark.gpu

DEV = "cuda"
HIDDEN, INTER, EXPERTS, LAYERS, TOPK = 4096, 2048, 16, 2, 6
REL_L2_BAR = 2e-3


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_expert_gemv_amd as qq
    qq.lib()
    return qq


def _canon(seed):
    """[layer][expert] = (w1, w3, w2) canonical numpy dicts (generated on the GPU, copied out)."""
    out = []
    for l in range(LAYERS):
        b13 = gen_matrix_bank(seed, [(l, e, m) for e in range(EXPERTS) for m in (0, 1)], INTER, HIDDEN, device=DEV)
        b2 = gen_matrix_bank(seed, [(l, e, 2) for e in range(EXPERTS)], HIDDEN, INTER, device=DEV)

        def one(b, i, rows, cols):
            return {"rows": rows, "cols": cols,
                    "signs": b["signs"][i].cpu().numpy().view(np.uint32),
                    "block_scales": b["block_scales"][i].cpu().numpy().view(np.float16),
                    "row_scales": b["row_scales"].cpu().numpy().view(np.float16),
                    "row_ptr": b["row_ptr"].cpu().numpy().astype(np.int64),
                    "out_cols": b["out_cols"][i].cpu().numpy().view(np.uint16),
                    "out_vals": b["out_vals"][i].cpu().numpy()}
        out.append([(one(b13, 2 * e, INTER, HIDDEN), one(b13, 2 * e + 1, INTER, HIDDEN), one(b2, e, HIDDEN, INTER))
                    for e in range(EXPERTS)])
    return out


@pytest.fixture(scope="module")
def loaded(q, tmp_path_factory):
    from quantized_expert_gemv_amd import pack_files as PF
    seed = config_seed(11)
    canon = _canon(seed)
    d = str(tmp_path_factory.mktemp("pack"))
    rng = np.random.default_rng(seed & 0xFFFFFFFF)
    biases = [rng.normal(0, 0.5, EXPERTS).astype(np.float32) for _ in range(LAYERS)]
    with PF.PackWriter(d) as w:
        for l in range(LAYERS):
            for e in range(EXPERTS):
                for p, m in zip(PF.PROJS, canon[l][e]):
                    w.add_gale(l, e, p, m)
            w.add_dense(f"layers.{l}.gate.selection_bias", biases[l])
    print("pack written; loading", flush=True)
    st = PF.load_stack(d, DEV)
    torch.cuda.synchronize()
    return seed, canon, biases, st


def _direct(q, m):
    """The same canonical matrix packed straight from memory (no files)."""
    from synth import CanonicalMatrix
    vals = m["out_vals"] if len(m["out_vals"]) else np.zeros(1, dtype=np.uint8)
    cm = CanonicalMatrix(
        rows=m["rows"], cols=m["cols"],
        signs=torch.from_numpy(np.ascontiguousarray(m["signs"]).view(np.int32)).to(DEV),
        block_scales=torch.from_numpy(np.ascontiguousarray(m["block_scales"]).view(np.int16)).to(DEV),
        row_scales=torch.from_numpy(np.ascontiguousarray(m["row_scales"]).view(np.int16)).to(DEV),
        row_ptr=torch.from_numpy(np.asarray(m["row_ptr"], dtype=np.int32)).to(DEV),
        out_cols=torch.from_numpy(np.ascontiguousarray(m["out_cols"]).view(np.int16)).to(DEV),
        out_vals=torch.from_numpy(np.ascontiguousarray(vals)).to(DEV))
    return q.pack_matrix(cm)


def test_loaded_layout_equals_direct_pack(q, loaded):
    seed, canon, biases, st = loaded
    assert (st.hidden, st.inter, st.experts, st.layer_ids) == (HIDDEN, INTER, EXPERTS, list(range(LAYERS)))
    for l in range(LAYERS):
        for e in range(EXPERTS):
            for j in range(3):
                a = st.matrices[l][e][j]
                b = _direct(q, canon[l][e][j])
                assert (a.rows, a.cols, a.nnz) == (b.rows, b.cols, b.nnz)
                assert torch.equal(a.signs.view(-1), b.signs.view(-1)), (l, e, j)
                assert torch.equal(a.block_scales.view(-1), b.block_scales.view(-1)), (l, e, j)
                assert torch.equal(a.row_scales.view(-1)[:a.rows], b.row_scales.view(-1)[:b.rows])
                assert torch.equal(a.row_ptr.view(-1)[:a.rows + 1], b.row_ptr.view(-1)[:b.rows + 1])
                nb = 2 * a.nnz
                assert torch.equal(a.out_cols.view(torch.uint8)[:nb], b.out_cols.view(torch.uint8)[:nb])
                nv = (a.nnz + 1) // 2
                assert torch.equal(a.out_vals.view(torch.uint8)[:nv], b.out_vals.view(torch.uint8)[:nv])
    for l in range(LAYERS):
        t = st.dense[f"layers.{l}.gate.selection_bias"]
        assert t.device.type == "cuda" and t.dtype == torch.float32
        assert np.array_equal(t.cpu().numpy(), biases[l])


@pytest.mark.parametrize("T", [1, 5, 300])
def test_loaded_layer_matches_direct_and_oracle(q, loaded, T):
    seed, canon, biases, st = loaded
    l = T % LAYERS
    direct = q.expert_table([tuple(_direct(q, m) for m in canon[l][e]) for e in range(EXPERTS)])
    x = gen_x(seed, (2000, T), T, HIDDEN, device=DEV)
    lg = gen_logits_normal(seed, (2000, T), T, EXPERTS, device=DEV)
    bias = st.dense[f"layers.{l}.gate.selection_bias"]
    print(f"loaded layer {l}, T={T}", flush=True)
    y, idx, w = q.moe_layer_fwd(st.tables[l], HIDDEN, INTER, lg, x, top_k=TOPK, select_bias=bias)
    yd, idxd, wd = q.moe_layer_fwd(direct, HIDDEN, INTER, lg, x, top_k=TOPK, select_bias=bias)
    assert torch.equal(idx, idxd) and torch.equal(w, wd) and torch.equal(y, yd)
    # the oracle reads the generator's matrices, not the files
    n = min(T, 8)
    yref, ridx, _ = O.moe(lambda e: canon[l][e], lg[:n].cpu().numpy(), x[:n].cpu().numpy(), k=TOPK,
                          select_bias=biases[l])
    assert np.array_equal(idx[:n].cpu().numpy(), ridx)
    err = O.rel_l2(y[:n].float().cpu().numpy().astype(np.float64), yref).max()
    print(f"loaded layer T={T} rel-L2 {err:.3e} over {n} tokens", flush=True)
    assert err <= REL_L2_BAR


def test_loaded_stack_one_launch_equals_layer_calls(q, loaded):
    seed, canon, biases, st = loaded
    xs = [gen_x(seed, (3000 + l,), 1, HIDDEN, device=DEV) for l in range(LAYERS)]
    lgs = [gen_logits_normal(seed, (3000 + l,), 1, EXPERTS, device=DEV) for l in range(LAYERS)]
    ys = [torch.empty(1, HIDDEN, dtype=torch.float16, device=DEV) for _ in range(LAYERS)]
    lt = q.layer_table([dict(experts=st.tables[l], logits=lgs[l], x=xs[l], y=ys[l],
                             select_bias=st.dense[f"layers.{l}.gate.selection_bias"]) for l in range(LAYERS)])
    ws = q.moe_workspace(q.decode_stack_workspace_bytes(HIDDEN, INTER, TOPK), DEV)
    print("loaded stack, one launch", flush=True)
    q.moe_decode_stack(HIDDEN, INTER, EXPERTS, TOPK, lt, ws=ws)
    for l in range(LAYERS):
        yr, _, _ = q.moe_layer_fwd(st.tables[l], HIDDEN, INTER, lgs[l], xs[l], top_k=TOPK,
                                   select_bias=st.dense[f"layers.{l}.gate.selection_bias"],
                                   flags=q.GALE_DECODE_STAGED)
        assert torch.equal(ys[l], yr), l
    assert q.sync_status(ws)[0] == 0
