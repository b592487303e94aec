"""The documented size limits of the library against the fp64 oracle.

  * GALE_MAX_COLS (16,384 columns: sixteen FWHT-1024 blocks, a workgroup of 1,024 threads);
  * GALE_MAX_ROWS (1,048,576 rows): the outputs of sampled rows, which the oracle computes from
    the same matrix restricted to those rows;
  * GALE_MAX_EXPERTS (512) with GALE_MAX_TOPK (8): routing over two 256-expert halves of the
    keys, through the one-token, decode and grouped paths, every token against the oracle.
The shapes are the DeepSeek-V4 GALE format's (sign bit per weight under a blocked FWHT-1024
rotation, fp16 scale per 128-weight block, about 1 % int4 outliers with a per-row fp16
scale) at the sizes the header allows.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config_seed, gen_logits_normal, gen_matrices, gen_matrix, gen_x

from tests.test_gpu_parity import REL_L2_BAR, np_of, oracle_pool

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_expert_gemv_amd as qq
    qq.lib()
    return qq


def row_subset(d, rows):
    """The canonical matrix restricted to the given rows, in the same format (entries of row n
    at row_ptr[n] .. row_ptr[n+1], int4 values two per byte, low nibble first)."""
    rp = d["row_ptr"]
    vals = O.decode_int4(d["out_vals"], int(rp[-1]))
    take = np.concatenate([np.arange(rp[n], rp[n + 1]) for n in rows]).astype(np.int64)
    counts = np.array([rp[n + 1] - rp[n] for n in rows], dtype=np.int64)
    v = (vals[take] & 0xF).astype(np.uint8)
    if v.size % 2:
        v = np.concatenate([v, np.zeros(1, np.uint8)])
    return {"rows": len(rows), "cols": d["cols"], "signs": d["signs"][rows], "block_scales": d["block_scales"][rows],
            "row_scales": d["row_scales"][rows], "row_ptr": np.concatenate([[0], np.cumsum(counts)]),
            "out_cols": d["out_cols"][take], "out_vals": (v[0::2] | (v[1::2] << 4)).astype(np.uint8)}


def test_row_subset_is_the_same_rows():
    # the helper itself: a subset of a small matrix dequantizes to the same rows
    m = gen_matrix(config_seed(31), (1,), 64, 2048).numpy()
    rows = [0, 3, 17, 63]
    assert np.array_equal(O.dequantize(row_subset(m, rows)), O.dequantize(m)[rows])


@pytest.mark.parametrize("n_tok", [1, 4])
def test_gemv_max_cols(q, n_tok):
    rows, cols = 48, 16384
    mats = gen_matrices(config_seed(32), [(0,), (1,)], rows, cols, device=DEV)
    tab = q.matrix_table([q.pack_matrix(m) for m in mats])
    x = gen_x(config_seed(32), (2, n_tok), 2 * n_tok, cols, device=DEV).view(2, n_tok, cols)
    y = q.expert_gemv(tab, rows, cols, x, y_dtype=torch.float32)
    for i in range(2):
        err = O.rel_l2(np_of(y[i]), O.gemv(mats[i].numpy(), x[i].cpu().numpy())).max()
        print(f"gemv [{rows}, {cols}] x {n_tok} tokens, matrix {i}: rel-L2 {err:.3e}")
        assert err <= 1e-4


def test_gemv_max_rows(q):
    rows, cols = 1 << 20, 1024
    m = gen_matrix(config_seed(33), (0,), rows, cols, device=DEV)
    tab = q.matrix_table([q.pack_matrix(m)])
    x = gen_x(config_seed(33), (1,), 1, cols, device=DEV)
    y = q.expert_gemv(tab, rows, cols, x[None], y_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    sample = sorted(set([0, 1, rows // 2, rows - 2, rows - 1] + rng.choice(rows, 59, replace=False).tolist()))
    ref = O.gemv(row_subset(m.numpy(), sample), x.cpu().numpy())[0]
    got = y[0, 0].cpu().numpy().astype(np.float64)[sample]
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"gemv [{rows}, {cols}]: {len(sample)} sampled rows, rel-L2 {err:.3e}")
    assert err <= 1e-4
    assert np.isfinite(y.cpu().numpy()).all()


@pytest.fixture(scope="module")
def wide_layer(q):
    # hidden 2048, inter 1024, top-8: the one-layer launch takes its larger task sets (four
    # sign tasks and two outlier rows per wavefront, loaded task by task)
    E, H, I = 512, 2048, 1024
    seed = config_seed(34)
    w13 = gen_matrices(seed, [(e, m) for e in range(E) for m in (0, 1)], I, H, device=DEV)
    w2 = gen_matrices(seed, [(e, 2) for e in range(E)], H, I, device=DEV)
    canon = [(w13[2 * e], w13[2 * e + 1], w2[e]) for e in range(E)]
    tab = q.expert_table([tuple(q.pack_matrix(mm) for mm in ex) for ex in canon])
    return seed, canon, tab


@pytest.mark.parametrize("T,flags", [(1, 0), (1, "staged"), (8, 0), (200, 0)])
def test_moe_max_experts_and_top_k(q, wide_layer, T, flags):
    seed, canon, tab = wide_layer
    E, H, I, K = 512, 2048, 1024, 8
    x = gen_x(seed, (7, T), T, H, device=DEV)
    lg = gen_logits_normal(seed, (7, T), T, E, device=DEV)
    fl = q.GALE_DECODE_STAGED if flags == "staged" else 0
    y, idx, w = q.moe_layer_fwd(tab, H, I, lg, x, top_k=K, flags=fl)
    ridx, rw = O.route(lg.cpu().numpy(), K)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    assert (ridx >= 256).any() and (ridx < 256).any()       # both halves of the keys chosen
    expert_of = lambda e: tuple(mm.numpy() for mm in canon[e])  # noqa: E731
    with oracle_pool() as ex:
        yref, _, _ = O.moe(expert_of, lg.cpu().numpy(), x.cpu().numpy(), k=K, map_fn=ex.map)
    err = O.rel_l2(np_of(y), yref).max()
    print(f"moe E={E} top-{K} T={T} {flags or ''}: rel-L2 {err:.3e}")
    assert err <= REL_L2_BAR


def test_one_launch_larger_task_sets_equal_staged(q, wide_layer):
    """Top-8 of 512 at hidden 2048: the one-layer launch with its task-by-task down phase equals
    the five-launch sequence bit for bit (routing, weights and outputs), on two tokens in turn."""
    seed, canon, tab = wide_layer
    E, H, I, K = 512, 2048, 1024, 8
    for t in range(2):
        x = gen_x(seed, (8, t), 1, H, device=DEV)
        lg = gen_logits_normal(seed, (8, t), 1, E, device=DEV)
        y1, i1, w1 = q.moe_layer_fwd(tab, H, I, lg, x, top_k=K)
        y5, i5, w5 = q.moe_layer_fwd(tab, H, I, lg, x, top_k=K, flags=q.GALE_DECODE_STAGED)
        assert torch.equal(i1, i5) and torch.equal(w1, w5)
        assert torch.equal(y1, y5), t
