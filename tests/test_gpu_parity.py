"""GPU parity of every libgale entry point against the fp64 oracle (MI355X only).

Inputs come from the seeded generator (synth); expected values from oracle/.
Bars: bit-exact for sign unpacking, outlier decoding and routing indices; relative
L2 <= 2e-3 per output vector for floating point (fp32 accumulation, fp16 output).
Closed-form cases with fp32 output use CLOSED_TOL = 1e-4: the activation enters the
matrix cores as four e4m3 terms (exact to ~2^-16 per element) and the MFMA's own
accumulation of a 128-long block carries ~2^-18 of the block's sum of |products|,
which for one 1024-column chunk is ~3e-5 of the result.
"""
import contextlib
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from synth import CanonicalMatrix, config_seed, gen_logits_normal, gen_logits_zipf, gen_matrices, gen_matrix, gen_x

pytestmark = pytest.mark.gpu

REL_L2_BAR = 2e-3
CLOSED_TOL = 1e-4
# threads for the oracle's independent per-matrix / per-expert evaluations (numpy releases the
# GIL in its array work); at most the 16 cores a GPU machine gives one GPU
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@contextlib.contextmanager
def oracle_pool():
    """A thread pool for the oracle with numpy's BLAS held to one thread per worker (BLAS
    threads inside every worker would oversubscribe the cores many times over)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(ORACLE_THREADS) as ex:
        yield ex


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_expert_gemv_amd as qq
    qq.lib()
    return qq


DEV = "cuda"


def canon_from_dict(d) -> CanonicalMatrix:
    """oracle-style numpy dict -> CanonicalMatrix on the GPU."""
    vals = d["out_vals"] if len(d["out_vals"]) else np.zeros(1, dtype=np.uint8)
    return CanonicalMatrix(
        rows=d["rows"], cols=d["cols"],
        signs=torch.from_numpy(np.ascontiguousarray(d["signs"]).view(np.int32)).to(DEV),
        block_scales=torch.from_numpy(np.ascontiguousarray(d["block_scales"], dtype=np.float16).view(np.int16)).to(DEV),
        row_scales=torch.from_numpy(np.ascontiguousarray(d["row_scales"], dtype=np.float16).view(np.int16)).to(DEV),
        row_ptr=torch.from_numpy(np.asarray(d["row_ptr"], dtype=np.int32)).to(DEV),
        out_cols=torch.from_numpy(np.ascontiguousarray(d["out_cols"], dtype=np.uint16).view(np.int16)).to(DEV),
        out_vals=torch.from_numpy(np.ascontiguousarray(vals, dtype=np.uint8)).to(DEV),
    )


def hadamard_sign_dict(N, K, scale_num=1.0):
    i = np.arange(1024, dtype=np.uint64)
    pc = (O.popcount(i[:, None] & i[None, :]) & 1).astype(np.uint8)
    bits = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 128), dtype=np.float64)
    for blk in range(min(N, K) // 1024):
        bits[blk * 1024:(blk + 1) * 1024, blk * 1024:(blk + 1) * 1024] = pc
        scales[blk * 1024:(blk + 1) * 1024, blk * 8:(blk + 1) * 8] = scale_num / 32.0
    return {"rows": N, "cols": K, "signs": np.packbits(bits, axis=1, bitorder="little").view(np.uint32),
            "block_scales": scales.astype(np.float16), "row_scales": np.zeros(N, dtype=np.float16),
            "row_ptr": np.zeros(N + 1, dtype=np.int64), "out_cols": np.zeros(0, dtype=np.uint16),
            "out_vals": np.zeros(0, dtype=np.uint8)}


def np_of(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# ----------------------------------------------------------------------------
# layout and decode: bit-exact
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols", [(2048, 4096), (4096, 2048), (48, 1024), (16, 7168)])
def test_sign_and_outlier_decode_bit_exact(q, rows, cols):
    m = gen_matrix(config_seed(1), (rows, cols), rows, cols, device=DEV)
    pm = q.pack_matrix(m)
    back = q.debug_unpack_signs(pm)
    assert torch.equal(back, m.signs)
    # device packer == host packer
    hs, hsc = q.pack_host(rows, cols, m.signs.cpu(), m.block_scales.cpu())
    assert torch.equal(pm.signs.view(-1).cpu(), hs.view(-1)) and torch.equal(pm.block_scales.view(-1).cpu(), hsc.view(-1))
    r, c, v = q.debug_unpack_outliers(pm)
    orr, occ, ovv = O.outlier_triplets(m.numpy())
    assert np.array_equal(r.cpu().numpy(), orr) and np.array_equal(c.cpu().numpy(), occ)
    assert np.array_equal(v.cpu().numpy(), ovv)


# ----------------------------------------------------------------------------
# FWHT
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_fwht_parity(q, dtype):
    x = gen_x(config_seed(2), (0,), 5, 4096, device=DEV).to(dtype)
    y = q.fwht1024(x, out_dtype=torch.float32)
    ref = O.rotate(np_of(x))
    err = np.abs(np_of(y) - ref).max() / np.abs(ref).max()
    assert err <= 1e-6, err
    # involution: H(H x) = x
    z = q.fwht1024(y)
    assert np.abs(np_of(z) - np_of(x)).max() <= 1e-5 * np.abs(np_of(x)).max()
    # fp16 output rounds to nearest
    y16 = q.fwht1024(x, out_dtype=torch.float16)
    assert np.abs(np_of(y16) - ref).max() <= np.abs(ref).max() * 2 ** -11


# ----------------------------------------------------------------------------
# GEMV
# ----------------------------------------------------------------------------
def test_gemv_single_matrix_config(q):
    """One [2048 out, 4096 in] matrix, one token (the single-matrix workload)."""
    m = gen_matrix(config_seed(1), (0,), 2048, 4096, device=DEV)
    x = gen_x(config_seed(1), (0,), 1, 4096, device=DEV)
    tab = q.matrix_table([q.pack_matrix(m)])
    ref = O.gemv(m.numpy(), x.cpu().numpy())
    y16 = q.expert_gemv(tab, 2048, 4096, x[None])
    y32 = q.expert_gemv(tab, 2048, 4096, x[None], y_dtype=torch.float32)
    e16 = O.rel_l2(np_of(y16[0]), ref).max()
    e32 = O.rel_l2(np_of(y32[0]), ref).max()
    print(f"gemv rel-L2 fp16 out {e16:.3e}  fp32 out {e32:.3e}")
    assert e16 <= REL_L2_BAR
    assert e32 <= 1e-4


@pytest.mark.parametrize("n_tok", [1, 2, 3, 4, 5, 7])
def test_gemv_tokens_and_ragged_tiles(q, n_tok):
    rows, cols, n_mat = 80, 2048, 3                      # 5 row tiles: ragged against 2 and 4 tiles per WG
    mats = gen_matrices(config_seed(3), [(i,) for i in range(n_mat)], rows, cols, device=DEV)
    x = torch.stack([gen_x(config_seed(3), (i, 1), n_tok, cols, device=DEV) for i in range(n_mat)])
    tab = q.matrix_table([q.pack_matrix(m) for m in mats])
    outs = {}
    for r in (1, 2, 4, 8):
        outs[r] = q.expert_gemv(tab, rows, cols, x, y_dtype=torch.float32, flags=q.gale_tiles_flag(r))
    for i in range(n_mat):
        ref = O.gemv(mats[i].numpy(), x[i].cpu().numpy())
        assert O.rel_l2(np_of(outs[1][i]), ref).max() <= 1e-4
    for r in (2, 4, 8):
        assert torch.equal(outs[r], outs[1])             # workgroup shape does not change the arithmetic


def test_gemv_shared_x_rotated_input_and_long_k(q):
    rows, cols = 64, 7168                                # 7 FWHT blocks (non power of two)
    mats = gen_matrices(config_seed(4), [(0,), (1,)], rows, cols, device=DEV)
    x = gen_x(config_seed(4), (5,), 2, cols, device=DEV)
    tab = q.matrix_table([q.pack_matrix(m) for m in mats])
    y = q.expert_gemv(tab, rows, cols, x, x_shared=True, y_dtype=torch.float32)
    xt = torch.from_numpy(O.rotate(np_of(x))).float().to(DEV)
    yr = q.expert_gemv(tab, rows, cols, xt, x_shared=True, y_dtype=torch.float32, flags=q.GALE_X_ROTATED)
    for i in range(2):
        ref = O.gemv(mats[i].numpy(), x.cpu().numpy())
        assert O.rel_l2(np_of(y[i]), ref).max() <= 1e-4
        assert O.rel_l2(np_of(yr[i]), ref).max() <= 1e-4


def test_gemv_hadamard_sign_identity(q):
    # rows carrying H's sign pattern with scale 1/32 return x itself
    d = hadamard_sign_dict(2048, 4096)
    tab = q.matrix_table([q.pack_matrix(canon_from_dict(d))])
    x = gen_x(config_seed(5), (0,), 3, 4096, device=DEV)
    y = q.expert_gemv(tab, 2048, 4096, x[None], y_dtype=torch.float32)
    assert O.rel_l2(np_of(y[0]), np_of(x[:, :2048])).max() <= CLOSED_TOL


def test_gemv_zero_bits_closed_form_and_subnormal_scales(q):
    N, K = 32, 4096
    m = gen_matrix(config_seed(6), (0,), N, K, device=DEV)
    d = m.numpy()
    d["signs"] = np.zeros_like(d["signs"])
    d["block_scales"] = np.full_like(d["block_scales"], np.float16(0.015625))
    d["row_scales"] = np.zeros_like(d["row_scales"])
    x = gen_x(config_seed(6), (1,), 1, K, device=DEV)
    y = q.expert_gemv(q.matrix_table([q.pack_matrix(canon_from_dict(d))]), N, K, x[None], y_dtype=torch.float32)
    xs = np_of(x[0])
    expect = 32.0 * 0.015625 * xs[0::1024].sum()
    assert np.abs(np_of(y[0]) - expect).max() <= CLOSED_TOL * abs(expect) + 1e-6
    # subnormal fp16 block scales are honoured, not flushed
    d2 = m.numpy()
    sub = np.array([2 ** -24, 3 * 2 ** -24, 2 ** -15, 1023 * 2 ** -24], dtype=np.float16)
    bs = d2["block_scales"].copy()
    bs[:, ::2] = sub[np.arange(bs[:, ::2].size).reshape(bs[:, ::2].shape) % 4]
    d2["block_scales"] = bs
    d2["row_scales"] = np.zeros_like(d2["row_scales"])
    y2 = q.expert_gemv(q.matrix_table([q.pack_matrix(canon_from_dict(d2))]), N, K, x[None], y_dtype=torch.float32)
    ref2 = O.gemv(d2, x.cpu().numpy())
    assert O.rel_l2(np_of(y2[0]), ref2).max() <= 1e-4


def test_gemv_outlier_edges(q):
    # scales 0: y is the outlier sparse dot alone; rows with 0, 1 and 300 outliers, columns 0 and K-1
    N, K = 32, 2048
    rng = np.random.default_rng(11)
    rp = [0]
    cols, vals = [], []
    for n in range(N):
        cnt = [0, 1, 300, 41][n % 4]
        cs = np.sort(rng.choice(K, size=cnt, replace=False)) if cnt else np.zeros(0, dtype=np.int64)
        if n == 5:
            cs = np.array([0, K - 1])
        cols.extend(cs.tolist())
        vals.extend(rng.integers(-8, 8, size=len(cs)).tolist())
        rp.append(len(cols))
    nib = [v & 0xF for v in vals] + ([0] if len(vals) % 2 else [])
    d = {"rows": N, "cols": K, "signs": rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32),
         "block_scales": np.zeros((N, K // 128), dtype=np.float16),
         "row_scales": np.full(N, 0.05, dtype=np.float16), "row_ptr": np.array(rp),
         "out_cols": np.array(cols, dtype=np.uint16),
         "out_vals": np.array([nib[i] | (nib[i + 1] << 4) for i in range(0, len(nib), 2)], dtype=np.uint8)}
    x = gen_x(config_seed(7), (0,), 2, K, device=DEV)
    tab = q.matrix_table([q.pack_matrix(canon_from_dict(d))])
    y = q.expert_gemv(tab, N, K, x[None], y_dtype=torch.float32)
    ref = O.gemv(d, x.cpu().numpy())
    err = np.abs(np_of(y[0]) - ref).max()
    assert err <= 1e-5 * np.abs(ref).max()
    assert np.all(np_of(y[0])[:, 0::4] == 0.0)           # rows without outliers give exactly 0


def test_gemv_many_matrices_sampled(q):
    """The launch shape of the sustained benchmark: many distinct matrices, one token each;
    every matrix's output against the oracle; all-zero activations give exact zeros."""
    n_mat = 64
    mats = gen_matrices(config_seed(1), [(100 + i,) for i in range(n_mat)], 2048, 4096, device=DEV)
    x = torch.stack([gen_x(config_seed(1), (100 + i,), 1, 4096, device=DEV) for i in range(n_mat)])
    tab = q.matrix_table([q.pack_matrix(m) for m in mats])
    y = q.expert_gemv(tab, 2048, 4096, x)
    y2 = q.expert_gemv(tab, 2048, 4096, x)
    assert torch.equal(y, y2)                            # deterministic
    xs = x.cpu().numpy()
    with oracle_pool() as ex:
        refs = list(ex.map(lambda i: O.gemv(mats[i].numpy(), xs[i]), range(n_mat)))
    for i in range(n_mat):
        assert O.rel_l2(np_of(y[i]), refs[i]).max() <= REL_L2_BAR, i
    # all-zero activations: exactly zero outputs (every term of the sum is zero)
    z = q.expert_gemv(tab, 2048, 4096, torch.zeros_like(x))
    assert torch.count_nonzero(z) == 0


@pytest.mark.parametrize("rows,cols,n_mat,xdt,rotated,shared,flags", [
    (2048, 4096, 40, torch.float16, False, False, 0),           # the single-matrix workload shape
    (80, 2048, 200, torch.float32, False, False, "t1"),         # ragged, many items per workgroup
    (80, 2048, 200, torch.float16, False, False, "t2"),
    (80, 2048, 97, torch.float16, False, False, "t4"),
    (64, 7168, 30, torch.float32, True, False, 0),              # 7 chunks, pre-rotated fp32 input
    (2048, 4096, 12, torch.float16, False, True, 0),            # one x shared by every matrix
    (2048, 4096, 24, torch.float16, False, False, "s1"),        # 2,048-entry outlier staging
    (2048, 4096, 24, torch.float16, False, False, "s2"),        # 4,096-entry outlier staging
    (48, 1024, 300, torch.float16, False, False, 0),            # one chunk: one wavefront per workgroup
    (32, 8192, 40, torch.float16, False, False, 0),             # eight chunks: the widest one-launch workgroup
])
def test_gemv_one_launch_equals_prepared(q, rows, cols, n_mat, xdt, rotated, shared, flags):
    """One token per matrix: the GEMV rotates and splits x itself, in one launch, with the same
    record code as the preparation kernel, so its output equals prepare + GEMV bit for bit
    (row tiles per unit, outlier stagings, dtypes, shared x, items crossing workgroups)."""
    f = {0: 0, "t1": q.gale_tiles_flag(1), "t2": q.gale_tiles_flag(2), "t4": q.gale_tiles_flag(4),
         "s1": q.gale_outlier_stage_flag(100), "s2": q.gale_outlier_stage_flag(200)}[flags]
    if rotated:
        f |= q.GALE_X_ROTATED
    mats = gen_matrices(config_seed(21), [(rows, cols, i) for i in range(n_mat)], rows, cols, device=DEV)
    tab = q.matrix_table([q.pack_matrix(m) for m in mats])
    n_x = 1 if shared else n_mat
    x = torch.stack([gen_x(config_seed(21), (rows, cols, 500 + i), 1, cols, device=DEV) for i in range(n_x)]).to(xdt)
    xin = x[0] if shared else x
    print(f"one-launch GEMV [{rows},{cols}] x{n_mat} {xdt} rotated={rotated} shared={shared} flags={flags}", flush=True)
    y1 = q.expert_gemv(tab, rows, cols, xin, x_shared=shared, y_dtype=torch.float32, flags=f)
    rec = q.prepare_activations(x.reshape(-1, cols), rotated=rotated)
    y2 = q.expert_gemv(tab, rows, cols, rec, x_shared=shared, y_dtype=torch.float32,
                       flags=(f & ~q.GALE_X_ROTATED) | q.GALE_X_PREPARED)
    assert torch.equal(y1, y2)
    i = n_mat - 1
    xi = (x[0] if shared else x[i]).float().cpu().numpy()
    ref = O.gemv(mats[i].numpy(), xi, pre_rotated=rotated)
    assert O.rel_l2(np_of(y1[i]), ref).max() <= CLOSED_TOL


# ----------------------------------------------------------------------------
# FFN
# ----------------------------------------------------------------------------
def _expert(q, seed, e, hidden=4096, inter=2048):
    w1, w3 = gen_matrices(seed, [(e, 0), (e, 1)], inter, hidden, device=DEV)
    w2 = gen_matrix(seed, (e, 2), hidden, inter, device=DEV)
    return (w1, w3, w2), (q.pack_matrix(w1), q.pack_matrix(w3), q.pack_matrix(w2))


def test_ffn_one_expert_config(q):
    (w1, w3, w2), packed = _expert(q, config_seed(2), 0)
    x = gen_x(config_seed(2), (0,), 1, 4096, device=DEV)
    y = q.expert_ffn(q.expert_table([packed]), 4096, 2048, x[None])
    ref = O.ffn(w1.numpy(), w3.numpy(), w2.numpy(), x.cpu().numpy())
    e = O.rel_l2(np_of(y[0]), ref).max()
    print(f"ffn rel-L2 {e:.3e}")
    assert e <= REL_L2_BAR


@pytest.mark.parametrize("shared", [False, True])
def test_ffn_one_token_equals_batched_token(q, shared):
    """One token per expert: both GEMV phases rotate and split their inputs themselves (one
    launch each); the same token inside a two-token batch goes through prepared records.
    Each token's products are independent of the other's, so the outputs agree bit for bit;
    and the one-token outputs match the oracle."""
    seed = config_seed(22)
    E = 12
    ex = [_expert(q, seed, e) for e in range(E)]
    tab = q.expert_table([p for _, p in ex])
    if shared:
        x1 = gen_x(seed, (9,), 1, 4096, device=DEV)
        x2 = torch.cat([x1, gen_x(seed, (10,), 1, 4096, device=DEV)])
    else:
        x1 = torch.stack([gen_x(seed, (100 + e,), 1, 4096, device=DEV) for e in range(E)])
        x2 = torch.cat([x1, torch.stack([gen_x(seed, (200 + e,), 1, 4096, device=DEV) for e in range(E)])], dim=1)
    y1 = q.expert_ffn(tab, 4096, 2048, x1, x_shared=shared)
    y2 = q.expert_ffn(tab, 4096, 2048, x2, x_shared=shared)
    assert torch.equal(y1[:, 0], y2[:, 0])
    for e in (0, E - 1):
        (w1, w3, w2), _ = ex[e]
        xe = (x1 if shared else x1[e]).cpu().numpy()
        ref = O.ffn(w1.numpy(), w3.numpy(), w2.numpy(), xe)
        assert O.rel_l2(np_of(y1[e]), ref).max() <= REL_L2_BAR


def test_ffn_tokens_and_experts(q):
    seed = config_seed(12)
    ex = [_expert(q, seed, e) for e in range(2)]
    x = gen_x(seed, (3,), 5, 4096, device=DEV)
    y = q.expert_ffn(q.expert_table([p for _, p in ex]), 4096, 2048, x, x_shared=True)
    for e in range(2):
        (w1, w3, w2), _ = ex[e]
        ref = O.ffn(w1.numpy(), w3.numpy(), w2.numpy(), x.cpu().numpy())
        assert O.rel_l2(np_of(y[e]), ref).max() <= REL_L2_BAR


def test_ffn_closed_form(q):
    w1 = canon_from_dict(hadamard_sign_dict(2048, 4096))
    w2 = canon_from_dict(hadamard_sign_dict(4096, 2048))
    p1, p2 = q.pack_matrix(w1), q.pack_matrix(w2)
    x = gen_x(config_seed(8), (0,), 2, 4096, device=DEV) * 0.25
    y = q.expert_ffn(q.expert_table([(p1, p1, p2)]), 4096, 2048, x[None])
    xs = np_of(x)[:, :2048]
    ref = np.zeros((2, 4096))
    ref[:, :2048] = xs * xs / (1 + np.exp(-xs))
    assert O.rel_l2(np_of(y[0]), ref).max() <= 1e-3     # fp16 output rounding dominates


@pytest.mark.parametrize("gate_scale,up_scale", [(1.0, 2.0), (2.0, 1.0)])
def test_ffn_closed_form_gate_and_up_differ(q, gate_scale, up_scale):
    # w1 (gate) and w3 (up) with different scales: y = silu(gate_scale x) * up_scale x on
    # the first 2048 features; a kernel that applied SiLU to the up projection would give
    # silu(up_scale x) * gate_scale x instead
    w1 = canon_from_dict(hadamard_sign_dict(2048, 4096, scale_num=gate_scale))
    w3 = canon_from_dict(hadamard_sign_dict(2048, 4096, scale_num=up_scale))
    w2 = canon_from_dict(hadamard_sign_dict(4096, 2048))
    p1, p3, p2 = q.pack_matrix(w1), q.pack_matrix(w3), q.pack_matrix(w2)
    x = gen_x(config_seed(8), (1,), 2, 4096, device=DEV) * 0.25
    y = q.expert_ffn(q.expert_table([(p1, p3, p2)]), 4096, 2048, x[None])
    xs = np_of(x)[:, :2048]
    ref = np.zeros((2, 4096))
    ref[:, :2048] = gate_scale * xs / (1 + np.exp(-gate_scale * xs)) * up_scale * xs
    swapped = np.zeros((2, 4096))
    swapped[:, :2048] = up_scale * xs / (1 + np.exp(-up_scale * xs)) * gate_scale * xs
    assert O.rel_l2(np_of(y[0]), ref).max() <= 1e-3
    assert O.rel_l2(swapped, ref).max() > 1e-1
    # the same expert through the one-launch decode layer (top-1 of one expert: weight 1)
    lg = torch.zeros(1, 1, dtype=torch.float32, device=DEV)
    for flags in (0, q.GALE_DECODE_STAGED):
        yl, _, _ = q.moe_layer_fwd(q.expert_table([(p1, p3, p2)]), 4096, 2048, lg, x[:1], top_k=1, flags=flags)
        assert O.rel_l2(np_of(yl), ref[:1]).max() <= 1e-3


# ----------------------------------------------------------------------------
# routing and MoE layer (decode path)
# ----------------------------------------------------------------------------
def test_route_exact_with_ties(q):
    lg = gen_logits_normal(config_seed(3), (9,), 40, 256)
    lg[3, :] = 0.0
    lg[4, [10, 20, 30, 40, 50, 60, 70]] = 9.0
    lg[5, :] = -5.0
    lg[5, 17] = -0.0
    lg[5, 16] = 0.0
    idx, w, off, perm = q.route_topk(lg.to(DEV), 6, group=True)
    ridx, rw = O.route(lg.numpy(), 6)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    roff, rperm = O.group_by_expert(ridx, 256)
    assert np.array_equal(off.cpu().numpy(), roff) and np.array_equal(perm.cpu().numpy(), rperm)
    # large-batch grouping (chunked kernels)
    lg2 = gen_logits_normal(config_seed(3), (10,), 300, 256)
    idx2, w2, off2, perm2 = q.route_topk(lg2.to(DEV), 6, group=True)
    ridx2, _ = O.route(lg2.numpy(), 6)
    roff2, rperm2 = O.group_by_expert(ridx2, 256)
    assert np.array_equal(idx2.cpu().numpy(), ridx2)
    assert np.array_equal(off2.cpu().numpy(), roff2) and np.array_equal(perm2.cpu().numpy(), rperm2)
    # few experts, ties among them: with as many experts as slots every expert is taken,
    # in (logit desc, index asc) order; a tie plus too few keys must not pass for no tie
    for row in ([1.0, 1.0, 2.0, 3.0, 4.0, 5.0], [3.0] * 7, [1.0, 1.0, 2.0, 3.0, 4.0, 5.0, 1.0, 0.0]):
        lg3 = torch.tensor([row, row[::-1]], dtype=torch.float32)
        idx3, w3, _, _ = q.route_topk(lg3.to(DEV), 6, group=True)
        ridx3, rw3 = O.route(lg3.numpy(), 6)
        assert np.array_equal(idx3.cpu().numpy(), ridx3), row
        assert np.abs(w3.cpu().numpy() - rw3).max() <= 1e-6


@pytest.fixture(scope="module")
def layer(q):
    seed = config_seed(3)
    E = 256
    w13 = gen_matrices(seed, [(e, m) for e in range(E) for m in (0, 1)], 2048, 4096, device=DEV)
    w2 = gen_matrices(seed, [(e, 2) for e in range(E)], 4096, 2048, device=DEV)
    canon = [(w13[2 * e], w13[2 * e + 1], w2[e]) for e in range(E)]
    packed = [(q.pack_matrix(a), q.pack_matrix(b), q.pack_matrix(c)) for a, b, c in canon]
    return seed, canon, q.expert_table(packed)


@pytest.mark.parametrize("T", [1, 2, 4, 16, 32, 63, 64])
def test_moe_decode_layer(q, layer, T):
    seed, canon, tab = layer
    x = gen_x(seed, (1000, T), T, 4096, device=DEV)
    lg = gen_logits_normal(seed, (1000, T), T, 256, device=DEV)
    y, idx, w = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6)
    y_again, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6)
    assert torch.equal(y, y_again)
    ridx, rw = O.route(lg.cpu().numpy(), 6)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    expert_of = lambda e: tuple(m.numpy() for m in canon[e])  # noqa: E731
    with oracle_pool() as ex:
        yref, _, _ = O.moe(expert_of, lg.cpu().numpy(), x.cpu().numpy(), k=6, map_fn=ex.map)
    err = O.rel_l2(np_of(y), yref).max()                 # every token
    print(f"moe T={T} rel-L2 {err:.3e}")
    assert err <= REL_L2_BAR


@pytest.mark.parametrize("variant", ["bias", "fixed"])
@pytest.mark.parametrize("T,flags", [(1, 0), (5, 0), (1, "staged"), (300, 0)])
def test_moe_routing_variants(q, layer, variant, T, flags):
    """Selection bias (moves the choice, not the weights) and fixed experts per token (hash
    routing) through the one-launch layer (T = 1), the five-launch decode sequence and the
    grouped path: routing and outputs against the oracle for every token."""
    seed, canon, tab = layer
    rng = np.random.default_rng(40 + T)
    x = gen_x(seed, (4000, T), T, 4096, device=DEV)
    lg = gen_logits_normal(seed, (4000, T), T, 256, device=DEV)
    lgn = lg.cpu().numpy()
    fl = q.GALE_DECODE_STAGED if flags == "staged" else 0
    if variant == "bias":
        bias_np = (rng.standard_normal(256) * 0.5).astype(np.float32)
        kw = {"select_bias": torch.from_numpy(bias_np).to(DEV)}
        ridx, rw = O.route(lgn, 6, select_bias=bias_np)
        assert not np.array_equal(ridx, O.route(lgn, 6)[0])          # the bias does move the choice
    else:
        fixed_np = np.stack([rng.permutation(256)[:6] for _ in range(T)]).astype(np.int32)
        kw = {"fixed_idx": torch.from_numpy(fixed_np).to(DEV)}
        ridx, rw = O.route(lgn, 6, fixed_idx=fixed_np)
    y, idx, w = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, flags=fl, **kw)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    expert_of = lambda e: tuple(m.numpy() for m in canon[e])  # noqa: E731
    okw = {"select_bias": bias_np} if variant == "bias" else {"fixed_idx": fixed_np}
    with oracle_pool() as ex:
        yref, _, _ = O.moe(expert_of, lgn, x.cpu().numpy(), k=6, map_fn=ex.map, **okw)
    err = O.rel_l2(np_of(y), yref).max()                 # every token
    print(f"routing {variant} T={T} {flags or ''}: rel-L2 {err:.3e}")
    assert err <= REL_L2_BAR


def test_moe_grouped_gemm_partial_tiles(q, layer):
    """Experts whose pair counts end a tile at every fragment boundary (1, 15, 16, 17, 63, 64,
    65, 127, 128, 129 pairs; fixed experts, one per token): the tile GEMM runs only the
    16-pair fragments that hold pairs.  Against the GEMV items and the oracle."""
    seed, canon, tab = layer
    counts = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129]
    exps = [3 + 7 * i for i in range(len(counts))]
    rng = np.random.default_rng(77)
    fixed_np = np.concatenate([np.full(c, e, np.int32) for c, e in zip(counts, exps)])
    rng.shuffle(fixed_np)
    T = fixed_np.size
    fixed_np = fixed_np.reshape(T, 1)
    x = gen_x(seed, (5000,), T, 4096, device=DEV)
    lg = gen_logits_normal(seed, (5000,), T, 256, device=DEV)
    kw = {"fixed_idx": torch.from_numpy(fixed_np).to(DEV)}
    yg, idx, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=1, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_GEMM, **kw)
    yi, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=1, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_ITEMS, **kw)
    assert np.array_equal(idx.cpu().numpy(), fixed_np)
    e_gi = O.rel_l2(np_of(yg), np_of(yi)).max()
    expert_of = lambda e: tuple(m.numpy() for m in canon[e])  # noqa: E731
    with oracle_pool() as ex:
        yref, _, _ = O.moe(expert_of, lg.cpu().numpy(), x.cpu().numpy(), k=1, fixed_idx=fixed_np, map_fn=ex.map)
    e_or = O.rel_l2(np_of(yg), yref).max()               # every token, the last row of each tile included
    print(f"grouped GEMM partial tiles: vs items {e_gi:.3e}, vs oracle {e_or:.3e}")
    assert max(e_gi, e_or) <= REL_L2_BAR


def test_moe_grouped_items_equal_decode_bitwise(q, layer):
    # the grouped path's GEMV work items compute each token independently, so on a
    # decode-sized batch they must reproduce the decode path bit for bit
    seed, canon, tab = layer
    T = 48
    x = gen_x(seed, (2000, T), T, 4096, device=DEV)
    lg = gen_logits_normal(seed, (2000, T), T, 256, device=DEV)
    yd, idd, wd = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, flags=q.GALE_PATH_DECODE)
    yg, idg, wg = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6,
                                  flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_ITEMS)
    assert torch.equal(idd, idg) and torch.equal(wd, wg)
    assert torch.equal(yd, yg)


@pytest.mark.parametrize("tiles", [1, 2, 3])
def test_moe_one_launch_equals_staged_bitwise(q, layer, tiles):
    """One token: the one-launch layer kernel against the five-launch sequence, bit for
    bit, over consecutive calls on one workspace (the generation in its synchronisation
    words moves on from call to call)."""
    seed, canon, tab = layer
    ws = q.moe_workspace(q.moe_workspace_bytes(1, 256, 6, 4096, 2048), DEV)
    for i in range(4):
        print(f"one-launch decode tiles={tiles} call {i}", flush=True)
        x = gen_x(seed, (3000 + i,), 1, 4096, device=DEV)
        lg = gen_logits_normal(seed, (3000 + i,), 1, 256, device=DEV)
        yf, idf, wf = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, ws=ws, flags=q.gale_layer_tiles_flag(tiles))
        ys, ids, wss = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, flags=q.GALE_DECODE_STAGED)
        assert torch.equal(idf, ids) and torch.equal(wf, wss)
        assert torch.equal(yf, ys)
    st, words, _ = q.sync_status(ws)
    assert st == 0 and words[0] == 4 and words[2] == 0
    ridx, _ = O.route(lg.cpu().numpy(), 6)
    assert np.array_equal(idf.cpu().numpy(), ridx)
    expert_of = lambda e: tuple(m.numpy() for m in canon[e])  # noqa: E731
    yref, _, _ = O.moe(expert_of, lg.cpu().numpy(), x.cpu().numpy(), k=6)
    assert O.rel_l2(np_of(yf), yref).max() <= REL_L2_BAR


@pytest.mark.parametrize("fill", ["random", "bytes01", "bytesFF", "arange64", "ones_f32"])
def test_moe_one_launch_unzeroed_sync_words(q, layer, fill):
    """Synchronisation words that were never zeroed (leftover data of several kinds): the
    call computes nothing (y keeps its contents) and the status query says why; after
    gale_sync_init the calls equal the five-launch sequence bit for bit."""
    seed, canon, tab = layer
    n = q.moe_workspace_bytes(1, 256, 6, 4096, 2048)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    if fill == "random":
        ws.random_(0, 256)
    elif fill == "bytes01":
        ws.fill_(1)
    elif fill == "bytesFF":
        ws.fill_(255)
    elif fill == "arange64":
        ws.view(torch.int64)[:] = torch.arange(n // 8, dtype=torch.int64, device=DEV)
    else:
        ws.view(torch.float32)[:] = 1.0
    x = gen_x(seed, (3100,), 1, 4096, device=DEV)
    lg = gen_logits_normal(seed, (3100,), 1, 256, device=DEV)
    sentinel = torch.full((1, 4096), 7.0, dtype=torch.float16, device=DEV)
    yf, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, ws=ws, y=sentinel.clone())
    torch.cuda.synchronize()
    assert torch.equal(yf, sentinel)
    st, _, detail = q.sync_status(ws)
    assert st == q.GALE_ERR_SYNC and "never zeroed" in detail
    q.sync_init(ws)
    for i in range(2):
        xi = gen_x(seed, (3101 + i,), 1, 4096, device=DEV)
        lgi = gen_logits_normal(seed, (3101 + i,), 1, 256, device=DEV)
        yf, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lgi, xi, top_k=6, ws=ws)
        ys, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lgi, xi, top_k=6, flags=q.GALE_DECODE_STAGED)
        assert torch.equal(yf, ys)
    assert q.sync_status(ws)[0] == 0


def test_moe_one_launch_wait_give_up_is_reported(q, layer):
    """A call whose waits give up (forced from the host: a zero time budget; every kernel
    still ends) leaves the error bit set: the status query reports it and later calls
    compute nothing until gale_sync_init, after which the results are exact again."""
    seed, canon, tab = layer
    ws = q.moe_workspace(q.moe_workspace_bytes(1, 256, 6, 4096, 2048), DEV)
    x = gen_x(seed, (3200,), 1, 4096, device=DEV)
    lg = gen_logits_normal(seed, (3200,), 1, 256, device=DEV)
    q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, ws=ws, flags=q.GALE_SYNC_NO_WAIT)
    torch.cuda.synchronize()
    st, words, detail = q.sync_status(ws)
    assert st == q.GALE_ERR_SYNC and (words[2] & 1) and "gave up" in detail
    sentinel = torch.full((1, 4096), 3.0, dtype=torch.float16, device=DEV)
    yf, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, ws=ws, y=sentinel.clone())
    torch.cuda.synchronize()
    assert torch.equal(yf, sentinel)
    q.sync_init(ws)
    yf, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, ws=ws)
    ys, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, flags=q.GALE_DECODE_STAGED)
    assert torch.equal(yf, ys)
    assert q.sync_status(ws)[0] == 0


def test_moe_decode_stack_equals_layer_calls(q, layer):
    """One token through a stack of layers in one launch equals the five-launch sequence of
    each layer bit for bit: with independent inputs per layer, and chained (x of layer l + 1
    is y of layer l, which the stack may read only once every row of it is stored); two
    calls in a row on one workspace."""
    seed, canon, tab = layer
    L = 5
    xs = [gen_x(seed, (4000 + l,), 1, 4096, device=DEV) for l in range(L)]
    lgs = [gen_logits_normal(seed, (4000 + l,), 1, 256, device=DEV) for l in range(L)]
    ws = q.moe_workspace(q.decode_stack_workspace_bytes(4096, 2048, 6), DEV)
    for rep in range(2):
        ys = [torch.empty(1, 4096, dtype=torch.float16, device=DEV) for _ in range(L)]
        idx = [torch.empty(1, 6, dtype=torch.int32, device=DEV) for _ in range(L)]
        wts = [torch.empty(1, 6, dtype=torch.float32, device=DEV) for _ in range(L)]
        lt = q.layer_table([dict(experts=tab, logits=lgs[l], x=xs[l], y=ys[l], topk_idx=idx[l], topk_w=wts[l])
                            for l in range(L)])
        print(f"decode stack independent layers, call {rep}", flush=True)
        q.moe_decode_stack(4096, 2048, 256, 6, lt, ws=ws)
        for l in range(L):
            yr, ir, wr = q.moe_layer_fwd(tab, 4096, 2048, lgs[l], xs[l], top_k=6, flags=q.GALE_DECODE_STAGED)
            assert torch.equal(idx[l], ir) and torch.equal(wts[l], wr)
            assert torch.equal(ys[l], yr), l
    # chained: x of layer l + 1 = y of layer l (raw SwiGLU outputs grow from layer to layer, so
    # the chain is short and the outputs are compared as bit patterns)
    Lc = 3
    ych = [torch.empty(1, 4096, dtype=torch.float16, device=DEV) for _ in range(Lc)]
    lt = q.layer_table([dict(experts=tab, logits=lgs[l], x=xs[0] if l == 0 else ych[l - 1], y=ych[l])
                        for l in range(Lc)])
    print("decode stack chained layers", flush=True)
    q.moe_decode_stack(4096, 2048, 256, 6, lt, ws=ws)
    xr = xs[0]
    for l in range(Lc):
        yr, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lgs[l], xr, top_k=6, flags=q.GALE_DECODE_STAGED)
        print(f"chained layer {l}: max |y| {yr.float().abs().max().item():.3g}", flush=True)
        if l == 0:
            assert torch.isfinite(yr.float()).all()     # the next layer reads real values
        assert torch.equal(ych[l].view(torch.int16), yr.view(torch.int16)), l
        xr = yr
    assert q.sync_status(ws)[0] == 0


def test_moe_decode_stack_mixed_routing(q, layer):
    """A stack whose layers route in turn by plain top-k, with a selection bias, plain again,
    with fixed experts and plain again (a plain layer after another layer takes its logits
    loaded while that layer ends; the variants load theirs in the layer): every layer equals
    its own call (routing, weights, outputs bit for bit), and the routing matches the oracle."""
    seed, canon, tab = layer
    L = 5
    rng = np.random.default_rng(55)
    xs = [gen_x(seed, (4500 + l,), 1, 4096, device=DEV) for l in range(L)]
    lgs = [gen_logits_normal(seed, (4500 + l,), 1, 256, device=DEV) for l in range(L)]
    bias = torch.from_numpy((rng.standard_normal(256) * 0.5).astype(np.float32)).to(DEV)
    fixed = torch.from_numpy(rng.permutation(256)[:6].astype(np.int32)[None]).to(DEV)
    kws = [{}, {"select_bias": bias}, {}, {"fixed_idx": fixed}, {}]
    ys = [torch.empty(1, 4096, dtype=torch.float16, device=DEV) for _ in range(L)]
    idx = [torch.empty(1, 6, dtype=torch.int32, device=DEV) for _ in range(L)]
    wts = [torch.empty(1, 6, dtype=torch.float32, device=DEV) for _ in range(L)]
    lt = q.layer_table([dict(experts=tab, logits=lgs[l], x=xs[l], y=ys[l], topk_idx=idx[l], topk_w=wts[l], **kws[l])
                        for l in range(L)])
    ws = q.moe_workspace(q.decode_stack_workspace_bytes(4096, 2048, 6), DEV)
    print("decode stack, mixed routing", flush=True)
    q.moe_decode_stack(4096, 2048, 256, 6, lt, ws=ws)
    for l in range(L):
        yr, ir, wr = q.moe_layer_fwd(tab, 4096, 2048, lgs[l], xs[l], top_k=6, flags=q.GALE_DECODE_STAGED, **kws[l])
        assert torch.equal(idx[l], ir) and torch.equal(wts[l], wr), l
        assert torch.equal(ys[l], yr), l
        okw = {k: v.cpu().numpy() for k, v in kws[l].items()}
        ridx, rw = O.route(lgs[l].cpu().numpy(), 6, **okw)
        assert np.array_equal(idx[l].cpu().numpy(), ridx), l
        assert np.abs(wts[l].cpu().numpy() - rw).max() <= 1e-6
    assert q.sync_status(ws)[0] == 0


def test_moe_one_launch_top_k_and_outlier_edges(q):
    """One token through experts whose rows carry 0, 1, 300 (past the staged outlier
    chunks) or 41 / 20 outliers, with top_k 1, 8 and 3 in turn on one workspace (the
    counter layout moves with top_k): equal to the staged sequence and to the oracle."""
    E = 8
    seed = config_seed(13)
    experts_np, packed = [], []
    for e in range(E):
        d1, d3, d2 = outlier_edge_dict(2048, 4096, 200 + e), outlier_edge_dict(2048, 4096, 300 + e), \
            outlier_edge_dict(4096, 2048, 400 + e)
        experts_np.append((d1, d3, d2))
        packed.append(tuple(q.pack_matrix(canon_from_dict(d)) for d in (d1, d3, d2)))
    tab = q.expert_table(packed)
    ws = q.moe_workspace(q.moe_workspace_bytes(1, E, 8, 4096, 2048), DEV)
    for i, k in enumerate([1, 8, 3]):
        print(f"one-launch decode edges top_k={k}", flush=True)
        x = gen_x(seed, (10 + i,), 1, 4096, device=DEV)
        lg = gen_logits_normal(seed, (10 + i,), 1, E, device=DEV)
        yf, idf, wf = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=k, ws=ws)
        ys, ids, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=k, flags=q.GALE_DECODE_STAGED)
        assert torch.equal(idf, ids) and torch.equal(yf, ys)
        yref, ridx, _ = O.moe(lambda e: experts_np[e], lg.cpu().numpy(), x.cpu().numpy(), k=k)
        assert np.array_equal(idf.cpu().numpy(), ridx)
        err = O.rel_l2(np_of(yf), yref).max()
        print(f"one-launch decode edges top_k={k} rel-L2 {err:.3e}")
        assert err <= REL_L2_BAR


@pytest.mark.parametrize("T,zipf", [(65, False), (2048, True)])
def test_moe_grouped_prefill(q, layer, T, zipf):
    """Grouped path (tile GEMM for the busy experts, GEMV items for the rest) at a ragged
    size just past the decode limit and at the prefill workload (2048 tokens,
    Zipf(1.1)-skewed top-6 of 256): routing exact for every token, EVERY token against the
    oracle (the oracle dequantizes each touched expert once and runs all its tokens), the
    all-items and all-GEMM variants against the oracle too, and run-to-run determinism."""
    seed, canon, tab = layer
    x = gen_x(seed, (3000, T), T, 4096, device=DEV)
    gen = gen_logits_zipf if zipf else gen_logits_normal
    lg = gen(seed, (3000, T), T, 256, device=DEV)
    y, idx, w = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6)
    y2, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6)
    assert torch.equal(y, y2)
    ridx, rw = O.route(lg.cpu().numpy(), 6)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    counts = np.bincount(ridx.ravel(), minlength=256)
    # every expert through the items path, and every expert through the tile GEMM
    yi, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_ITEMS)
    yg, _, _ = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_GEMM)
    torch.cuda.synchronize()
    expert_of = lambda e: tuple(m.numpy() for m in canon[e])  # noqa: E731
    with oracle_pool() as ex:
        yref, _, _ = O.moe(expert_of, lg.cpu().numpy(), x.cpu().numpy(), k=6, map_fn=ex.map)
    err = O.rel_l2(np_of(y), yref)
    err_items = O.rel_l2(np_of(yi), yref)
    err_gemm = O.rel_l2(np_of(yg), yref)
    print(f"grouped T={T} max expert load {counts.max()}: rel-L2 vs oracle over all {T} tokens: hybrid "
          f"{err.max():.3e} (median {np.median(err):.3e}), items {err_items.max():.3e}, GEMM {err_gemm.max():.3e}")
    assert err.max() <= REL_L2_BAR and err_items.max() <= REL_L2_BAR and err_gemm.max() <= REL_L2_BAR


def outlier_edge_dict(N, K, seed):
    """Random signs and block scales; outliers per row cycling through 0, 1, 300 and
    round(0.01 K), one row with columns 0 and K - 1 only."""
    rng = np.random.default_rng(seed)
    rp, cols, vals = [0], [], []
    for n in range(N):
        cnt = [0, 1, 300, int(0.01 * K + 0.5)][n % 4]
        cs = np.sort(rng.choice(K, size=cnt, replace=False)) if cnt else np.zeros(0, dtype=np.int64)
        if n == 5:
            cs = np.array([0, K - 1])
        cols.extend(cs.tolist())
        vals.extend(rng.integers(-8, 8, size=len(cs)).tolist())
        rp.append(len(cols))
    nib = [v & 0xF for v in vals] + ([0] if len(vals) % 2 else [])
    return {"rows": N, "cols": K, "signs": rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32),
            "block_scales": (np.abs(rng.standard_normal((N, K // 128))) * 0.02).astype(np.float16),
            "row_scales": np.full(N, 0.05, dtype=np.float16), "row_ptr": np.array(rp),
            "out_cols": np.array(cols, dtype=np.uint16),
            "out_vals": np.array([nib[i] | (nib[i + 1] << 4) for i in range(0, len(nib), 2)], dtype=np.uint8)}


def test_moe_grouped_gemm_outlier_edges(q):
    # w2 rows carry 0, 1, 300 or 20 outliers (too many for the GEMM's LDS staging, so
    # the tiles read them from HBM); w1/w3 are standard (staged); tiles partly filled
    E, T = 4, 80
    seed = config_seed(12)
    w13 = gen_matrices(seed, [(e, m) for e in range(E) for m in (0, 1)], 2048, 4096)
    experts_np, packed = [], []
    for e in range(E):
        d2 = outlier_edge_dict(4096, 2048, 100 + e)
        m1, m3 = w13[2 * e], w13[2 * e + 1]
        experts_np.append((m1.numpy(), m3.numpy(), d2))
        packed.append((q.pack_matrix(m1.to(DEV)), q.pack_matrix(m3.to(DEV)), q.pack_matrix(canon_from_dict(d2))))
    tab = q.expert_table(packed)
    x = gen_x(seed, (1,), T, 4096, device=DEV)
    lg = gen_logits_normal(seed, (2,), T, E, device=DEV)
    y, idx, w = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=2, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_GEMM)
    yref, ridx, _ = O.moe(lambda e: experts_np[e], lg.cpu().numpy(), x.cpu().numpy(), k=2)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    err = O.rel_l2(np_of(y), yref).max()
    print(f"grouped GEMM outlier edges rel-L2 {err:.3e}")
    assert err <= REL_L2_BAR


def test_moe_grouped_gemm_hidden_8192(q):
    # hidden 8192 (64 scale blocks): past the GEMM's bucket table, so its tiles walk the CSR
    # lists in HBM; the GEMV items run 16 wavefronts per workgroup.  GEMM and items against
    # each other and against the oracle on every token.
    E, T, H, I = 2, 80, 8192, 2048
    seed = config_seed(13)
    w13 = gen_matrices(seed, [(e, m) for e in range(E) for m in (0, 1)], I, H)
    w2 = gen_matrices(seed, [(e, 2) for e in range(E)], H, I)
    canon = [(w13[2 * e], w13[2 * e + 1], w2[e]) for e in range(E)]
    tab = q.expert_table([tuple(q.pack_matrix(m.to(DEV)) for m in ex) for ex in canon])
    x = gen_x(seed, (1,), T, H, device=DEV)
    lg = gen_logits_normal(seed, (2,), T, E, device=DEV)
    yg, idx, _ = q.moe_layer_fwd(tab, H, I, lg, x, top_k=1, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_GEMM)
    yi, _, _ = q.moe_layer_fwd(tab, H, I, lg, x, top_k=1, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_ITEMS)
    with oracle_pool() as ex:
        yref, ridx, _ = O.moe(lambda e: tuple(m.numpy() for m in canon[e]), lg.cpu().numpy(), x.cpu().numpy(),
                              k=1, map_fn=ex.map)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    e_or = O.rel_l2(np_of(yg), yref).max()
    e_oi = O.rel_l2(np_of(yi), yref).max()
    e_gi = O.rel_l2(np_of(yg), np_of(yi)).max()
    print(f"grouped GEMM hidden 8192: vs oracle {e_or:.3e} (items {e_oi:.3e}), vs items {e_gi:.3e}")
    assert max(e_or, e_oi, e_gi) <= REL_L2_BAR


@pytest.mark.parametrize("T", [1, 4])
def test_moe_decode_hidden_8192(q, T):
    # the decode path at hidden 8192: the five-launch sequence (the one-launch layer takes
    # hidden <= 4096), gate/up workgroups of 16 wavefronts
    E, H, I = 8, 8192, 2048
    seed = config_seed(14)
    w13 = gen_matrices(seed, [(e, m) for e in range(E) for m in (0, 1)], I, H)
    w2 = gen_matrices(seed, [(e, 2) for e in range(E)], H, I)
    canon = [(w13[2 * e], w13[2 * e + 1], w2[e]) for e in range(E)]
    tab = q.expert_table([tuple(q.pack_matrix(m.to(DEV)) for m in ex) for ex in canon])
    x = gen_x(seed, (1, T), T, H, device=DEV)
    lg = gen_logits_normal(seed, (2, T), T, E, device=DEV)
    y, idx, _ = q.moe_layer_fwd(tab, H, I, lg, x, top_k=2)
    yref, ridx, _ = O.moe(lambda e: tuple(m.numpy() for m in canon[e]), lg.cpu().numpy(), x.cpu().numpy(), k=2)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    err = O.rel_l2(np_of(y), yref).max()
    print(f"decode hidden 8192 T={T}: rel-L2 {err:.3e}")
    assert err <= REL_L2_BAR


def clustered_outlier_dict(N, K, seed):
    """Random signs and block scales; every row has 12 outliers in its first 128 columns
    and 2 in its last 128, so a group of 16 rows holds 192 entries in block 0."""
    rng = np.random.default_rng(seed)
    rp, cols, vals = [0], [], []
    for n in range(N):
        cs = np.concatenate([np.sort(rng.choice(128, size=12, replace=False)),
                             K - 128 + np.sort(rng.choice(128, size=2, replace=False))])
        cols.extend(cs.tolist())
        vals.extend(rng.integers(-8, 8, size=len(cs)).tolist())
        rp.append(len(cols))
    nib = [v & 0xF for v in vals] + ([0] if len(vals) % 2 else [])
    return {"rows": N, "cols": K, "signs": rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32),
            "block_scales": (np.abs(rng.standard_normal((N, K // 128))) * 0.02).astype(np.float16),
            "row_scales": np.full(N, 0.05, dtype=np.float16), "row_ptr": np.array(rp),
            "out_cols": np.array(cols, dtype=np.uint16),
            "out_vals": np.array([nib[i] | (nib[i + 1] << 4) for i in range(0, len(nib), 2)], dtype=np.uint8)}


def test_moe_grouped_gemm_dense_buckets(q):
    # w1 and w2 rows carry their outliers in the first and last blocks: staged, with
    # more than 64 entries in one (row group, block) bucket
    E, T = 3, 70
    seed = config_seed(13)
    w3s = gen_matrices(seed, [(e, 1) for e in range(E)], 2048, 4096)
    experts_np, packed = [], []
    for e in range(E):
        d1 = clustered_outlier_dict(2048, 4096, 200 + e)
        d2 = clustered_outlier_dict(4096, 2048, 300 + e)
        m3 = w3s[e]
        experts_np.append((d1, m3.numpy(), d2))
        packed.append((q.pack_matrix(canon_from_dict(d1)), q.pack_matrix(m3.to(DEV)), q.pack_matrix(canon_from_dict(d2))))
    tab = q.expert_table(packed)
    x = gen_x(seed, (1,), T, 4096, device=DEV)
    lg = gen_logits_normal(seed, (2,), T, E, device=DEV)
    y, idx, w = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=2, flags=q.GALE_PATH_GROUPED | q.GALE_GROUPED_GEMM)
    yref, ridx, _ = O.moe(lambda e: experts_np[e], lg.cpu().numpy(), x.cpu().numpy(), k=2)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    err = O.rel_l2(np_of(y), yref).max()
    print(f"grouped GEMM dense outlier buckets rel-L2 {err:.3e}")
    assert err <= REL_L2_BAR


def test_moe_closed_form(q):
    E = 16
    w1 = q.pack_matrix(canon_from_dict(hadamard_sign_dict(2048, 4096)))
    base2 = hadamard_sign_dict(4096, 2048)
    experts = []
    for e in range(E):
        d = dict(base2)
        d["block_scales"] = (base2["block_scales"].astype(np.float64) * (1.0 + e / 256.0)).astype(np.float16)
        experts.append((w1, w1, q.pack_matrix(canon_from_dict(d))))
    tab = q.expert_table(experts)
    x = gen_x(config_seed(9), (0,), 3, 4096, device=DEV) * 0.25
    lg = gen_logits_normal(config_seed(9), (0,), 3, E, device=DEV)
    y, idx, w = q.moe_layer_fwd(tab, 4096, 2048, lg, x, top_k=6)
    xs = np_of(x)[:, :2048]
    coef = (w.cpu().numpy().astype(np.float64) * (1.0 + idx.cpu().numpy() / 256.0)).sum(axis=1)
    ref = np.zeros((3, 4096))
    ref[:, :2048] = coef[:, None] * xs * xs / (1 + np.exp(-xs))
    assert O.rel_l2(np_of(y), ref).max() <= 1e-3


@pytest.mark.gpu
@pytest.mark.parametrize("n_bytes,sink_words", [(16, 1), (1 << 20, 64), ((1 << 20) + 48, 4096)])
def test_read_stream_reads_every_word(q, n_bytes, sink_words):
    """The streaming-read diagnostic reads every 16-byte granule once: the XOR of its per-workgroup
    words equals the XOR of all 32-bit words of the buffer."""
    g = torch.Generator().manual_seed(n_bytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_bytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = host.to(DEV)
    sink = torch.zeros(sink_words, dtype=torch.int32, device=DEV)
    rc = q.lib().gale_read_stream(buf.data_ptr(), n_bytes, sink.data_ptr(), sink_words,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    grid = min((n_bytes // 16 + 255) // 256, sink_words)
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(sink[:grid].cpu().numpy().view(np.uint32)))
    assert got == want
