"""The whole resident stack of the benchmark against the fp64 oracle.

43 layers x 256 experts x {w1, w3, w2} (33,024 packed matrices, 46.0 GB in HBM, the
DeepSeek-V4-Flash GALE card's "What is in the pack" shapes) run through one
gale_moe_decode_stack launch with an independent seeded token per layer, in the launch
configuration the benchmark times.  Every layer's routing must equal the oracle's exactly and
every layer's output must be within the parity bar of the oracle's route + six FFNs + combine
(each touched expert dequantized once by the oracle).
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import config_seed, gen_logits_normal, gen_x

from tests.test_gpu_parity import REL_L2_BAR, oracle_pool

pytestmark = pytest.mark.gpu

HIDDEN, INTER, EXPERTS, TOPK, LAYERS = 4096, 2048, 256, 6, 43


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_expert_gemv_amd as qq
    qq.lib()
    return qq


def test_full_stack_one_launch_against_oracle(q):
    import bench
    dev = torch.device("cuda:0")
    seed = config_seed(4)
    print("building the 43-layer resident stack", flush=True)
    tables, _ = bench.build_stack(q, synth, LAYERS, seed, dev)
    xs = [gen_x(seed, (0x10000 + l,), 1, HIDDEN, device=dev) for l in range(LAYERS)]
    lgs = [gen_logits_normal(seed, (0x20000 + l,), 1, EXPERTS, device=dev) for l in range(LAYERS)]
    ys = [torch.empty(1, HIDDEN, dtype=torch.float16, device=dev) for _ in range(LAYERS)]
    idx = [torch.empty(1, TOPK, dtype=torch.int32, device=dev) for _ in range(LAYERS)]
    wts = [torch.empty(1, TOPK, dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    lt = q.layer_table([dict(experts=tables[l], logits=lgs[l], x=xs[l], y=ys[l], topk_idx=idx[l], topk_w=wts[l])
                        for l in range(LAYERS)])
    ws = q.moe_workspace(q.decode_stack_workspace_bytes(HIDDEN, INTER, TOPK), dev)
    print("one launch through 43 layers", flush=True)
    q.moe_decode_stack(HIDDEN, INTER, EXPERTS, TOPK, lt, ws=ws)
    torch.cuda.synchronize()
    assert q.sync_status(ws)[0] == 0

    lg_np = [lg.cpu().numpy() for lg in lgs]
    x_np = [x.float().cpu().numpy().astype(np.float64) for x in xs]
    touched = {}
    for l in range(LAYERS):
        ridx, rw = O.route(lg_np[l], TOPK)
        assert np.array_equal(idx[l].cpu().numpy(), ridx), l
        assert np.abs(wts[l].cpu().numpy() - rw).max() <= 1e-6, l
        for e in ridx[0]:
            touched[(l, int(e))] = tuple(
                synth.gen_matrix(seed, (l, int(e), m), r, c, device=dev).numpy()
                for m, (r, c) in enumerate([(INTER, HIDDEN), (INTER, HIDDEN), (HIDDEN, INTER)]))
    del tables
    torch.cuda.empty_cache()
    print(f"oracle over {len(touched)} touched experts", flush=True)

    def layer_ref(l):
        return O.moe(lambda e: touched[(l, e)], lg_np[l], x_np[l], k=TOPK)[0]

    with oracle_pool() as ex:
        refs = list(ex.map(layer_ref, range(LAYERS)))
    errs = [float(O.rel_l2(ys[l].float().cpu().numpy().astype(np.float64), refs[l]).max()) for l in range(LAYERS)]
    print(f"43-layer stack: max rel-L2 {max(errs):.3e} (layer {int(np.argmax(errs))})", flush=True)
    assert max(errs) <= REL_L2_BAR
