"""The entry point that allocates nothing (gale_moe_decode_stack_static: its workspace is a
library-owned device array per GPU) against gale_moe_decode_stack on a caller workspace, bit for
bit, on two calls in a row (the second smaller), through the C ABI."""
import numpy as np
import pytest
import torch

from synth import config_seed, gen_logits_normal, gen_matrices, gen_x

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_expert_gemv_amd as qq
    qq.lib()
    return qq


def _experts(q, seed, E):
    w13 = gen_matrices(seed, [(e, m) for e in range(E) for m in (0, 1)], 2048, 4096, device=DEV)
    w2 = gen_matrices(seed, [(e, 2) for e in range(E)], 4096, 2048, device=DEV)
    return q.expert_table([(q.pack_matrix(w13[2 * e]), q.pack_matrix(w13[2 * e + 1]), q.pack_matrix(w2[e]))
                           for e in range(E)])


def _layers(q, tab, seed, L, k, tag):
    recs = []
    for l in range(L):
        recs.append(dict(experts=tab, logits=gen_logits_normal(seed, (tag, l), 1, 16, device=DEV),
                         x=gen_x(seed, (tag, l), 1, 4096, device=DEV),
                         y=torch.full((1, 4096), 5.0, dtype=torch.float16, device=DEV),
                         topk_idx=torch.full((1, k), -1, dtype=torch.int32, device=DEV),
                         topk_w=torch.zeros(1, k, dtype=torch.float32, device=DEV)))
    return recs


def test_static_entry_equals_workspace_entry(q):
    seed = config_seed(21)
    tab = _experts(q, seed, 16)
    lib = q.lib()
    st = torch.cuda.current_stream().cuda_stream
    for L, k, tag in ((5, 6, 500), (3, 4, 600)):          # the second call is smaller
        print(f"static-scratch decode stack: {L} layers, top-{k}", flush=True)
        a = _layers(q, tab, seed, L, k, tag)
        b = _layers(q, tab, seed, L, k, tag)
        ta, tb = q.layer_table(a), q.layer_table(b)
        rc = lib.gale_moe_decode_stack_static(4096, 2048, 16, k, L, ta.ptr(), 0, st)
        assert rc == 0, lib.gale_last_error().decode()
        q.moe_decode_stack(4096, 2048, 16, k, tb)
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(a[l]["topk_idx"], b[l]["topk_idx"]) and torch.equal(a[l]["topk_w"], b[l]["topk_w"])
            assert torch.equal(a[l]["y"], b[l]["y"]), (L, k, l)
            assert not torch.equal(a[l]["y"], torch.full_like(a[l]["y"], 5.0))   # written


def test_static_entry_rejects_oversize():
    import quantized_expert_gemv_amd as qq
    lib = qq.lib()
    fake = 1 << 40                                      # never dereferenced: rejected on the host
    # top-6 of an intermediate size of 3072 needs 40,960 + 73,728 + 148,992 workspace bytes
    assert lib.gale_moe_decode_stack_static(4096, 3072, 16, 6, 2, fake, 0, None) == -5
    assert b"static array" in lib.gale_last_error()
