"""The seeded generator: counter-based bits match the reference definition, any matrix
regenerates on its own, and the draws have the stated structure (CPU only)."""
import numpy as np
import torch

import synth
from synth import gen as G


def test_mix64_tensor_matches_python_int():
    key = G.stream_key(G.config_seed(1), 3, 4)
    idx = torch.arange(1000, dtype=torch.int64)
    got = G.bits64(key, idx).numpy().view(np.uint64)
    ref = [G.mix64_int(key + (i + 1) * G.GOLDEN) for i in range(1000)]
    assert [int(v) for v in got] == ref


def test_single_matrix_regenerates_identically():
    seed = G.config_seed(4)
    bulk = G.gen_matrices(seed, [(0, 0, 0), (0, 5, 2), (1, 7, 1)], 64, 2048)
    one = G.gen_matrix(seed, (0, 5, 2), 64, 2048)
    for f in ("signs", "block_scales", "row_scales", "row_ptr", "out_cols", "out_vals"):
        assert torch.equal(getattr(bulk[1], f), getattr(one, f))
    assert not torch.equal(bulk[0].signs, bulk[1].signs)


def test_distinct_uniform_columns():
    keys = G.bits64(12345, torch.arange(4000, dtype=torch.int64))
    c = G._distinct_uniform(keys, 41, 4096)
    assert c.shape == (4000, 41)
    assert bool((c[:, 1:] > c[:, :-1]).all())
    assert int(c.min()) >= 0 and int(c.max()) < 4096
    hist = torch.bincount(c.flatten(), minlength=4096).float()
    assert abs(hist.mean().item() - 4000 * 41 / 4096) < 1e-3
    assert hist.std().item() < 8.0           # ~ sqrt(40) for a uniform draw


def test_x_spikes_and_logits():
    x = G.gen_x(G.config_seed(1), (0,), 3, 4096).float()
    big = (x.abs() > 6.0).sum(dim=1)
    assert bool((big <= 4).all()) and int(big.sum()) >= 3
    lg = G.gen_logits_normal(G.config_seed(3), (0,), 64, 256)
    assert abs(lg.mean().item()) < 0.02 and abs(lg.std().item() - 1.0) < 0.02
    z = G.gen_logits_zipf(G.config_seed(5), (0,), 512, 256)
    counts = torch.bincount(z.topk(6, dim=1).indices.flatten(), minlength=256)
    assert int(counts.max()) > 20 * max(1, int(counts.median()))
