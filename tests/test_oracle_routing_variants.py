"""Pins of the oracle's routing variants (CPU): the selection bias of DeepSeek's balancing
term (DeepSeek-V4-Pro GALE page, serving notes on the tier bias: it moves the choice, never
the weights) and hash routing from a token-to-expert table (DeepSeek-V4-Flash 180B REAP
card, lineage notes), each checked against closed forms and brute force."""
import itertools

import numpy as np

import oracle as O


def softmax(v):
    """fp64 softmax of fp32 logits (the values the routing sees)."""
    v = np.asarray(np.asarray(v, dtype=np.float32), dtype=np.float64)
    e = np.exp(v - v.max())
    return e / e.sum()


def test_zero_bias_is_plain_routing():
    lg = np.random.default_rng(3).standard_normal((9, 40)).astype(np.float32)
    a = O.route(lg, 6)
    b = O.route(lg, 6, select_bias=np.zeros(40, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bias_moves_the_choice_not_the_weights():
    # logits 1.0, 0.9, 0.5: plain top-2 is (0, 1); a bias of 0.2 on expert 1 puts it first
    # (1.1 > 1.0), and the weights stay softmax(0.9, 1.0) in slot order
    lg = np.array([[1.0, 0.9, 0.5]], dtype=np.float32)
    idx, w = O.route(lg, 2, select_bias=np.array([0.0, 0.2, 0.0], np.float32))
    assert idx.tolist() == [[1, 0]]
    assert np.allclose(w[0], softmax([0.9, 1.0]), rtol=0, atol=1e-15)
    # a bias that brings expert 2 into the top-2 gives it the weight of its own logit
    idx, w = O.route(lg, 2, select_bias=np.array([0.0, 0.0, 0.45], np.float32))
    assert idx.tolist() == [[0, 2]]                  # 0.95 > 0.9
    assert np.allclose(w[0], softmax([1.0, 0.5]), rtol=0, atol=1e-15)


def test_bias_ties_go_to_the_lower_index_on_fp32_sums():
    # 0.25 + 0.5 and 0.5 + 0.25 are the same fp32 number: the lower index ranks first
    lg = np.array([[0.25, 0.5, 0.0]], dtype=np.float32)
    idx, _ = O.route(lg, 2, select_bias=np.array([0.5, 0.25, 0.0], np.float32))
    assert idx.tolist() == [[0, 1]]


def test_large_negative_bias_excludes_an_expert():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((20, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    bias[int(np.argmax(lg[0]))] = -1e30
    idx, _ = O.route(lg, 4, select_bias=bias)
    assert not (idx == int(np.argmax(lg[0]))).any()


def test_bias_choice_matches_brute_force():
    rng = np.random.default_rng(7)
    E, k = 7, 3
    for _ in range(20):
        lg = rng.standard_normal((1, E)).astype(np.float32)
        bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
        score = lg[0] + bias
        best = max(itertools.combinations(range(E), k), key=lambda c: sorted(score[list(c)].tolist(), reverse=True))
        idx, w = O.route(lg, k, select_bias=bias)
        assert sorted(idx[0].tolist()) == sorted(best)
        assert np.allclose(w[0], softmax(lg[0, idx[0]]), rtol=0, atol=1e-15)


def test_fixed_experts_take_their_own_logits_in_slot_order():
    lg = np.array([[0.1, 2.0, -1.0, 0.7]], dtype=np.float32)
    idx, w = O.route(lg, 3, fixed_idx=np.array([[2, 0, 3]]))
    assert idx.tolist() == [[2, 0, 3]]
    assert np.allclose(w[0], softmax([-1.0, 0.1, 0.7]), rtol=0, atol=1e-15)
    assert abs(w.sum() - 1.0) < 1e-15


def test_moe_with_the_routers_own_choice_as_table_is_plain_moe():
    # hash routing that happens to pick the router's own top-k reproduces the plain layer
    from synth import config_seed, gen_logits_normal, gen_matrix, gen_x
    seed = config_seed(30)
    E, k, H, I = 5, 2, 1024, 1024
    mats = {e: tuple(gen_matrix(seed, (e, m), r, c).numpy() for m, r, c in ((0, I, H), (1, I, H), (2, H, I)))
            for e in range(E)}
    lg = gen_logits_normal(seed, (1,), 3, E).numpy()
    x = gen_x(seed, (2,), 3, H).numpy()
    y, idx, w = O.moe(lambda e: mats[e], lg, x, k=k)
    y2, idx2, w2 = O.moe(lambda e: mats[e], lg, x, k=k, fixed_idx=idx)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2) and np.array_equal(y, y2)
    # and a bias that cannot change the order changes nothing
    y3, idx3, _ = O.moe(lambda e: mats[e], lg, x, k=k, select_bias=np.full(E, 0.5, np.float32))
    assert np.array_equal(idx, idx3) and np.array_equal(y, y3)
