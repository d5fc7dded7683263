"""Pins of the oracle's router: logits against a float64 library matmul,
selection against a brute-force full sort, the exact-tie rule driven through
the real route path, and the softmax gates against closed forms."""
import numpy as np
import pytest


def _brute_topk(l, k):
    """Full stable sort by (descending logit, ascending index)."""
    order = np.lexsort((np.arange(l.shape[0]), -l.astype(np.float64)))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (8, 8), (128, 8), (256, 8), (5, 3)])
def test_selection_matches_full_sort(orc, E, k):
    rng = np.random.default_rng([E, k])
    H, T = 64, 7
    W = rng.normal(0, 0.05, (E, H)).astype(np.float32)
    b = rng.normal(0, 1, E).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    idx, gates, logits, margin = orc.route_topk(x, W, b, k)
    ref = (x.astype(np.float64) @ W.T.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    assert np.array_equal(logits, ref)
    for t in range(T):
        assert list(idx[t]) == list(_brute_topk(logits[t], k))
        srt = np.sort(logits[t].astype(np.float64))[::-1]
        exp_margin = srt[k - 1] - srt[k] if k < E else np.inf
        assert margin[t] == np.float32(exp_margin)


def _one_hot_route(orc, logits_wanted, k, H=16):
    """Drive chosen logits through the real route path: x = e_0 and
    W_r[:, 0] = the wanted logits, so every logit is one exact product."""
    l = np.asarray(logits_wanted, dtype=np.float32)
    W = np.zeros((l.shape[0], H), dtype=np.float32)
    W[:, 0] = l
    x = np.zeros((1, H), dtype=np.float32)
    x[0, 0] = 1.0
    return orc.route_topk(x, W, None, k)


def test_all_equal_logits_take_lowest_indices(orc):
    idx, gates, logits, _ = _one_hot_route(orc, [0.25] * 16, 8)
    assert list(idx[0]) == list(range(8))
    assert np.all(gates[0] == np.float32(1 / 8))


def test_tie_across_the_boundary(orc):
    # experts 3 and 9 tie for the last slot: the lower index (3) is chosen
    l = [0.0] * 12
    l[1], l[5], l[3], l[9] = 2.0, 1.5, 0.75, 0.75
    idx, _, _, margin = _one_hot_route(orc, l, 3)
    assert list(idx[0]) == [1, 5, 3]
    assert margin[0] == 0.0


def test_tie_order_inside_the_selection(orc):
    l = [0.5, 1.0, 0.5, 1.0, -1.0, 1.0]
    idx, gates, _, _ = _one_hot_route(orc, l, 4)
    assert list(idx[0]) == [1, 3, 5, 0]
    assert gates[0][0] == gates[0][1] == gates[0][2]


def test_signed_zero_is_a_tie(orc):
    l = [-1.0, -0.0, 0.0, -0.0, -2.0]
    idx, gates, _, _ = _one_hot_route(orc, l, 2)
    assert list(idx[0]) == [1, 2]
    assert gates[0][0] == gates[0][1] == np.float32(0.5)


def test_k1_gate_is_exactly_one(orc):
    rng = np.random.default_rng(11)
    W = rng.normal(0, 0.05, (128, 64)).astype(np.float32)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    _, gates, _, _ = orc.route_topk(x, W, None, 1)
    assert np.all(gates == 1.0)


def test_two_expert_gates_are_a_logistic(orc):
    # softmax over two logits a > b is 1 / (1 + e^(b - a)) and its complement
    a, b = 1.25, -0.5
    idx, gates, _, _ = _one_hot_route(orc, [b, a, -3.0], 2)
    assert list(idx[0]) == [1, 0]
    g0 = 1.0 / (1.0 + np.exp(b - a))
    assert abs(gates[0][0] - g0) <= 1e-7 and abs(gates[0][1] - (1 - g0)) <= 1e-7


def test_gates_sum_to_one_and_descend(orc):
    rng = np.random.default_rng(12)
    W = rng.normal(0, 0.05, (256, 128)).astype(np.float32)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    idx, gates, logits, _ = orc.route_topk(x, W, None, 8)
    assert np.all(np.abs(gates.astype(np.float64).sum(1) - 1.0) <= 1e-6)
    assert np.all(np.diff(gates, axis=1) <= 0)
    for t in range(16):
        sel = logits[t][idx[t]].astype(np.float64)
        z = np.exp(sel - sel.max())
        assert np.allclose(gates[t], z / z.sum(), rtol=1e-6, atol=1e-7)


def test_bias_alone_sets_the_logits(orc):
    b = np.array([0.3, -1.0, 2.5, 0.3, 7.0], dtype=np.float32)
    W = np.ones((5, 8), dtype=np.float32)
    idx, _, logits, _ = orc.route_topk(np.zeros((1, 8), dtype=np.float32), W, b, 3)
    assert np.array_equal(logits[0], b)
    assert list(idx[0]) == [4, 2, 0]


def test_non_finite_logit_is_rejected(orc):
    import oracle
    W = np.full((4, 8), 3e38, dtype=np.float32)
    x = np.full((1, 8), 10.0, dtype=np.float32)
    with pytest.raises(oracle.OracleError):
        orc.route_topk(x, W, None, 2)
