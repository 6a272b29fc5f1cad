"""Pins of the oracle's router (page "Thinking Machines首發大模型：9750億參數，
完整開放權重", section "架構": sigmoid scores, a selection-only load-balancing
bias, the chosen scores normalized into weights) against an independent numpy
formulation and hand cases."""
import numpy as np

import oracle


def _numpy_router(logits, bias, k):
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    key = s + bias.astype(np.float64)[None, :]
    ids = np.argsort(-key, axis=1, kind="stable")[:, :k]      # stable: the lower index wins a tie
    sel = np.take_along_axis(s, ids, axis=1)
    return ids.astype(np.int32), sel / sel.sum(axis=1, keepdims=True)


def test_router_matches_numpy():
    g = np.random.default_rng(301)
    for T, E, k in ((50, 8, 2), (33, 384, 8), (7, 256, 6), (5, 17, 17)):
        logits = g.standard_normal((T, E)).astype(np.float32)
        bias = (0.3 * g.standard_normal(E)).astype(np.float32)
        ids, w = oracle.router_sigmoid_topk(logits, bias, k)
        ids_n, w_n = _numpy_router(logits, bias, k)
        assert np.array_equal(ids, ids_n)
        assert np.allclose(w, w_n, rtol=1e-15, atol=0)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-15)


def test_router_bias_steers_the_choice_not_the_weights():
    logits = np.zeros((1, 4), np.float32)                       # every score 1/2
    bias = np.array([0.0, 0.1, 0.0, 0.2], np.float32)
    ids, w = oracle.router_sigmoid_topk(logits, bias, 2)
    assert ids.tolist() == [[3, 1]]
    assert w.tolist() == [[0.5, 0.5]]                           # plain scores, normalized
    # keys 0.881, 0.6, 0.5, 0.469: expert 0, then 1 (its bias lifts it above expert 2)
    logits = np.array([[2.0, 0.0, 0.0, -1.0]], np.float32)
    ids, w = oracle.router_sigmoid_topk(logits, bias, 2)
    s = 1.0 / (1.0 + np.exp(-logits[0].astype(np.float64)))
    assert ids.tolist() == [[0, 1]]
    assert np.allclose(w[0], [s[0] / (s[0] + s[1]), s[1] / (s[0] + s[1])], rtol=1e-15)


def test_router_ties_and_full_selection():
    ids, w = oracle.router_sigmoid_topk(np.zeros((2, 6), np.float32), np.zeros(6, np.float32), 3)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]              # equal keys: lower index first
    assert np.allclose(w, 1.0 / 3.0, rtol=1e-15)
    g = np.random.default_rng(302)
    logits = g.standard_normal((4, 9)).astype(np.float32)
    ids, w = oracle.router_sigmoid_topk(logits, np.zeros(9, np.float32), 9)
    for row, l in zip(ids, logits):
        assert sorted(row.tolist()) == list(range(9))          # k = E: a permutation
        assert np.all(np.diff(l[row]) <= 0)                     # in descending score order
