"""Pins of the oracle's routers against the pages' worked example, closed forms
and brute force (no GPU).

Softmax top-k [BAGEL, the commit moving the MoE router top-K to the GPU]; the
DeepSeek V4 sqrtsoftplus router [GGUF, the DeepSeek V4 routing scoring
commit]."""
import itertools
import math
import os

import numpy as np

import oracle


def _golden(name):
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", name)):
        if line.strip() and not line.startswith("#"):
            key, *vals = line.split()
            rows[key] = vals
    return rows


def test_softmax_router_worked_example():
    # tests/golden/router_topk.txt: logits (1, 5, 3, 4) at k = 2 select experts
    # 1 and 3, the weights sum to 1 and the larger logit gets the larger weight.
    g = _golden("router_topk.txt")
    logits = np.array([[float(v) for v in g["logits"]]])
    ids, w = oracle.router_topk_softmax(logits, int(g["k"][0]))
    assert sorted(ids[0].tolist()) == sorted(int(v) for v in g["experts"])
    assert abs(w.sum() - float(g["weight_sum"][0])) < 1e-15
    assert w[0][list(ids[0]).index(1)] > w[0][list(ids[0]).index(3)]
    # closed form: two logits one apart share the weight as sigmoid(+-1)
    assert ids[0].tolist() == [1, 3]
    assert abs(w[0, 0] - 1 / (1 + math.exp(-1))) < 1e-15
    assert abs(w[0, 1] - 1 / (1 + math.exp(1))) < 1e-15


def test_softmax_router_brute_force():
    # The selected set is the k-subset with the largest logit sum (distinct
    # logits), and its weights are exp(l) normalised over that subset.
    rng = np.random.default_rng(1)
    for E, k in [(5, 1), (6, 2), (7, 3), (8, 4), (6, 6)]:
        L = rng.permutation(E)[None, :] * 0.37 - 1.1
        ids, w = oracle.router_topk_softmax(L, k)
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(L[0, list(c)]))
        assert sorted(ids[0].tolist()) == sorted(best)
        assert all(L[0, ids[0, j]] > L[0, ids[0, j + 1]] for j in range(k - 1))
        ex = [math.exp(L[0, i]) for i in ids[0]]
        assert np.allclose(w[0], np.array(ex) / sum(ex), rtol=1e-14, atol=0)


def test_softmax_router_full_k_is_softmax():
    # k = E: the weights are the full softmax, listed in descending order.
    L = np.random.default_rng(2).standard_normal((3, 16))
    ids, w = oracle.router_topk_softmax(L, 16)
    e = np.exp(L)
    full = e / e.sum(1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-14)
    assert np.array_equal(np.sort(ids, 1), np.tile(np.arange(16), (3, 1)))


def test_softmax_router_ties_take_lower_index():
    L = np.zeros((2, 10))
    L[1, [2, 7, 9]] = 3.0
    ids, w = oracle.router_topk_softmax(L, 4)
    assert ids[0].tolist() == [0, 1, 2, 3]
    assert np.allclose(w[0], 0.25, rtol=0, atol=1e-15)
    assert ids[1].tolist() == [2, 7, 9, 0]


def test_softplus_stable_form():
    # softplus(0) = ln 2; softplus(x) -> x for large x with no overflow (the
    # plain log(1 + exp(x)) is inf in fp32 past about 88.7); np.logaddexp(0, x)
    # is an independent evaluation of log(1 + e^x).
    sp = oracle._softplus_f32(np.array([0.0, 100.0, 200.0, -20.0, 3.5, -0.25], np.float32))
    assert abs(sp[0] - math.log(2)) < 1e-7
    assert sp[1] == np.float32(100.0) and sp[2] == np.float32(200.0)
    assert np.isfinite(sp).all()
    ref = np.logaddexp(0.0, np.array([0.0, 100.0, 200.0, -20.0, 3.5, -0.25]))
    assert np.allclose(sp, ref, rtol=3e-7, atol=0)


def test_sqrtsoftplus_router_scores_and_weights():
    # Weight of a selected expert = sqrt(log(1 + e^l)) * routed scaling factor.
    L = np.array([[0.0, 2.0, -1.0, 0.5, 4.0]])
    ids, w, biased = oracle.router_sqrtsoftplus(L, np.zeros(5, np.float32), 2, 2.5)
    assert ids[0].tolist() == [4, 1]
    for j, e in enumerate(ids[0]):
        assert abs(w[0, j] - math.sqrt(math.log1p(math.exp(L[0, e]))) * 2.5) < 1e-12
    assert abs(biased[0, 0] - math.sqrt(math.log(2))) < 1e-7


def test_sqrtsoftplus_zero_bias_matches_logit_order():
    # sqrt(softplus) is increasing, so with zero bias the selection is the
    # top-k of the logits themselves (well separated logits).
    rng = np.random.default_rng(3)
    L = np.stack([rng.permutation(288) * 0.01 - 1.0 for _ in range(4)])
    ids, _, _ = oracle.router_sqrtsoftplus(L, np.zeros(288, np.float32), 6, 1.0)
    ref, _ = oracle.router_topk_softmax(L, 6)
    assert np.array_equal(ids, ref)


def test_sqrtsoftplus_bias_selects_but_does_not_weight():
    # The bias decides the choice (aux-loss-free balancing) but the weight is
    # the unbiased score: a small logit with a large bias wins, weighted by
    # its own sqrt(softplus).
    L = np.array([[3.0, 0.0, 1.0]])
    bias = np.array([0.0, 5.0, 0.0], np.float32)
    ids, w, biased = oracle.router_sqrtsoftplus(L, bias, 1, 1.0)
    assert ids[0].tolist() == [1]
    assert abs(w[0, 0] - math.sqrt(math.log(2))) < 1e-12
    assert abs(biased[0, 1] - (math.sqrt(math.log(2)) + 5.0)) < 1e-6
    # brute force over 2-subsets of a tiny case with random bias
    rng = np.random.default_rng(4)
    L = rng.standard_normal((1, 6))
    bias = rng.standard_normal(6).astype(np.float32)
    ids, _, _ = oracle.router_sqrtsoftplus(L, bias, 2, 1.0)
    score = [math.sqrt(math.log1p(math.exp(L[0, e]))) + float(bias[e]) for e in range(6)]
    best = max(itertools.combinations(range(6), 2), key=lambda c: score[c[0]] + score[c[1]])
    assert sorted(ids[0].tolist()) == sorted(best)


def test_gated_shared_residual_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4; a missing
    # gate is weight 1; a very negative logit switches the shared expert off.
    moe = np.array([[1.0, -2.0], [0.5, 0.0], [3.0, 1.0], [0.0, 0.0]])
    shared = np.array([[4.0, 8.0], [-4.0, 2.0], [1.0, 1.0], [10.0, -10.0]])
    res = np.array([[0.25, 0.5], [1.0, 1.0], [-1.0, 2.0], [7.0, 7.0]])
    g = np.array([0.0, math.log(3), -math.log(3), -800.0])
    out = oracle.gated_shared_residual(moe, shared, g, res)
    expect = np.array([[0.25 + 2.0 + 1.0, 0.5 + 4.0 - 2.0],
                       [1.0 - 3.0 + 0.5, 1.0 + 1.5 + 0.0],
                       [-1.0 + 0.25 + 3.0, 2.0 + 0.25 + 1.0],
                       [7.0, 7.0]])
    assert np.allclose(out, expect, rtol=0, atol=1e-12)
    assert np.array_equal(oracle.gated_shared_residual(moe, shared), moe + shared)
    assert np.array_equal(oracle.gated_shared_residual(moe, None, None, res), moe + res)


def test_combine_pairs_closed_forms():
    # two tokens, k = 2: token 0 mixes rows 0 and 1; token 1's second pair is
    # dropped (expert id out of range), so only row 2 counts, weighted.
    y = np.array([[1.0, 2.0], [10.0, 20.0], [3.0, -3.0], [1e9, 1e9]])
    ids = np.array([[0, 1], [1, 4]])
    w = np.array([[0.25, 0.75], [0.5, 0.5]])
    out = oracle.combine_pairs(y, ids, w, 4)
    assert np.array_equal(out, np.array([[7.75, 15.5], [1.5, -1.5]]))
    # k = 1 with unit weights is the identity on the rows
    y1 = np.arange(12.0).reshape(3, 4)
    assert np.array_equal(oracle.combine_pairs(y1, np.zeros((3, 1), int), np.ones((3, 1)), 1), y1)


def test_softmax_bias_router():
    # logits (2, 1, 0), bias (0, 0, 1): p = softmax = (e^2, e, 1) / (e^2 + e + 1);
    # p_2 + 1 beats p_0, so k = 1 picks expert 2 with weight 1, and k = 2 picks
    # 2 then 0 with the renormalised p: 1 / (1 + e^2) and e^2 / (1 + e^2).
    L = np.array([[2.0, 1.0, 0.0]])
    b = np.array([0.0, 0.0, 1.0], np.float32)
    ids, w = oracle.router_topk_softmax(L, 1, b)
    assert ids.tolist() == [[2]] and abs(w[0, 0] - 1.0) < 1e-15
    ids, w = oracle.router_topk_softmax(L, 2, b)
    assert ids.tolist() == [[2, 0]]
    e2 = math.exp(2.0)
    assert np.allclose(w[0], [1 / (1 + e2), e2 / (1 + e2)], rtol=1e-14, atol=0)
    # a zero bias gives the unbiased router's choice and weights (distinct logits)
    rng = np.random.default_rng(9)
    L = np.stack([rng.permutation(64) * 0.05 for _ in range(5)])
    ids0, w0 = oracle.router_topk_softmax(L, 8)
    ids1, w1 = oracle.router_topk_softmax(L, 8, np.zeros(64, np.float32))
    assert np.array_equal(ids0, ids1) and np.allclose(w0, w1, rtol=1e-13, atol=0)
