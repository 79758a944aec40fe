"""Pins for the oracle's matmuls, MoE stages, routing plan and the router
recipe of the synthetic inputs (CPU only).

Brute force on tiny shapes uses pure-Python loops over scalar decodes of the
blocks (not the oracle's vectorised decoders), non-square shapes everywhere so
that a transposed operand fails, and special cases that reduce the MoE to a
dense matmul.
"""
import math
import struct


import numpy as np
import pytest

import oracle
import synth


def _scalar_q8_0(W, e, n, k):
    blk = W.blocks[e, n, k // 32]
    d = struct.unpack("<e", bytes(blk[0:2]))[0]
    q = struct.unpack("<b", bytes(blk[2 + k % 32:3 + k % 32]))[0]
    return q * d


def _scalar_int4(W, e, n, k):
    word = int(W.qs[e, n, k // 8])
    q = (word >> (4 * (k % 8))) & 15
    s = struct.unpack("<e", struct.pack("<H", int(W.scale[e, n, k // W.group])))[0]
    b = struct.unpack("<e", struct.pack("<H", int(W.bias[e, n, k // W.group])))[0]
    return s * q + b


def _act(bits, dtype):
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", int(bits)))[0]
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


@pytest.mark.parametrize("fmt,scalar", [("q8_0", _scalar_q8_0), ("int4", _scalar_int4)])
def test_qmm_brute_force(fmt, scalar):
    rng = np.random.default_rng(7)
    M, N, K = 3, 5, 64 if fmt == "int4" else 96
    W = synth.weights(fmt, rng, 1, N, K)
    xb = synth.activations(rng, M, K, "f16")
    x64 = oracle.act_to_f64(xb, "f16")
    y = oracle.qmm(x64, W)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += _act(xb[m, k], "f16") * scalar(W, 0, n, k)
            assert abs(acc - y[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_silu_identities():
    z = np.linspace(-30, 30, 601)
    s = oracle.silu(z)
    assert oracle.silu(0.0) == 0.0
    assert np.allclose(s - oracle.silu(-z), z, rtol=0, atol=1e-12)  # silu(z) - silu(-z) = z
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu(-40.0)) < 1e-15
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_plan_against_sorted_and_invariants():
    rng = np.random.default_rng(1)
    T, k, E, bm = 37, 3, 9, 4
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[5, 1] = E + 3      # out of range: dropped and counted
    ids[9, 0] = -1
    p = oracle.plan(ids, E, bm)
    flat = ids.reshape(-1)
    keep = [q for q in range(T * k) if 0 <= flat[q] < E]
    assert p["dropped"] == 2
    assert list(p["sorted"]) == sorted(keep, key=lambda q: (flat[q], q))
    assert p["counts"].sum() == len(keep) and p["offsets"][-1] == len(keep)
    rows = []
    for e, r0, n in p["tiles"]:
        assert 1 <= n <= bm
        seg = p["sorted"][r0:r0 + n]
        assert np.all(flat[seg] == e)
        rows.extend(range(r0, r0 + n))
    assert rows == list(range(len(keep)))


def _tiny_moe(E=3, T=5, k=2, H=64, I=64, fmt="int4", act="bf16", seed=4):
    rng = np.random.default_rng(seed)
    x = synth.activations(rng, T, H, act)
    ids, w = synth.routing_softmax(rng, T, E, k)
    wgu = synth.weights(fmt, rng, E, 2 * I, H)
    wd = synth.weights(fmt, rng, E, H, I)
    return x, ids, w, wgu, wd


def test_moe_brute_force_pairs():
    x, ids, w, wgu, wd = _tiny_moe()
    T, k = ids.shape
    H, I = wd.N, wd.K
    x64 = oracle.act_to_f64(x, "bf16")
    out = oracle.moe_ffn(x64, ids, w, wgu, wd)
    for t in range(T):
        ref = np.zeros(H)
        for j in range(k):
            e = int(ids[t, j])
            h = np.zeros(I)
            for i in range(I):
                g = sum(x64[t, c] * _scalar_int4(wgu, e, i, c) for c in range(H))
                u = sum(x64[t, c] * _scalar_int4(wgu, e, I + i, c) for c in range(H))
                h[i] = g / (1 + math.exp(-g)) * u
            for n in range(H):
                ref[n] += float(w[t, j]) * sum(h[i] * _scalar_int4(wd, e, n, i) for i in range(I))
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12)


def test_moe_single_expert_is_dense_ffn():
    x, _, _, wgu, wd = _tiny_moe(E=1)
    T = x.shape[0]
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    x64 = oracle.act_to_f64(x, "bf16")
    gu = oracle.qmm(x64, wgu)
    I = wgu.N // 2
    dense = oracle.qmm(oracle.silu(gu[:, :I]) * gu[:, I:], wd)
    assert np.allclose(oracle.moe_ffn(x64, ids, w, wgu, wd), dense, rtol=1e-13, atol=1e-13)


def test_moe_identical_experts_weights_sum_to_one():
    x, ids, w, wgu, wd = _tiny_moe(E=4, k=3)
    same_gu = synth.QWeights("int4", 4, wgu.N, wgu.K, 64, qs=np.repeat(wgu.qs[:1], 4, 0),
                             scale=np.repeat(wgu.scale[:1], 4, 0), bias=np.repeat(wgu.bias[:1], 4, 0))
    same_d = synth.QWeights("int4", 4, wd.N, wd.K, 64, qs=np.repeat(wd.qs[:1], 4, 0),
                            scale=np.repeat(wd.scale[:1], 4, 0), bias=np.repeat(wd.bias[:1], 4, 0))
    x64 = oracle.act_to_f64(x, "bf16")
    many = oracle.moe_ffn(x64, ids, w.astype(np.float64), same_gu, same_d)
    one = oracle.moe_ffn(x64, np.zeros((x.shape[0], 1), np.int32), np.ones((x.shape[0], 1)), same_gu, same_d)
    assert np.allclose(many, one * w.astype(np.float64).sum(1, keepdims=True), rtol=1e-12, atol=1e-12)


def test_moe_sampled_matches_full():
    x, ids, w, wgu, wd = _tiny_moe(E=4, T=6, k=2, fmt="q8_0", act="f16")
    x64 = oracle.act_to_f64(x, "f16")
    h = oracle.moe_gate_up(x64, ids, wgu)
    out = oracle.moe_down_combine(h, ids, w, wd)
    pairs = [0, 5, 11]
    cols = np.array([0, 7, 31])
    assert np.allclose(oracle.moe_gate_up_rows(x64, ids, wgu, pairs, cols), h[pairs][:, cols], rtol=1e-13, atol=1e-14)
    tokens = [1, 4]
    hp = {p: h[p] for p in range(h.shape[0])}
    assert np.allclose(oracle.moe_down_rows(hp, ids, w, wd, tokens, cols), out[tokens][:, cols], rtol=1e-13, atol=1e-14)


def test_moe_exact_integer_case():
    # Power-of-two scales, small integer activations: every sum is an integer
    # below 2**24, so the fp64 oracle equals exact integer arithmetic.
    T, E, k, H, N = 4, 2, 1, 64, 6
    rng = np.random.default_rng(8)
    W = synth.q8_0(rng, E, N, H)
    W.blocks[..., 0:2] = np.frombuffer(struct.pack("<H", 0x3C00), np.uint8)  # d = 1
    xi = rng.integers(-4, 5, size=(T, H))
    xb = synth.f16_bits(xi.astype(np.float32))
    y = oracle.qmm(oracle.act_to_f64(xb, "f16"), W, e=1)
    codes = W.blocks[1, :, :, 2:].view(np.int8).reshape(N, H).astype(np.int64)
    assert np.array_equal(y, (xi @ codes.T).astype(np.float64))


def _expert0_as_dense(W):
    """Routed expert 0 of a stacked int4 weight, as a dense [1, N, K] weight."""
    return synth.QWeights("int4", 1, W.N, W.K, W.group, qs=W.qs[:1].copy(), scale=W.scale[:1].copy(),
                          bias=W.bias[:1].copy())


@pytest.mark.parametrize("h_dtype", [None, "bf16"])
def test_moe_ffn_shared_expert_equal_to_routed(h_dtype):
    """The shared-expert branch of moe_ffn (gate/up, SwiGLU, the h storage
    rounding, down, then the gated add): with the shared weights equal to
    routed expert 0 and every token routed top-1 to expert 0 with weight 1,
    the shared term equals the routed output, so the result is exactly twice
    it, 1 + sigmoid(0) = 1.5 times it with gate logits 0, and 1 + 3/4 with
    gate logits ln 3 -- a swapped gate/up half, a dropped rounding or a
    misplaced gate in the shared branch breaks the equality."""
    x, _, _, wgu, wd = _tiny_moe(E=3, T=6, k=2)
    T = x.shape[0]
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    x64 = oracle.act_to_f64(x, "bf16")
    routed = oracle.moe_ffn(x64, ids, w, wgu, wd, h_dtype=h_dtype)
    shared = (_expert0_as_dense(wgu), _expert0_as_dense(wd))
    assert np.abs(routed).max() > 0
    both = oracle.moe_ffn(x64, ids, w, wgu, wd, h_dtype=h_dtype, shared=shared)
    assert np.array_equal(both, 2.0 * routed)
    half = oracle.moe_ffn(x64, ids, w, wgu, wd, h_dtype=h_dtype, shared=shared, shared_gate=np.zeros(T))
    assert np.array_equal(half, 1.5 * routed)
    g3 = oracle.moe_ffn(x64, ids, w, wgu, wd, h_dtype=h_dtype, shared=shared, shared_gate=np.full(T, math.log(3.0)))
    assert np.allclose(g3, 1.75 * routed, rtol=1e-15, atol=0)
    res = np.arange(T * wd.N, dtype=np.float64).reshape(T, wd.N) / 7.0
    with_res = oracle.moe_ffn(x64, ids, w, wgu, wd, h_dtype=h_dtype, shared=shared, residual=res)
    assert np.array_equal(with_res, 2.0 * routed + res)


def test_moe_ffn_shared_expert_brute_force():
    """The shared branch against scalar loops over the blocks (a shared
    expert unlike any routed one): out_t = routed_t + silu(g_t) * u_t . Wsd^T."""
    x, ids, w, wgu, wd = _tiny_moe(E=2, T=3, k=1, H=64, I=64, seed=9)
    rng = np.random.default_rng(10)
    H, I = wd.N, wd.K
    sgu = synth.int4(rng, 1, 2 * I, H)
    sd = synth.int4(rng, 1, H, I)
    x64 = oracle.act_to_f64(x, "bf16")
    routed = oracle.moe_ffn(x64, ids, w, wgu, wd)
    got = oracle.moe_ffn(x64, ids, w, wgu, wd, shared=(sgu, sd))
    for t in range(x.shape[0]):
        hs = np.zeros(I)
        for i in range(I):
            g = sum(x64[t, c] * _scalar_int4(sgu, 0, i, c) for c in range(H))
            u = sum(x64[t, c] * _scalar_int4(sgu, 0, I + i, c) for c in range(H))
            hs[i] = g / (1 + math.exp(-g)) * u
        ref = routed[t] + np.array([sum(hs[i] * _scalar_int4(sd, 0, n, i) for i in range(I)) for n in range(H)])
        assert np.allclose(got[t], ref, rtol=1e-12, atol=1e-12)


def test_synth_pair_weights_are_softmax_of_selected_logits():
    """The routing recipe of the inputs: ids are the k largest logits of the
    row, weights exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected ones
    (they sum to 1 and fall along the row)."""
    logits = np.array([[1.0, 5.0, 3.0, 4.0], [0.5, -1.0, 2.0, 2.5]], np.float32)
    ids, w = synth._pairs_from_keys(logits, 2)
    assert ids.tolist() == [[1, 3], [3, 2]]
    e1 = 1.0 / (1.0 + math.exp(-1.0))  # softmax of (a, a - 1): sigmoid(1), sigmoid(-1)
    assert np.allclose(w[0], [e1, 1 - e1], rtol=1e-7)
    e2 = 1.0 / (1.0 + math.exp(-0.5))
    assert np.allclose(w[1], [e2, 1 - e2], rtol=1e-7)
    rng = np.random.default_rng(3)
    ids, w = synth.routing_softmax(rng, 50, 16, 4)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6) and np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 4 for r in ids.tolist())
