"""Router top-k on the device against the oracle's routers.

Softmax top-k selects by comparing the logits themselves, so expert ids and
their order are compared bit for bit (equal logits: lower index first).  The
sqrtsoftplus selection is decided on fp32 scores that the kernel and the
oracle compute with different fp32 libm routines, so ids are compared where
the oracle's boundary gap is wider than a few ulp and checked for validity
(no unselected expert scores clearly above a selected one) everywhere.
Weights: fp32 softmax against fp64 within 2e-6 absolute; sqrtsoftplus weights
within the pages' 1e-5 absolute."""
import math

import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import TOL, normwise_err, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _logits(rng, T, E, dt, sigma=1.0):
    x = synth.router_logits(rng, T, E, dt, sigma)
    if dt == "f32":
        return torch.from_numpy(x).cuda(), x.astype(np.float64)
    t = torch_act(x, dt)
    return t, to_f64(t)


def test_worked_example():
    L = torch.tensor([[1.0, 5.0, 3.0, 4.0]], device="cuda")
    ids, w = qm.router_topk(L, 2)
    assert ids.cpu().tolist() == [[1, 3]]
    w = w.cpu().numpy().astype(np.float64)
    assert abs(w.sum() - 1.0) < 1e-6 and w[0, 0] > w[0, 1]
    _, ref = oracle.router_topk_softmax(np.array([[1.0, 5.0, 3.0, 4.0]]), 2)
    assert np.allclose(w, ref, rtol=0, atol=2e-6)


@pytest.mark.parametrize("T,E,k,dt", [
    (2048, 128, 8, "bf16"),   # 128 experts, top-8
    (999, 256, 8, "f32"),
    (333, 60, 4, "f16"),      # experts not a multiple of 64
    (64, 1024, 8, "bf16"),    # the expert limit
    (65, 8, 8, "f32"),        # k = E
    (7, 1, 1, "f32"),
    (130, 513, 3, "bf16"),
])
def test_softmax_matches_oracle(T, E, k, dt):
    rng = np.random.default_rng(T * 7 + E)
    L, L64 = _logits(rng, T, E, dt, sigma=2.0)
    ids, w = qm.router_topk(L, k)
    ref_ids, ref_w = oracle.router_topk_softmax(L64, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=0, atol=2e-6)


def test_softmax_ties_and_special_values():
    T, E, k = 16, 96, 8
    rng = np.random.default_rng(11)
    L = rng.integers(-3, 4, size=(T, E)).astype(np.float32)  # many equal logits
    L[0] = 0.0
    L[1, ::2] = -0.0
    L[2, :] = -np.inf
    L[2, 50] = 1.0
    L[3, [5, 9, 70]] = np.nan
    L[4, :90] = np.nan
    L[5, [3, 66]] = np.inf
    ids, w = qm.router_topk(torch.from_numpy(L).cuda(), k)
    with np.errstate(invalid="ignore"):  # infinite or NaN maxima make NaN weights on both sides
        ref_ids, ref_w = oracle.router_topk_softmax(L.astype(np.float64), k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert ids.cpu().numpy()[0].tolist() == list(range(k))
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=0, atol=2e-6, equal_nan=True)


def _check_sqrtsoftplus(L64, bias, k, scale, ids, w):
    ids = ids.cpu().numpy()
    w = w.cpu().numpy().astype(np.float64)
    ref_ids, _, biased = oracle.router_sqrtsoftplus(L64, bias, k, scale)
    b64 = biased.astype(np.float64)
    tol = 4 * np.spacing(np.abs(b64).max(axis=1, keepdims=True).astype(np.float32)).astype(np.float64)
    sel = np.take_along_axis(b64, ids.astype(np.int64), 1)
    mask = np.ones_like(b64, bool)
    np.put_along_axis(mask, ids.astype(np.int64), False, 1)
    rest = np.where(mask, b64, -np.inf).max(1)
    # valid: ids distinct, in range, no unselected expert clearly better, best first
    assert all(len(set(r.tolist())) == k for r in ids)
    assert ids.min() >= 0 and ids.max() < L64.shape[1]
    assert (sel.min(1) >= rest - tol[:, 0]).all()
    assert (np.diff(sel, axis=1) <= tol).all()
    # unique where the oracle's boundary is clear
    srt = -np.sort(-b64, axis=1)
    clear = (srt[:, k - 1] - srt[:, k] > tol[:, 0]) if k < b64.shape[1] else np.ones(len(b64), bool)
    assert clear.mean() > 0.95
    assert np.array_equal(np.sort(ids[clear], 1), np.sort(ref_ids[clear], 1))
    # weights: the unbiased score of the chosen expert, from the fp64 logit
    l = np.take_along_axis(L64, ids.astype(np.int64), 1)
    ref_w = np.sqrt(np.maximum(l, 0) + np.log1p(np.exp(-np.abs(l)))) * scale
    assert np.allclose(w, ref_w, rtol=0, atol=1e-5)


@pytest.mark.parametrize("T,E,k,dt,scale", [
    (2048, 288, 6, "bf16", 1.5),   # 288 experts, top-6
    (512, 512, 8, "f32", 2.5),     # 512 experts
    (100, 256, 8, "f16", 1.0),
    (31, 1000, 8, "f32", 1.0),
])
def test_sqrtsoftplus_matches_oracle(T, E, k, dt, scale):
    rng = np.random.default_rng(E + k)
    L, L64 = _logits(rng, T, E, dt, sigma=3.0)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    ids, w = qm.router_topk(L, k, scoring=qm.ROUTER_SQRTSOFTPLUS, bias=torch.from_numpy(bias).cuda(),
                            scale=scale)
    _check_sqrtsoftplus(L64, bias, k, scale, ids, w)


def test_sqrtsoftplus_large_logits_and_no_bias():
    # |logit| up to 120: the stable softplus stays finite (exp(120) overflows fp32)
    rng = np.random.default_rng(5)
    T, E, k = 64, 288, 6
    L = (rng.uniform(-120, 120, size=(T, E))).astype(np.float32)
    ids, w = qm.router_topk(torch.from_numpy(L).cuda(), k, scoring=qm.ROUTER_SQRTSOFTPLUS)
    assert torch.isfinite(w).all()
    _check_sqrtsoftplus(L.astype(np.float64), np.zeros(E, np.float32), k, 1.0, ids, w)
    # zero bias: sqrt(softplus) is increasing, so the choice is the logit top-k
    ref_ids, _ = oracle.router_topk_softmax(L.astype(np.float64), k)
    assert np.array_equal(np.sort(ids.cpu().numpy(), 1), np.sort(ref_ids, 1))


def _check_validity(b64, ids, k):
    """GPU ids against fp32 oracle selection scores b64 [T, E]: distinct, in
    range, best first and no unselected expert clearly better (a few ulp);
    equal to the oracle's set where the boundary gap is clear."""
    tol = 4 * np.spacing(np.abs(b64).max(axis=1, keepdims=True).astype(np.float32)).astype(np.float64)
    sel = np.take_along_axis(b64, ids.astype(np.int64), 1)
    mask = np.ones_like(b64, bool)
    np.put_along_axis(mask, ids.astype(np.int64), False, 1)
    rest = np.where(mask, b64, -np.inf).max(1)
    assert all(len(set(r.tolist())) == k for r in ids)
    assert (sel.min(1) >= rest - tol[:, 0]).all()
    assert (np.diff(sel, axis=1) <= tol).all()
    srt = -np.sort(-b64, axis=1)
    return (srt[:, k - 1] - srt[:, k] > tol[:, 0]) if k < b64.shape[1] else np.ones(len(b64), bool)


@pytest.mark.parametrize("T,E,k,dt", [(1024, 32, 4, "bf16"), (300, 256, 8, "f32"), (77, 1000, 8, "f16")])
def test_softmax_bias_matches_oracle(T, E, k, dt):
    # softmax-then-bias: p = softmax over all experts, select on p + bias,
    # weights the selected p renormalised
    rng = np.random.default_rng(T + E)
    L, L64 = _logits(rng, T, E, dt, sigma=2.0)
    bias = (0.05 * rng.standard_normal(E)).astype(np.float32)
    ids, w = qm.router_topk(L, k, bias=torch.from_numpy(bias).cuda())
    ids = ids.cpu().numpy()
    ref_ids, _ = oracle.router_topk_softmax(L64, k, bias)
    b64 = oracle.router_softmax_bias_scores(L64, bias).astype(np.float64)
    clear = _check_validity(b64, ids, k)
    assert clear.mean() > 0.95
    assert np.array_equal(np.sort(ids[clear], 1), np.sort(ref_ids[clear], 1))
    p64 = np.exp(L64 - L64.max(1, keepdims=True))
    sel = np.take_along_axis(p64, ids.astype(np.int64), 1)
    assert np.allclose(w.cpu().numpy(), sel / sel.sum(1, keepdims=True), rtol=0, atol=2e-6)


def test_bias_decides_but_does_not_weight():
    L = torch.tensor([[3.0, 0.0, 1.0, -2.0]], device="cuda")
    bias = torch.tensor([0.0, 5.0, 0.0, 0.0], device="cuda")
    ids, w = qm.router_topk(L, 2, scoring=qm.ROUTER_SQRTSOFTPLUS, bias=bias)
    assert ids.cpu().tolist() == [[1, 0]]
    assert abs(w[0, 0].item() - math.sqrt(math.log(2))) < 1e-6
    assert abs(w[0, 1].item() - math.sqrt(math.log1p(math.exp(3.0)))) < 1e-6


def test_empty_batch_launches_nothing():
    ids, w = qm.router_topk(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), 8)
    assert ids.shape == (0, 8) and w.shape == (0, 8)


def test_router_feeds_the_prefill_path():
    # logits -> device router -> plan -> gathered gate/up (SwiGLU) -> down ->
    # combine, against the oracle router and the oracle MoE FFN.
    inp = synth.qwen_a3b_prefill(256, E=32)
    T, k, E, H = inp.T, inp.k, inp.E, inp.H
    rng = np.random.default_rng(21)
    L, L64 = _logits(rng, T, E, "bf16", sigma=2.0)
    x = torch_act(inp.x, "bf16")
    gu, dn = upload(inp.w_gate_up), upload(inp.w_down)
    ids, w = qm.router_topk(L, k)
    bm = 80
    plan = qm.moe_plan(ids, E, bm)
    h = qm.moe_gather_qmm(gu, plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU)
    y = qm.moe_gather_qmm(dn, plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, out_dtype=qm.F32)
    out = qm.moe_combine(y, plan, T, k, E, w, out_dtype=qm.F32)
    ref_ids, ref_w = oracle.router_topk_softmax(L64, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=0, atol=2e-6)
    srt = qm.plan_views(plan, T, k, E)["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(inp.x, "bf16"), ref_ids, inp.w_gate_up)[srt]
    hg = to_f64(h)
    assert normwise_err(hg, href, "bf16") <= TOL
    hp = np.zeros_like(href)
    hp[srt] = hg
    oref = oracle.moe_down_combine(hp, ref_ids, ref_w, inp.w_down)
    assert normwise_err(to_f64(out), oref, "f32") <= TOL
