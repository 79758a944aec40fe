"""GPU checks of the split units of the LDS-ring gathered matmul (int4, and
IQ2_XXS, Q2_K, MXFP4, Q4_K, Q6_K, FP8 and Q8_0 with fp16 activations).

With a routing plan of at least 2048 pairs (which carries a work-balancing
area), the ring kernel looks at each XCD's units (tiles x, x + 8,
... of XCD x, times the column blocks): when they fill whole rounds of the
XCD's resident workgroups plus a short last round (at most a quarter of
one), those last units are split into 4 parts along K when each part keeps
at least 4 K tiles.  The parts are dealt after the whole units; each parks
its fp32 sums in the plan, and the last to finish adds the parts in part
order and writes the unit.

Checked on shapes where a host model of that rule (the same counts) says
units are split:

  * every output of the gathered matmul against the fp64 oracle (normwise
    2e-3 bound of tests/_helpers): SwiGLU with bf16 activations and group
    64, STORE with fp16 activations and group 128 (K = 1280: 20 K tiles, so
    parts start at tiles 5, 10, 15, in the middle of a group), the weighted
    combine into fp32 with bf16, group 128;
  * the IQ2_XXS ring kernel (fp16 activations, SwiGLU, K = 1280: parts start
    inside a 256-value super-block) and the Q2_K one (STORE into fp32, parts
    starting on the odd tile of a pair that shares a 512-byte code half) and
    the MXFP4 one (SwiGLU, scales folded into the fp16 operands, and with
    every exponent out of that range, the fp32-scale loop) and the
    Q4_K one (SwiGLU, parts starting inside a super-block) and the Q6_K one
    (STORE into fp32; a part starting on an odd tile loads its pair's top
    bits itself), the FP8 one (STORE into fp32, parts starting inside a
    128-value scale block) and the two-stage Q8_0 one (SwiGLU) against the
    fp64 oracle;
  * two calls give bit-identical outputs (the parts are summed in a fixed
    order whichever finishes last);
  * the plan's tickets are zero after every call.
"""
import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import TOL, normwise_err, report, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BM = 80
PARTS = 4


def _sk_offset_words(T, k, E):
    P = T * k
    words = 8 + E + E + 1 + P
    words = (words + 3) & ~3
    words += 4 * (min(P, E) + P // 16) + P
    words += ((P + 1023) // 1024) * E
    return (words + 63) & ~63


def _model_split_units(n_tiles, n_nt, KT, resident):
    """Units split into K parts: per XCD x, ux = ceil((n_tiles - x) / 8) *
    n_nt units over sx = resident / 8 workgroups; the ux mod sx units past
    the last whole round are split when there are at most sx / 4 of them and
    each part keeps at least 4 K tiles."""
    sx = resident // 8
    total = 0
    for x in range(8):
        nq = (n_tiles - x + 7) // 8 if n_tiles > x else 0
        ux = nq * n_nt
        if 0 < sx <= 64 and ux > sx and KT >= 4 * PARTS:
            R = ux % sx
            if R <= sx // 4:
                total += R
    return total


def _resident():
    return min(64, 2 * torch.cuda.get_device_properties(0).multi_processor_count // 8) * 8


def _setup(act, group, N, K, seed, T=512, E=64, k=8):
    rng = np.random.default_rng(seed)
    x = synth.activations(rng, T, K, act)
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.int4(rng, E, N, K, group)
    return T, E, k, x, ids, w, W


def _plan(ids, T, k, E, n_nt, KT):
    plan = qm.moe_plan(torch.from_numpy(ids).cuda(), E, BM)
    v = qm.plan_views(plan, T, k, E)
    n_tiles = int(v["header"][1].item())
    assert _model_split_units(n_tiles, n_nt, KT, _resident()) > 0, "shape does not split units"
    return plan, v


def _tickets_zero(plan, T, k, E):
    off = _sk_offset_words(T, k, E)
    assert plan.numel() >= off + 512
    assert int(plan[off:off + 512].abs().sum().item()) == 0


def _pair_rows(x64, ids, W):
    """fp64 x_t . W[e]^T for every pair, in pair order."""
    T, k = ids.shape
    y = np.zeros((T * k, W.N))
    flat = ids.reshape(-1)
    for e in range(W.E):
        pairs = np.nonzero(flat == e)[0]
        if len(pairs):
            y[pairs] = x64[pairs // k] @ oracle.dequant_rows(W, e, np.arange(W.N)).astype(np.float64).T
    return y


def test_split_units_swiglu_bf16_group64():
    N, K = 4096, 1280
    T, E, k, x, ids, w, W = _setup("bf16", 64, N, K, 11)
    plan, v = _plan(ids, T, k, E, n_nt=N // 2 // 128, KT=K // 64)
    gu = upload(W)
    xd = torch_act(x, "bf16")
    h1 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.BF16)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    h2 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.BF16)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(h1, h2)
    srt = v["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "bf16"), ids, W)[srt]
    err = normwise_err(to_f64(h1), href, "bf16")
    assert err <= TOL, (err, report(to_f64(h1), href))


def test_split_units_store_f16_group128():
    N, K = 2048, 1280
    T, E, k, x, ids, w, W = _setup("f16", 128, N, K, 12)
    plan, v = _plan(ids, T, k, E, n_nt=N // 256, KT=K // 64)
    dw = upload(W)
    xd = torch_act(x, "f16")
    y1 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    y2 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(y1, y2)
    srt = v["sorted"].cpu().numpy()
    yref = _pair_rows(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(y1), yref, "f32")
    assert err <= TOL, (err, report(to_f64(y1), yref))


def test_split_units_weighted_combine_bf16_group128():
    N, K = 2048, 1280
    T, E, k, x, ids, w, W = _setup("bf16", 128, N, K, 13)
    plan, v = _plan(ids, T, k, E, n_nt=N // 256, KT=K // 64)
    dw = upload(W)
    xd = torch_act(x, "bf16")
    out = torch.zeros((T, N), dtype=torch.float32, device="cuda")
    qm.moe_gather_qmm(dw, plan, T, k, xd, topk_w=torch.from_numpy(w).cuda(), epilogue=qm.EPI_WEIGHTED_COMBINE,
                      out=out)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    x64 = oracle.act_to_f64(x, "bf16")
    oref = oracle.moe_down_combine(x64[np.arange(T * k) // k], ids, w, W)
    err = normwise_err(to_f64(out), oref, "f32")
    assert err <= TOL, (err, report(to_f64(out), oref))


def test_split_units_iq2_xxs_swiglu_f16():
    N, K, T, E, k = 4096, 1280, 512, 64, 8
    rng = np.random.default_rng(16)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.iq2_xxs(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 2 // 128, KT=K // 64)
    gu = upload(W)
    xd = torch_act(x, "f16")
    h1 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    h2 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(h1, h2)
    srt = v["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(h1), href, "f16")
    assert err <= TOL, (err, report(to_f64(h1), href))


def test_split_units_q2_k_store_f16():
    N, K, T, E, k = 2048, 1280, 512, 64, 8
    rng = np.random.default_rng(12)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.q2_k(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 256, KT=K // 64)
    dw = upload(W)
    xd = torch_act(x, "f16")
    y1 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    y2 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(y1, y2)
    srt = v["sorted"].cpu().numpy()
    yref = _pair_rows(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(y1), yref, "f32")
    assert err <= TOL, (err, report(to_f64(y1), yref))


def test_split_units_mxfp4_swiglu_f16():
    N, K, T, E, k = 4096, 1280, 512, 64, 8
    rng = np.random.default_rng(16)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.mxfp4(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 2 // 128, KT=K // 64)
    gu = upload(W)
    xd = torch_act(x, "f16")
    h1 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    h2 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(h1, h2)
    srt = v["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(h1), href, "f16")
    assert err <= TOL, (err, report(to_f64(h1), href))


def test_split_units_mxfp4_unfolded_scales():
    # every block exponent at 2^-14, below the range the fp16 operands can
    # carry exactly: each workgroup runs the fp32-scale loop, split parts too
    # (SwiGLU into fp32, where the small products keep full precision)
    N, K, T, E, k = 4096, 1280, 512, 64, 8
    rng = np.random.default_rng(16)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.mxfp4(rng, E, N, K)
    W.blocks[..., 0] = 113
    plan, v = _plan(ids, T, k, E, n_nt=N // 2 // 128, KT=K // 64)
    gu = upload(W)
    xd = torch_act(x, "f16")
    h1 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F32)
    h2 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F32)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(h1, h2)
    srt = v["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(h1), href, "f32")
    assert err <= TOL, (err, report(to_f64(h1), href))


def test_split_units_q4_k_swiglu_f16():
    N, K, T, E, k = 4096, 1280, 512, 64, 8
    rng = np.random.default_rng(16)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.q4_k(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 2 // 128, KT=K // 64)
    gu = upload(W)
    xd = torch_act(x, "f16")
    h1 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    h2 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(h1, h2)
    srt = v["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(h1), href, "f16")
    assert err <= TOL, (err, report(to_f64(h1), href))


def test_split_units_q6_k_store_f16():
    N, K, T, E, k = 2048, 1280, 512, 64, 8
    rng = np.random.default_rng(12)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.q6_k(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 256, KT=K // 64)
    dw = upload(W)
    xd = torch_act(x, "f16")
    y1 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    y2 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(y1, y2)
    srt = v["sorted"].cpu().numpy()
    yref = _pair_rows(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(y1), yref, "f32")
    assert err <= TOL, (err, report(to_f64(y1), yref))


def test_split_units_fp8_store_f16():
    N, K, T, E, k = 2048, 1280, 512, 64, 8
    rng = np.random.default_rng(12)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.fp8(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 256, KT=K // 64)
    dw = upload(W)
    xd = torch_act(x, "f16")
    y1 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    y2 = qm.moe_gather_qmm(dw, plan, T, k, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(y1, y2)
    srt = v["sorted"].cpu().numpy()
    yref = _pair_rows(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(y1), yref, "f32")
    assert err <= TOL, (err, report(to_f64(y1), yref))


def test_split_units_q8_0_swiglu_f16():
    N, K, T, E, k = 4096, 1280, 512, 64, 8
    rng = np.random.default_rng(16)
    x = synth.activations(rng, T, K, "f16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    W = synth.q8_0(rng, E, N, K)
    plan, v = _plan(ids, T, k, E, n_nt=N // 2 // 128, KT=K // 64)
    gu = upload(W)
    xd = torch_act(x, "f16")
    h1 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    h2 = qm.moe_gather_qmm(gu, plan, T, k, xd, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F16)
    torch.cuda.synchronize()
    _tickets_zero(plan, T, k, E)
    assert torch.equal(h1, h2)
    srt = v["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "f16"), ids, W)[srt]
    err = normwise_err(to_f64(h1), href, "f16")
    assert err <= TOL, (err, report(to_f64(h1), href))


def test_model_of_the_split_rule():
    """The host model itself on hand-made counts (64 workgroups per XCD)."""
    # 17 tiles x 8 column blocks: XCD 0 has 3 tiles = 24 units (< one round): no split
    assert _model_split_units(17, 8, 16, 512) == 0
    # 8 * 9 tiles x 8 column blocks: 72 units per XCD = one round + 8 (<= 16): 8 split per XCD
    assert _model_split_units(72, 8, 16, 512) == 64
    # 8 * 11 tiles x 8: 88 = 64 + 24 (> 16): none
    assert _model_split_units(88, 8, 16, 512) == 0
    # K too short for 4 parts of at least 4 K tiles
    assert _model_split_units(72, 8, 8, 512) == 0
