"""GPU parity of the decode GEMV (moe_gemv) against the fp64 oracle through
the C ABI: the int4 Qwen-shaped decode workload at its real size (hidden 2048,
intermediate 512, top-8 of 256 experts, B in {1, 4, 8}), the other formats at
small sizes, run-to-run identity of the sum-folded combine, and agreement with
the prefill GEMM at T = B."""
import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import TOL, normwise_err, report, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _gemv(x, ids, w, Wgu, Wd, act):
    code = qm.F16 if act == "f16" else qm.BF16
    xd = torch_act(x, act)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    gu_d, d_d = upload(Wgu), upload(Wd)
    h = qm.moe_gemv(gu_d, xd, ids_d, epilogue=qm.EPI_SWIGLU, out_dtype=code)
    out = qm.moe_gemv(d_d, h, ids_d, w_d, epilogue=qm.EPI_WEIGHTED_COMBINE, out_dtype=code)
    torch.cuda.synchronize()
    return h, out, (gu_d, d_d, xd, ids_d, w_d)


def _check(x, ids, w, Wgu, Wd, act):
    B, k = ids.shape
    x64 = oracle.act_to_f64(x, act)
    h, out, dev = _gemv(x, ids, w, Wgu, Wd, act)
    href = oracle.moe_gate_up(x64, ids, Wgu)
    hg = to_f64(h).reshape(B * k, -1)
    e1 = normwise_err(hg, href, act)
    assert e1 <= TOL, ("gate/up", e1, report(hg, href))
    oref = oracle.moe_down_combine(hg, ids, w, Wd)
    og = to_f64(out)
    e2 = normwise_err(og, oref, act)
    assert e2 <= TOL, ("down", e2, report(og, oref))
    return h, out, dev


@pytest.mark.parametrize("B", [1, 4, 8])
def test_gemv_qwen_decode_int4_full_size(B):
    inp = synth.qwen_a3b_decode(B)
    h, out, dev = _check(inp.x, inp.ids, inp.w, inp.w_gate_up, inp.w_down, "bf16")
    # sum-folded combine is deterministic
    gu_d, d_d, xd, ids_d, w_d = dev
    out2 = qm.moe_gemv(d_d, h, ids_d, w_d, epilogue=qm.EPI_WEIGHTED_COMBINE, out_dtype=qm.BF16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("gu,dn,act", [("q8_0", "q8_0", "f16"), ("q8_0", "q8_0", "bf16"),
                                       ("iq2_xxs", "q2_k", "f16"), ("iq2_xxs", "q2_k", "bf16"),
                                       ("int4", "int4", "f16"), ("mxfp4", "mxfp4", "bf16"),
                                       ("mxfp4", "mxfp4", "f16"), ("fp8", "fp8", "bf16"), ("fp8", "fp8", "f16"),
                                       ("q4_k", "q6_k", "f16"), ("q6_k", "q4_k", "bf16"), ("q4_k", "q4_k", "bf16"),
                                       ("q6_k", "q6_k", "f16")])
def test_gemv_formats(gu, dn, act):
    rng = np.random.default_rng(len(gu) * 7 + len(act))
    B, E, k, H, I = 4, 16, 4, 1024, 512
    x = synth.activations(rng, B, H, act)
    ids, w = synth.routing_softmax(rng, B, E, k)
    ids[0] = [1, 2, 3, 4]
    ids[1] = [2, 1, 5, 6]      # shared experts across tokens
    Wgu = synth.int4(rng, E, 2 * I, H) if gu == "int4" else synth.weights(gu, rng, E, 2 * I, H)
    Wd = synth.int4(rng, E, H, I) if dn == "int4" else synth.weights(dn, rng, E, H, I)
    _check(x, ids, w, Wgu, Wd, act)


def test_gemv_matches_prefill_gemm_at_t_eq_b():
    inp = synth.qwen_a3b_decode(4, E=32)
    B, k = inp.ids.shape
    h, out, (gu_d, d_d, xd, ids_d, w_d) = _gemv(inp.x, inp.ids, inp.w, inp.w_gate_up, inp.w_down, "bf16")
    plan = qm.moe_plan(ids_d, inp.E, 16)
    hp = qm.moe_gather_qmm(gu_d, plan, B, k, xd, bm=16, epilogue=qm.EPI_SWIGLU, out_dtype=qm.F32)
    torch.cuda.synchronize()
    srt = qm.plan_views(plan, B, k, inp.E)["sorted"].cpu().numpy()
    a = to_f64(h).reshape(B * k, -1)[srt]
    b = to_f64(hp)
    assert normwise_err(a, b, "bf16") <= TOL


def test_gemv_dropped_ids_contribute_nothing():
    inp = synth.qwen_a3b_decode(2, E=16)
    ids = inp.ids.copy()
    ids[0, 3] = -1
    ids[1, 0] = 16
    w = inp.w.copy()
    w[0, 3] = 0.0
    w[1, 0] = 0.0
    x64 = oracle.act_to_f64(inp.x, "bf16")
    h, out, _ = _gemv(inp.x, ids, inp.w, inp.w_gate_up, inp.w_down, "bf16")
    hg = to_f64(h).reshape(ids.size, -1)
    valid = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < 16)
    ids_c = np.where(valid.reshape(ids.shape), ids, 0)
    oref = oracle.moe_down_combine(np.where(valid[:, None], hg, 0.0), ids_c, w, inp.w_down)
    assert normwise_err(to_f64(out), oref, "bf16") <= TOL


def test_gemv_int4_many_tokens_per_expert():
    # 32 tokens on each of two experts: the int4 kernels take tokens 8 at a time
    rng = np.random.default_rng(12)
    B, E, k, H, I = 32, 2, 2, 512, 256
    x = synth.activations(rng, B, H, "bf16")
    ids = np.tile(np.array([[0, 1]], np.int32), (B, 1))
    ids[::3] = ids[::3, ::-1]
    w = rng.random((B, k)).astype(np.float32)
    _check(x, ids, w, synth.int4(rng, E, 2 * I, H), synth.int4(rng, E, H, I), "bf16")


@pytest.mark.parametrize("group,I", [(32, 512), (32, 1024)])
def test_gemv_int4_generic_shapes(group, I):
    # group 32 takes the generic kernels
    rng = np.random.default_rng(group + I)
    B, E, k, H = 3, 8, 4, 512
    x = synth.activations(rng, B, H, "bf16")
    ids, w = synth.routing_softmax(rng, B, E, k)
    _check(x, ids, w, synth.int4(rng, E, 2 * I, H, group), synth.int4(rng, E, H, I, group), "bf16")


@pytest.mark.parametrize("B,H,I,k,act", [
    (3, 128, 128, 2, "bf16"),    # K = 128: two tiles, a partial run per wave
    (2, 4096, 256, 4, "f16"),    # gate/up K = 4096: eight waves split K
    (5, 512, 1024, 8, "bf16"),   # combine K = 1024, top-8: sixteen waves
    (4, 256, 2048, 2, "f16"),    # combine K = 2048, top-2: four runs per slot
    (9, 512, 512, 8, "bf16"),    # nine tokens: a second pass of activation rows
    (4, 512, 2048, 8, "bf16"),   # combine K = 2048, top-8: generic combine kernel
])
def test_gemv_int4_split_shapes(B, H, I, k, act):
    rng = np.random.default_rng(B * 1000 + H + I + k)
    E = 12
    x = synth.activations(rng, B, H, act)
    ids, w = synth.routing_softmax(rng, B, E, k)
    if B == 9:
        ids[:, 0] = 5  # every token on expert 5
    _check(x, ids, w, synth.int4(rng, E, 2 * I, H), synth.int4(rng, E, H, I), act)


def test_gemv_int4_repeated_expert_within_token():
    # a token may name one expert several times: the expert then has more
    # slots than there are tokens, served over several passes
    rng = np.random.default_rng(77)
    B, E, k, H, I = 2, 4, 4, 256, 128
    x = synth.activations(rng, B, H, "bf16")
    ids = np.array([[1, 1, 1, 1], [1, 1, 2, 2]], np.int32)
    w = rng.random((B, k)).astype(np.float32)
    _check(x, ids, w, synth.int4(rng, E, 2 * I, H), synth.int4(rng, E, H, I), "bf16")


@pytest.mark.parametrize("fmt,act,H,I", [("mxfp4", "f16", 4096, 2048), ("q8_0", "bf16", 1024, 512),
                                         ("iq2_xxs", "f16", 1024, 512), ("fp8", "bf16", 4096, 2048)])
def test_gemv_generic_single_token(fmt, act, H, I):
    # one token per call takes the one-token-per-pass kernels; the token names
    # expert 3 twice (two passes over its weights)
    rng = np.random.default_rng(len(fmt) + H)
    E, k = 8, 6
    x = synth.activations(rng, 1, H, act)
    ids = np.array([[3, 5, 3, 0, 1, 7]], np.int32)
    w = rng.random((1, k)).astype(np.float32)
    Wgu = synth.weights(fmt, rng, E, 2 * I, H)
    Wd = synth.weights(fmt if fmt != "iq2_xxs" else "q2_k", rng, E, H, I)
    _check(x, ids, w, Wgu, Wd, act)


@pytest.mark.parametrize("fmt,act,H,I", [("int4", "bf16", 2048, 512), ("fp8", "f16", 1024, 512),
                                         ("mxfp4", "bf16", 1024, 512)])
def test_gemv_largest_batch(fmt, act, H, I):
    # the largest decode batch a call takes (64 tokens x top-8 = 512 slots),
    # with skewed routing so some experts serve many tokens (several passes)
    rng = np.random.default_rng(64 + len(fmt))
    B, E, k = qm.MAX_GEMV_BATCH, 24, qm.MAX_TOPK
    x = synth.activations(rng, B, H, act)
    ids, w = synth.routing_zipf(rng, B, E, k, 1.1)
    Wgu = synth.int4(rng, E, 2 * I, H) if fmt == "int4" else synth.weights(fmt, rng, E, 2 * I, H)
    Wd = synth.int4(rng, E, H, I) if fmt == "int4" else synth.weights(fmt, rng, E, H, I)
    _check(x, ids, w, Wgu, Wd, act)


@pytest.mark.parametrize("fmt,act", [("fp8", "bf16"), ("mxfp4", "f16"), ("q8_0", "bf16")])
def test_gemv_generic_combine_is_reproducible(fmt, act):
    # the sum-folded combine adds each slot's products in a fixed order: two
    # calls give the same bits, and the result matches the oracle
    rng = np.random.default_rng(5 + len(fmt))
    B, E, k, H, I = 8, 12, 6, 1024, 512
    x = synth.activations(rng, B, H, act)
    ids, w = synth.routing_softmax(rng, B, E, k)
    h, out, dev = _check(x, ids, w, synth.weights(fmt, rng, E, 2 * I, H), synth.weights(fmt, rng, E, H, I), act)
    gu_d, d_d, xd, ids_d, w_d = dev
    code = qm.F16 if act == "f16" else qm.BF16
    out2 = qm.moe_gemv(d_d, h, ids_d, w_d, epilogue=qm.EPI_WEIGHTED_COMBINE, out_dtype=code)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
