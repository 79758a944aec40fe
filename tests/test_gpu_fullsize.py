"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (routing plan with bm = 80, gathered gate/up with SwiGLU,
gathered down into per-pair rows, the deterministic top-k combine), checked
on sampled outputs that the fp64 oracle computes one by one:

  * Qwen3.6-A3B-shaped int4 prefill: T = 2048, H = 2048, E = 256, I = 512, k = 8
  * DSv4-flash-shaped prefill: T = 2048, H = 4096, E = 256, I = 2048, k = 6,
    IQ2_XXS gate/up, Q2_K down, fp16 activations; the same shapes with MXFP4
    experts, with FP8 E4M3 block experts and with Q4_K gate/up and Q6_K down
    (k-quant oracle parity unpinned)
  * mixed-format FFN block: T = 8192, H = 4096, E = 256, I = 2048, k = 8, Zipf
    routing, plus a Q8_0 shared expert and four Q8_0 4096 x 4096 projections,
    bf16 combine output

Stage-wise (each GEMM is fed the bytes the GPU consumed): sampled h entries
against the oracle's gate/up rows, sampled outputs against the oracle's down
rows fed the GPU's h.  End to end: sampled outputs against the oracle's whole
FFN for those tokens, with h rounded to the activation dtype where the GPU
stores it (reading c9) and nothing else taken from the GPU.  Tolerance: the
normwise 2e-3 bound of tests/_helpers.
"""
import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import CODES, TOL, normwise_err, report, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BM = 80  # the benchmark's tile height


def _run_moe(inp, base=None):
    """The benchmark's prefill sequence: plan, gate/up with SwiGLU, down into
    per-pair rows (sorted order, activation dtype), the deterministic top-k
    combine (plus an fp32 base) rounded to the output dtype."""
    T, k, E = inp.T, inp.k, inp.E
    act = CODES[inp.act]
    x = torch_act(inp.x, inp.act)
    ids = torch.from_numpy(inp.ids).cuda()
    w = torch.from_numpy(inp.w).cuda()
    gu, dn = upload(inp.w_gate_up), upload(inp.w_down)
    plan = qm.moe_plan(ids, E, BM)
    h = qm.moe_gather_qmm(gu, plan, T, k, x, bm=BM, epilogue=qm.EPI_SWIGLU, out_dtype=act)
    y = qm.moe_gather_qmm(dn, plan, T, k, h, bm=BM, a_mode=qm.A_SORTED_ROWS, epilogue=qm.EPI_STORE, out_dtype=act)
    out = qm.moe_combine(y, plan, T, k, E, w, base=base, out_dtype=CODES[inp.out])
    del gu, dn
    return x, plan, h, out


def _check_gate_up(inp, plan, h, rng, n_pairs=48, n_cols=64):
    P = inp.T * inp.k
    pairs = rng.choice(P, n_pairs, replace=False)
    cols = rng.choice(inp.I, n_cols, replace=False)
    x64 = oracle.act_to_f64(inp.x, inp.act)
    ref = oracle.moe_gate_up_rows(x64, inp.ids, inp.w_gate_up, pairs, cols)
    pos = qm.plan_views(plan, inp.T, inp.k, inp.E)["inv"].cpu().numpy()
    got = to_f64(h[torch.from_numpy(pos[pairs]).long().cuda()])[:, cols]
    err = normwise_err(got, ref, inp.act)
    assert err <= TOL, ("gate/up", err, report(got, ref))


def _h_rows(inp, plan, h, tokens):
    """fp64 h of every pair of the given tokens, as the GPU stored it."""
    pos = qm.plan_views(plan, inp.T, inp.k, inp.E)["inv"].cpu().numpy()
    pairs = [t * inp.k + j for t in tokens for j in range(inp.k)]
    hh = to_f64(h[torch.from_numpy(pos[pairs]).long().cuda()])
    return {p: hh[i] for i, p in enumerate(pairs)}


def _check_end_to_end(inp, out, rng, n_tokens, n_cols=64, base_rows=None):
    """Sampled outputs against the oracle's FFN for n_tokens tokens: h of every
    pair of those tokens over all I columns, rounded to the activation dtype,
    then down + weighted combine on n_cols sampled columns (plus the shared
    expert's rows, formed the same way, when base_rows is given)."""
    tokens = rng.choice(inp.T, n_tokens, replace=False)
    cols = rng.choice(inp.H, n_cols, replace=False)
    x64 = oracle.act_to_f64(inp.x, inp.act)
    pairs = [int(t) * inp.k + j for t in tokens for j in range(inp.k)]
    h = oracle.moe_gate_up_rows(x64, inp.ids, inp.w_gate_up, pairs, np.arange(inp.I))
    h = oracle.out_to_f64(oracle.round_out(h, inp.act), inp.act)
    ref = oracle.moe_down_rows({p: h[i] for i, p in enumerate(pairs)}, inp.ids, inp.w, inp.w_down, tokens, cols)
    if base_rows is not None:
        ref = ref + base_rows(tokens, cols)
    got = to_f64(out[torch.from_numpy(tokens).long().cuda()])[:, cols]
    err = normwise_err(got, ref, inp.out)
    assert err <= TOL, ("end to end", err, report(got, ref))


def test_fullsize_qwen_a3b_int4_prefill():
    inp = synth.qwen_a3b_prefill(2048)
    rng = np.random.default_rng(101)
    x, plan, h, out = _run_moe(inp)
    torch.cuda.synchronize()
    _check_gate_up(inp, plan, h, rng)
    tokens = rng.choice(inp.T, 24, replace=False)
    cols = rng.choice(inp.H, 64, replace=False)
    ref = oracle.moe_down_rows(_h_rows(inp, plan, h, tokens), inp.ids, inp.w, inp.w_down, tokens, cols)
    got = to_f64(out[torch.from_numpy(tokens).long().cuda()])[:, cols]
    err = normwise_err(got, ref, inp.out)
    assert err <= TOL, ("down+combine", err, report(got, ref))
    _check_end_to_end(inp, out, rng, 16)


@pytest.mark.parametrize("experts", ["iq2_xxs/q2_k", "mxfp4", "fp8", "q4_k/q6_k"])
def test_fullsize_dsv4_flash_prefill(experts):
    make = {"iq2_xxs/q2_k": synth.dsv4_flash_prefill, "mxfp4": synth.dsv4_flash_mxfp4_prefill,
            "fp8": synth.dsv4_flash_fp8_prefill, "q4_k/q6_k": synth.dsv4_flash_kquant_prefill}[experts]
    inp = make(2048)
    rng = np.random.default_rng(102)
    x, plan, h, out = _run_moe(inp)
    torch.cuda.synchronize()
    _check_gate_up(inp, plan, h, rng)
    tokens = rng.choice(inp.T, 16, replace=False)
    cols = rng.choice(inp.H, 64, replace=False)
    ref = oracle.moe_down_rows(_h_rows(inp, plan, h, tokens), inp.ids, inp.w, inp.w_down, tokens, cols)
    got = to_f64(out[torch.from_numpy(tokens).long().cuda()])[:, cols]
    err = normwise_err(got, ref, inp.out)
    assert err <= TOL, ("down+combine", err, report(got, ref))
    _check_end_to_end(inp, out, rng, 8)


def test_fullsize_mixed_ffn_block():
    inp = synth.mixed_ffn(8192)
    rng = np.random.default_rng(103)
    act = CODES[inp.act]
    # shared expert: silu(g) * u, its down projection in fp32 is the combine's base
    sgu, sdn = upload(inp.shared_gate_up), upload(inp.shared_down)
    x0 = torch_act(inp.x, inp.act)
    hs = qm.qmm_dense(sgu, x0, qm.EPI_SWIGLU, act)
    base = qm.qmm_dense(sdn, hs, qm.EPI_STORE, qm.F32)
    x, plan, h, out = _run_moe(inp, base=base)
    proj = [qm.qmm_dense(upload(Wp), x, qm.EPI_STORE, act) for Wp in inp.projections]
    torch.cuda.synchronize()
    _check_gate_up(inp, plan, h, rng)

    x64 = oracle.act_to_f64(inp.x, inp.act)
    tokens = rng.choice(inp.T, 16, replace=False)
    # shared gate/up on sampled tokens and columns
    SI = inp.shared_down.K
    scols = rng.choice(SI, 64, replace=False)
    Wg = oracle.dequant_rows(inp.shared_gate_up, 0, np.concatenate([scols, scols + SI])).astype(np.float64)
    gu = x64[tokens] @ Wg.T
    ref_hs = oracle.silu(gu[:, :64]) * gu[:, 64:]
    tok_d = torch.from_numpy(tokens).long().cuda()
    hs64 = to_f64(hs[tok_d])
    err = normwise_err(hs64[:, scols], ref_hs, inp.act)
    assert err <= TOL, ("shared gate/up", err)
    # routed down + combine + shared down (stage-wise: the GPU's h and hs)
    cols = rng.choice(inp.H, 64, replace=False)
    ref = oracle.moe_down_rows(_h_rows(inp, plan, h, tokens), inp.ids, inp.w, inp.w_down, tokens, cols)
    Wsd = oracle.dequant_rows(inp.shared_down, 0, cols).astype(np.float64)
    ref = ref + hs64 @ Wsd.T
    got = to_f64(out[tok_d])[:, cols]
    err = normwise_err(got, ref, inp.out)
    assert err <= TOL, ("down+combine+shared", err, report(got, ref))
    # end to end: routed FFN plus the shared expert, every h rounded to the
    # activation dtype where the GPU stores it

    def shared_rows(tok, c):
        Wsg = oracle.dequant_rows(inp.shared_gate_up, 0, np.arange(2 * SI)).astype(np.float64)
        g = x64[tok] @ Wsg.T
        hs_ref = oracle.silu(g[:, :SI]) * g[:, SI:]
        hs_ref = oracle.out_to_f64(oracle.round_out(hs_ref, inp.act), inp.act)
        return hs_ref @ oracle.dequant_rows(inp.shared_down, 0, c).astype(np.float64).T

    _check_end_to_end(inp, out, rng, 8, base_rows=shared_rows)
    # the four projections
    for j, Wp in enumerate(inp.projections):
        pc = rng.choice(inp.H, 64, replace=False)
        refp = x64[tokens] @ oracle.dequant_rows(Wp, 0, pc).astype(np.float64).T
        gotp = to_f64(proj[j][tok_d])[:, pc]
        err = normwise_err(gotp, refp, inp.act)
        assert err <= TOL, (f"projection {j}", err, report(gotp, refp))
