"""GPU checks of the boundary's size contract, through the C ABI:

* any output row count n: the splitters pad the stacked rows to whole
  16-row blocks and the matmul kernels mask the tail (dense qmm, the
  gathered MoE matmul with E * n not a multiple of 16, the decode GEMV);
* decode K that is any multiple of 32 up to 8192 (lanes past a row's last
  32-value chunk are masked; four chunks per lane above 4096);
* standalone dequant of a row count that is not a multiple of 16 (bit-exact);
* a plan whose header names another call (tile height, tokens, top-k,
  experts) makes the gathered matmul and the combine write nothing.

Tolerances: the normwise bound of tests/_helpers (TOL), bit-exact dequant.
"""
import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import TOL, normwise_err, report, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _w(fmt, rng, E, N, K):
    return synth.int4(rng, E, N, K, 64) if fmt == "int4" else synth.weights(fmt, rng, E, N, K)


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "iq2_xxs", "int4", "mxfp4"])
@pytest.mark.parametrize("N", [40, 200])
def test_dense_any_n(fmt, N):
    act = "bf16" if N == 40 else "f16"
    rng = np.random.default_rng(N + len(fmt))
    M, K = 37, 512
    W = _w(fmt, rng, 1, N, K)
    x = synth.activations(rng, M, K, act)
    ref = oracle.qmm(oracle.act_to_f64(x, act), W)
    y = qm.qmm_dense(upload(W), torch_act(x, act), qm.EPI_STORE, qm.F32)
    torch.cuda.synchronize()
    err = normwise_err(to_f64(y), ref, "f32")
    assert err <= TOL, (fmt, N, err, report(to_f64(y), ref))


@pytest.mark.parametrize("gu,dn,act", [("int4", "int4", "bf16"), ("q8_0", "q8_0", "f16"), ("iq2_xxs", "q2_k", "f16")])
def test_gathered_moe_any_n(gu, dn, act):
    """E = 3 experts with gate/up n = 2 * 20 and down n = 56: neither E * n is
    a multiple of 16, so 16-row blocks straddle experts."""
    rng = np.random.default_rng(7)
    T, E, k, H, I, Hd = 50, 3, 2, 512, 20, 56
    x = synth.activations(rng, T, H, act)
    ids, w = synth.routing_softmax(rng, T, E, k)
    Wgu = _w(gu, rng, E, 2 * I, H)
    Kd = 256 if dn in ("q2_k", "iq2_xxs") else 64   # down K = the block multiple nearest above I
    Wd = _w(dn, rng, E, Hd, Kd)
    code = qm.F16 if act == "f16" else qm.BF16
    ids_d = torch.from_numpy(ids).cuda()
    plan = qm.moe_plan(ids_d, E, 80)
    h = qm.moe_gather_qmm(upload(Wgu), plan, T, k, torch_act(x, act), epilogue=qm.EPI_SWIGLU, out_dtype=code)
    # the down stage reads sorted rows of a K = Kd activation: h padded with zeros
    hp = torch.zeros((T * k, Kd), dtype=h.dtype, device="cuda")
    hp[:, :I] = h
    y = qm.moe_gather_qmm(upload(Wd), plan, T, k, hp, a_mode=qm.A_SORTED_ROWS, epilogue=qm.EPI_STORE,
                          out_dtype=qm.F32)
    torch.cuda.synchronize()
    srt = qm.plan_views(plan, T, k, E)["sorted"].cpu().numpy()
    x64 = oracle.act_to_f64(x, act)
    href = oracle.moe_gate_up(x64, ids, Wgu)[srt]
    hg = to_f64(h)
    e1 = normwise_err(hg, href, act)
    assert e1 <= TOL, ("gate/up", e1, report(hg, href))
    flat = ids.reshape(-1)
    h64 = to_f64(hp)
    yref = np.stack([oracle.dequant_rows(Wd, int(flat[p]), np.arange(Hd)).astype(np.float64) @ h64[i]
                     for i, p in enumerate(srt)])
    e2 = normwise_err(to_f64(y), yref, "f32")
    assert e2 <= TOL, ("down", e2, report(to_f64(y), yref))


def _gemv_store_ref(x64, ids, W):
    B, k = ids.shape
    out = np.zeros((B, k, W.N))
    for b in range(B):
        for j in range(k):
            out[b, j] = oracle.dequant_rows(W, int(ids[b, j]), np.arange(W.N)).astype(np.float64) @ x64[b]
    return out


@pytest.mark.parametrize("fmt,K,B,act", [("q8_0", 1408, 3, "f16"), ("int4", 1408, 1, "bf16"),
                                          ("q8_0", 7168, 3, "bf16"), ("q8_0", 7168, 1, "f16"),
                                          ("mxfp4", 3072, 2, "f16"), ("iq2_xxs", 1536, 2, "bf16")])
def test_gemv_generic_k(fmt, K, B, act):
    """Decode GEMV with K / 32 not a power of two (masked lanes) and above
    4096 (four chunks per lane): STORE, SWIGLU and the sum-folded combine."""
    rng = np.random.default_rng(K + B)
    E, k, I = 8, 4, 64
    x = synth.activations(rng, B, K, act)
    ids, w = synth.routing_softmax(rng, B, E, k)
    Wgu = _w(fmt, rng, E, 2 * I, K)
    code = qm.F16 if act == "f16" else qm.BF16
    xd, ids_d = torch_act(x, act), torch.from_numpy(ids).cuda()
    gu = upload(Wgu)
    y = qm.moe_gemv(gu, xd, ids_d, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    h = qm.moe_gemv(gu, xd, ids_d, epilogue=qm.EPI_SWIGLU, out_dtype=code)
    torch.cuda.synchronize()
    x64 = oracle.act_to_f64(x, act)
    yref = _gemv_store_ref(x64, ids, Wgu)
    e1 = normwise_err(to_f64(y), yref, "f32")
    assert e1 <= TOL, ("store", e1, report(to_f64(y), yref))
    href = oracle.silu(yref[..., :I]) * yref[..., I:]
    e2 = normwise_err(to_f64(h), href, act)
    assert e2 <= TOL, ("swiglu", e2)
    # sum-folded down with K = I = 64 (two chunks per row, lanes masked)
    Wd = _w("q8_0" if fmt != "int4" else "int4", rng, E, K, I)
    out = qm.moe_gemv(upload(Wd), h, ids_d, torch.from_numpy(w).cuda(), epilogue=qm.EPI_WEIGHTED_COMBINE,
                      out_dtype=qm.F32)
    torch.cuda.synchronize()
    oref = oracle.moe_down_combine(to_f64(h).reshape(B * k, I), ids, w, Wd)
    e3 = normwise_err(to_f64(out), oref, "f32")
    assert e3 <= TOL, ("combine", e3, report(to_f64(out), oref))


@pytest.mark.parametrize("fmt", ["q8_0", "int4", "mxfp4", "iq2_xxs"])
def test_gemv_any_n(fmt):
    """Decode GEMV on weights with n = 40 rows per expert (E * n = 320 not a
    multiple of 16 per expert block): STORE and the sum-folded combine."""
    rng = np.random.default_rng(40 + len(fmt))
    B, E, k, K, N = 3, 8, 4, 512, 40
    x = synth.activations(rng, B, K, "f16")
    ids, w = synth.routing_softmax(rng, B, E, k)
    W = _w(fmt, rng, E, N, K)
    xd, ids_d = torch_act(x, "f16"), torch.from_numpy(ids).cuda()
    dw = upload(W)
    y = qm.moe_gemv(dw, xd, ids_d, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    a = synth.activations(rng, B * k, K, "f16").reshape(B, k, K)
    out = qm.moe_gemv(dw, torch_act(a, "f16"), ids_d, torch.from_numpy(w).cuda(),
                      epilogue=qm.EPI_WEIGHTED_COMBINE, out_dtype=qm.F32)
    torch.cuda.synchronize()
    yref = _gemv_store_ref(oracle.act_to_f64(x, "f16"), ids, W)
    assert normwise_err(to_f64(y), yref, "f32") <= TOL
    oref = oracle.moe_down_combine(oracle.act_to_f64(a, "f16").reshape(B * k, K), ids, w, W)
    e = normwise_err(to_f64(out), oref, "f32")
    assert e <= TOL, (e, report(to_f64(out), oref))


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "iq2_xxs", "int4", "mxfp4"])
def test_dequant_any_row_count(fmt):
    rng = np.random.default_rng(20)
    rows, K = 20, 512
    W = _w(fmt, rng, 1, rows, K)
    ref = oracle.dequant(W)
    for code, rnd in ((qm.F32, None), (qm.F16, "f16"), (qm.BF16, "bf16")):
        got = qm.dequant(upload(W), code)
        torch.cuda.synchronize()
        if rnd is None:
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.astype(np.float32).view(np.uint32))
        else:
            bits = got.cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(bits, oracle.round_out(ref, rnd))


def test_plan_header_mismatch_writes_nothing():
    """A plan built for another tile height, token count or expert count
    gives the gathered matmul no tiles and the combine nothing to write, so
    the outputs keep their previous contents."""
    rng = np.random.default_rng(5)
    T, E, k, H, I = 40, 6, 2, 256, 64
    x = synth.activations(rng, T, H, "bf16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    Wgu = synth.int4(rng, E, 2 * I, H)
    gu = upload(Wgu)
    ids_d = torch.from_numpy(ids).cuda()
    xd = torch_act(x, "bf16")
    sentinel = torch.full((T * k, I), 3.0, dtype=torch.bfloat16, device="cuda")
    for bm_plan, bm_call in ((64, 80), (80, 48)):
        plan = qm.moe_plan(ids_d, E, bm_plan)
        h = sentinel.clone()
        qm.moe_gather_qmm(gu, plan, T, k, xd, bm=bm_call, epilogue=qm.EPI_SWIGLU, out=h)
        torch.cuda.synchronize()
        assert torch.equal(h, sentinel), (bm_plan, bm_call)
    # a plan for fewer tokens: same buffer size class, other header
    plan = qm.moe_plan(ids_d[: T // 2].contiguous(), E, 80, plan=torch.zeros(qm.plan_bytes(T, k, E, 80) // 4,
                                                                                 dtype=torch.int32, device="cuda"))
    h = sentinel.clone()
    qm.moe_gather_qmm(gu, plan, T, k, xd, bm=80, epilogue=qm.EPI_SWIGLU, out=h)
    y = torch.ones((T * k, I), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, I), 5.0, dtype=torch.bfloat16, device="cuda")
    qm.moe_combine(y, plan, T, k, E, torch.from_numpy(w).cuda(), out=out)
    torch.cuda.synchronize()
    assert torch.equal(h, sentinel)
    assert torch.equal(out, torch.full_like(out, 5.0))
    # the matching plan still works
    plan = qm.moe_plan(ids_d, E, 80)
    h = qm.moe_gather_qmm(gu, plan, T, k, xd, bm=80, epilogue=qm.EPI_SWIGLU, out_dtype=qm.BF16)
    torch.cuda.synchronize()
    srt = qm.plan_views(plan, T, k, E)["sorted"].cpu().numpy()
    href = oracle.moe_gate_up(oracle.act_to_f64(x, "bf16"), ids, Wgu)[srt]
    assert normwise_err(to_f64(h), href, "bf16") <= TOL
