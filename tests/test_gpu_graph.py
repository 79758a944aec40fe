"""Captured HIP graphs of the hot path replay as launched.

The decode layer (gate/up SwiGLU GEMV, then the sum-folded down GEMV) and the
prefill sequence (routing plan, gathered gate/up with SwiGLU, gathered down
with the top-k weighted scatter-add, cast) are captured once and replayed
several times, with other eager work, a clobbered output and a
synchronisation between replays.  Every replay must reproduce the eager
result: bit for bit where the kernels are deterministic (decode, gate/up),
within the normwise bound where fp32 atomics decide the summation order (the
scatter-add)."""
import numpy as np
import pytest

import block_quantized_moe_amd as qm
import synth
from _helpers import TOL, normwise_err, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def test_graph_decode_layer_replays():
    inp = synth.qwen_a3b_decode(4, E=32)
    x = torch_act(inp.x, "bf16")
    ids = torch.from_numpy(inp.ids).cuda()
    w = torch.from_numpy(inp.w).cuda()
    gu, dn = upload(inp.w_gate_up), upload(inp.w_down)
    B, k = inp.ids.shape
    h = torch.empty((B, k, inp.I), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, inp.H), dtype=torch.bfloat16, device="cuda")

    def layer():
        qm.moe_gemv(gu, x, ids, epilogue=qm.EPI_SWIGLU, out=h)
        qm.moe_gemv(dn, h, ids, w, epilogue=qm.EPI_WEIGHTED_COMBINE, out=out)

    layer()
    torch.cuda.synchronize()
    ref_h, ref = h.clone(), out.clone()
    g = _capture(layer)
    x2 = torch_act(synth.activations(np.random.default_rng(5), B, inp.H, "bf16"), "bf16")
    for rep in range(4):
        h.fill_(float("nan"))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), ref_h.view(torch.int16)), rep
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        # other eager work on the same weights between replays
        qm.moe_gemv(gu, x2, ids, epilogue=qm.EPI_SWIGLU)
        torch.cuda.synchronize()


def test_graph_prefill_sequence_replays():
    inp = synth.qwen_a3b_prefill(256, E=32)
    T, k, E, H, I = inp.T, inp.k, inp.E, inp.H, inp.I
    bm = 80
    x = torch_act(inp.x, "bf16")
    ids = torch.from_numpy(inp.ids).cuda()
    w = torch.from_numpy(inp.w).cuda()
    gu, dn = upload(inp.w_gate_up), upload(inp.w_down)
    plan = torch.empty(qm.plan_bytes(T, k, E, bm) // 4, dtype=torch.int32, device="cuda")
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    acc = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        qm.moe_plan(ids, E, bm, plan=plan)
        qm.moe_gather_qmm(gu, plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU, out=h)
        qm.moe_gather_qmm(dn, plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, topk_w=w,
                          epilogue=qm.EPI_WEIGHTED_COMBINE, out=acc)
        qm.combine_cast(acc, qm.BF16, out=out)  # also clears acc for the next step

    step()
    torch.cuda.synchronize()
    ref_h, ref = h.clone(), to_f64(out)
    g = _capture(step)
    for rep in range(4):
        h.fill_(float("nan"))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), ref_h.view(torch.int16)), rep
        err = normwise_err(to_f64(out), ref, "bf16")
        assert err <= TOL, (rep, err)
        assert torch.count_nonzero(acc).item() == 0, rep
        # other eager work between replays
        qm.moe_gather_qmm(gu, plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU)
        torch.cuda.synchronize()


def test_graph_prefill_store_combine_replays():
    # the bench's prefill step: plan, gate/up SwiGLU, down STORE per pair,
    # deterministic combine -- every replay bit-identical to the eager run
    inp = synth.qwen_a3b_prefill(256, E=32)
    T, k, E, H, I = inp.T, inp.k, inp.E, inp.H, inp.I
    bm = 80
    x = torch_act(inp.x, "bf16")
    ids = torch.from_numpy(inp.ids).cuda()
    w = torch.from_numpy(inp.w).cuda()
    gu, dn = upload(inp.w_gate_up), upload(inp.w_down)
    plan = torch.empty(qm.plan_bytes(T, k, E, bm) // 4, dtype=torch.int32, device="cuda")
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        qm.moe_plan(ids, E, bm, plan=plan)
        qm.moe_gather_qmm(gu, plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU, out=h)
        qm.moe_gather_qmm(dn, plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, epilogue=qm.EPI_STORE, out=y)
        qm.moe_combine(y, plan, T, k, E, w, out=out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(step)
    for rep in range(4):
        out.fill_(float("nan"))
        plan.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        qm.moe_gather_qmm(gu, plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU)
        torch.cuda.synchronize()
