"""GPU: the entry point that allocates nothing (the WEIGHTED_COMBINE gathered
matmul and the cast with the library's fixed fp32 accumulator) against the
entry points it stands in for -- qmoe_moe_gather_qmm(WEIGHTED_COMBINE) into a
caller accumulator, then qmoe_combine_cast -- and against the oracle, on two
calls in a row, the second with a smaller input (the fixed array keeps the
first call's contents, which the second must clear)."""
import ctypes

import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import TOL, normwise_err, report, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _stage(T, seed, E=16, k=4, H=1024, I=256):
    rng = np.random.default_rng(seed)
    x = synth.activations(rng, T, H, "bf16")
    ids, w = synth.routing_softmax(rng, T, E, k)
    ids[0, 0] = E + 5                      # one dropped pair
    Wgu, Wd = synth.int4(rng, E, 2 * I, H), synth.int4(rng, E, H, I)
    ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    plan = qm.moe_plan(ids_d, E, 80)
    h = qm.moe_gather_qmm(upload(Wgu), plan, T, k, torch_act(x, "bf16"), epilogue=qm.EPI_SWIGLU,
                          out_dtype=qm.BF16)
    return ids, w, w_d, Wd, upload(Wd), plan, h


def test_no_alloc_combine_matches_caller_accumulator():
    for T, seed, od in ((600, 1, qm.F32), (150, 2, qm.BF16)):   # the second call is smaller
        ids, w, w_d, Wd, dn, plan, h = _stage(T, seed)
        k = ids.shape[1]
        acc = torch.zeros((T, Wd.N), dtype=torch.float32, device="cuda")
        qm.moe_gather_qmm(dn, plan, T, k, h, a_mode=qm.A_SORTED_ROWS, topk_w=w_d,
                          epilogue=qm.EPI_WEIGHTED_COMBINE, out=acc)
        ref_dev = qm.combine_cast(acc, od)
        got = qm.moe_gather_qmm_combine_static(dn, plan, T, k, h, w_d, out_dtype=od)
        torch.cuda.synchronize()
        dt = {qm.F32: "f32", qm.BF16: "bf16"}[od]
        e_dev = normwise_err(to_f64(got), to_f64(ref_dev), dt)
        assert e_dev <= TOL, ("against the caller-accumulator path", T, e_dev)
        # and against the oracle fed the GPU's h (stage-wise)
        srt = qm.plan_views(plan, T, k, Wd.E)["sorted"].cpu().numpy()
        n_valid = int(((ids >= 0) & (ids < Wd.E)).sum())
        hh = to_f64(h)
        h_pairs = np.zeros((T * k, hh.shape[1]))
        h_pairs[srt[:n_valid]] = hh[:n_valid]
        ref = oracle.moe_down_combine(h_pairs, ids, w, Wd)
        e = normwise_err(to_f64(got), ref, dt)
        assert e <= TOL, ("against the oracle", T, e, report(to_f64(got), ref))


def test_no_alloc_rejects_sizes_past_its_array():
    L = qm.lib()
    cap = int(L.qmoe_static_acc_bytes())
    assert cap == 32 << 20
    P = ctypes.c_void_p(256)
    w = qm._Weights(qm.INT4, 16, 2048, 512, 64, 0, 256, 0, 256, 0, 0, 0, 0, 0)
    t_over = cap // (4 * 2048) + 1
    st = L.qmoe_moe_gather_qmm_combine_static(ctypes.byref(w), P, t_over, 4, 80, P, qm.BF16, qm.A_SORTED_ROWS,
                                              P, P, qm.BF16, None)
    assert st == -5
