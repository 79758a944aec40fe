"""GPU parity of the prefill matmuls (dense qmm and the gathered MoE GEMM)
against the fp64 CPU oracle, through the C ABI.

* exact-integer cases (power-of-two scales, small integer activations) must
  match bit for bit in any summation order;
* random cases must meet the normwise bound (TOL, net of the output rounding);
* MoE cases check each stage against the oracle fed the bytes the GPU stage
  consumed (stage-wise), the deterministic combine for run-to-run identity, and
  the degenerate routings (empty experts, one hot expert, k = 1, dropped ids).
"""
import struct

import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import TOL, normwise_err, report, to_f64, torch_act, upload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FMTS = ["q8_0", "q2_k", "iq2_xxs", "int4", "mxfp4", "fp8", "q4_k", "q6_k"]


def _w(fmt, rng, E, N, K):
    return synth.int4(rng, E, N, K, 64) if fmt == "int4" else synth.weights(fmt, rng, E, N, K)


# ------------------------------------------------------------------ dense

def test_dense_q8_0_smoke_cell():
    # M=32 N=256 K=2048 fp16, Q8_0 weights, fp16 out.
    x, W = synth.dense_q8_0()
    ref = oracle.qmm(oracle.act_to_f64(x, "f16"), W)
    y = qm.qmm_dense(upload(W), torch_act(x, "f16"), qm.EPI_STORE, qm.F16)
    torch.cuda.synchronize()
    err = normwise_err(to_f64(y), ref, "f16")
    assert err <= TOL, (err, report(to_f64(y), ref))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_dense_random_ragged(fmt, act):
    rng = np.random.default_rng(hash((fmt, act)) % 2**32)
    M, N, K = 45, 208, 512    # N: 13 blocks of 16 rows (the tiled layouts), not a multiple of the 256-row tile
    if fmt == "fp8":
        N = 384               # 3 rows of 128 x 128 scale blocks, still not a multiple of the 256-row tile
    W = _w(fmt, rng, 1, N, K)
    x = synth.activations(rng, M, K, act)
    ref = oracle.qmm(oracle.act_to_f64(x, act), W)
    y = qm.qmm_dense(upload(W), torch_act(x, act), qm.EPI_STORE, qm.F32)
    torch.cuda.synchronize()
    err = normwise_err(to_f64(y), ref, "f32")
    assert err <= TOL, (err, report(to_f64(y), ref))


def _exact_weights(fmt, rng, E, N, K):
    """Weights whose decoded values are small integers (exact everywhere)."""
    W = _w(fmt, rng, E, N, K)
    h = lambda v: np.frombuffer(struct.pack("<e", v), np.uint8)
    if fmt == "q8_0":
        W.blocks[..., 0:2] = h(1.0)
        q = W.blocks[..., 2:34].view(np.int8)
        q[...] = np.clip(q, -8, 8)
    elif fmt == "q2_k":
        W.blocks[..., 80:82] = h(1.0)
        W.blocks[..., 82:84] = h(1.0)
    elif fmt == "q4_k":
        W.blocks[..., 0:4] = np.concatenate([h(1.0), h(1.0)])   # values scale*q - min, at most 945
    elif fmt == "q6_k":
        W.blocks[..., 208:210] = h(1.0)                          # values scale*(q - 32), |v| <= 2048
    elif fmt == "mxfp4":
        W.blocks[..., 0] = 128         # scale 2: values 0, +-1, +-2, +-3, +-4, +-6, +-8, +-12
    elif fmt == "fp8":
        # integer-valued E4M3 codes (+-1, 2, 3, 4, 6, 8) under power-of-two block scales
        ints = np.array([0x38, 0x40, 0x44, 0x48, 0x4C, 0x50], np.uint8)
        W.qs[...] = ints[rng.integers(0, 6, size=W.qs.shape)] | (rng.integers(0, 2, size=W.qs.shape) << 7).astype(np.uint8)
        W.scale[...] = np.where(rng.random(W.scale.shape) < 0.5, 1.0, 2.0).astype(np.float32)
    elif fmt == "iq2_xxs":
        W.blocks[..., 0:2] = h(8.0)    # group scale 8 * (0.5 + s) / 4 = 1 + 2s
        W.grid = np.random.default_rng(1).choice(np.array([1, 2, 3], np.uint8), size=(256, 8))
    else:
        W.scale[...] = 0x3C00          # 1.0
        W.bias[...] = 0xC800           # -8.0
    return W


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_dense_exact_integer_bit_exact(fmt, act):
    rng = np.random.default_rng(99)
    M, N, K = 33, (384 if fmt == "fp8" else 144), 512
    W = _exact_weights(fmt, rng, 1, N, K)
    xi = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    x = synth.f16_bits(xi) if act == "f16" else synth.bf16_bits(xi)
    ref = oracle.qmm(oracle.act_to_f64(x, act), W)
    assert np.all(np.abs(ref) < 2 ** 24) and np.array_equal(ref, np.rint(ref))
    y = qm.qmm_dense(upload(W), torch_act(x, act), qm.EPI_STORE, qm.F32)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), ref)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_dense_fp8_every_code_through_the_matmul(act):
    # one-hot activation rows pick single weight columns: y[m, n] = e4m3(w[n, m]) * scale
    # exactly, for every non-NaN E4M3 byte under several block scales
    rng = np.random.default_rng(12)
    N, K = 256, 256
    W = synth.fp8(rng, 1, N, K)
    codes = np.array([b for b in range(256) if b & 0x7F != 0x7F], np.uint8)
    W.qs[0] = codes[(np.arange(K)[None, :] + 5 * np.arange(N)[:, None]) % codes.size]
    W.scale[0] = np.array([[1.0, 2.0 ** -12], [2.0 ** 7, 0.0371]], np.float32)
    one = 0x3C00 if act == "f16" else 0x3F80
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = one
    y = qm.qmm_dense(upload(W), torch_act(x, act), qm.EPI_STORE, qm.F32)
    torch.cuda.synchronize()
    ref = oracle.dequant(W)[0].T             # [K, N]: y[m, n] = w[n, m]
    assert np.array_equal(to_f64(y), ref.astype(np.float64))


def test_dense_swiglu_and_accumulate():
    rng = np.random.default_rng(4)
    M, I, K = 70, 96, 256
    W = _w("q8_0", rng, 1, 2 * I, K)
    x = synth.activations(rng, M, K, "f16")
    x64 = oracle.act_to_f64(x, "f16")
    gu = oracle.qmm(x64, W)
    href = oracle.silu(gu[:, :I]) * gu[:, I:]
    dw = upload(W)
    h = qm.qmm_dense(dw, torch_act(x, "f16"), qm.EPI_SWIGLU, qm.F16)
    acc = torch.ones((M, 2 * I), dtype=torch.float32, device="cuda")
    qm.qmm_dense(dw, torch_act(x, "f16"), qm.EPI_ACCUMULATE, qm.F32, out=acc)
    torch.cuda.synchronize()
    assert normwise_err(to_f64(h), href, "f16") <= TOL
    assert normwise_err(to_f64(acc), gu + 1.0, "f32") <= TOL


# ------------------------------------------------------------------ MoE

def _moe_case(gu_fmt, d_fmt, act, T=200, E=16, k=4, H=512, I=256, seed=3, routing="softmax"):
    rng = np.random.default_rng(seed)
    x = synth.activations(rng, T, H, act)
    ids, w = (synth.routing_zipf if routing == "zipf" else synth.routing_softmax)(rng, T, E, k)
    return x, ids, w, _w(gu_fmt, rng, E, 2 * I, H), _w(d_fmt, rng, E, H, I)


def _run_moe(x, ids, w, Wgu, Wd, act, bm=80, deterministic=False, out_dtype=None):
    T, k = ids.shape
    E = Wgu.E
    code = qm.F16 if act == "f16" else qm.BF16
    xd = torch_act(x, act)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    gu_d, d_d = upload(Wgu), upload(Wd)
    plan = qm.moe_plan(ids_d, E, bm)
    n_valid = int(((ids >= 0) & (ids < E)).sum())
    h = qm.moe_gather_qmm(gu_d, plan, T, k, xd, bm=bm, epilogue=qm.EPI_SWIGLU, out_dtype=code, n_rows=n_valid)
    oc = code if out_dtype is None else out_dtype
    if deterministic:
        y = qm.moe_gather_qmm(d_d, plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, epilogue=qm.EPI_STORE,
                              out_dtype=qm.F32, n_rows=n_valid)
        out = qm.moe_combine(y, plan, T, k, E, w_d, out_dtype=oc)
    else:
        acc = torch.zeros((T, Wd.N), dtype=torch.float32, device="cuda")
        qm.moe_gather_qmm(d_d, plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, topk_w=w_d,
                          epilogue=qm.EPI_WEIGHTED_COMBINE, out=acc)
        out = qm.combine_cast(acc, oc)
        torch.cuda.synchronize()
        assert float(acc.abs().max()) == 0.0  # the cast clears the accumulator
    torch.cuda.synchronize()
    srt = qm.plan_views(plan, T, k, E)["sorted"][:n_valid].cpu().numpy()
    return h, srt, out


def _check_moe(x, ids, w, Wgu, Wd, act, **kw):
    T, k = ids.shape
    x64 = oracle.act_to_f64(x, act)
    h, srt, out = _run_moe(x, ids, w, Wgu, Wd, act, **kw)
    # stage 1: h in sorted order vs the oracle's per-pair h
    href = oracle.moe_gate_up(x64, ids, Wgu)[srt]
    hg = to_f64(h)
    e1 = normwise_err(hg, href, act)
    assert e1 <= TOL, ("gate/up", e1, report(hg, href))
    # stage 2 fed the GPU's h (mapped back to pair order)
    hp = np.zeros((T * k, Wgu.N // 2))
    hp[srt] = hg
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < Wgu.E)
    ids_c = np.where(valid.reshape(ids.shape), ids, 0)
    w_c = np.where(valid.reshape(ids.shape), w, 0).astype(np.float64)
    oref = oracle.moe_down_combine(hp, ids_c, w_c, Wd)
    og = to_f64(out)
    od = {qm.F16: "f16", qm.BF16: "bf16", qm.F32: "f32"}[kw.get("out_dtype") or (qm.F16 if act == "f16" else qm.BF16)]
    e2 = normwise_err(og, oref, od)
    assert e2 <= TOL, ("down+combine", e2, report(og, oref))
    return h, out


@pytest.mark.parametrize("gu,dn,act", [("int4", "int4", "bf16"), ("int4", "int4", "f16"),
                                       ("iq2_xxs", "q2_k", "f16"), ("iq2_xxs", "q2_k", "bf16"),
                                       ("q8_0", "q8_0", "f16"), ("q8_0", "q8_0", "bf16"),
                                       ("mxfp4", "mxfp4", "bf16"), ("mxfp4", "mxfp4", "f16"),
                                       ("fp8", "fp8", "bf16"), ("fp8", "fp8", "f16"),
                                       ("q4_k", "q6_k", "f16"), ("q6_k", "q4_k", "bf16")])
def test_moe_stagewise(gu, dn, act):
    x, ids, w, Wgu, Wd = _moe_case(gu, dn, act, seed=len(gu) + len(act))
    _check_moe(x, ids, w, Wgu, Wd, act)


def test_moe_deterministic_combine_is_reproducible():
    x, ids, w, Wgu, Wd = _moe_case("int4", "int4", "bf16", seed=11)
    _, o1 = _check_moe(x, ids, w, Wgu, Wd, "bf16", deterministic=True)
    _, o2 = _check_moe(x, ids, w, Wgu, Wd, "bf16", deterministic=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("bm", [16, 64, 80])
def test_moe_hot_expert_many_tiles_and_empty_experts(bm):
    # every token picks expert 3 first (300 rows: several tiles), experts 8.. unused
    x, ids, w, Wgu, Wd = _moe_case("int4", "int4", "bf16", T=300, E=12, k=2, seed=21)
    ids[:, 0] = 3
    ids[:, 1] = np.where(ids[:, 1] == 3, 4, ids[:, 1] % 8)
    _check_moe(x, ids, w, Wgu, Wd, "bf16", bm=bm)


def test_moe_top1_dropped_ids_and_single_token():
    x, ids, w, Wgu, Wd = _moe_case("iq2_xxs", "q2_k", "f16", T=37, E=8, k=1, seed=5)
    w[:] = 1.0
    ids[0, 0] = -1
    ids[5, 0] = 99
    _check_moe(x, ids, w, Wgu, Wd, "f16")
    x1, ids1, w1, Wgu1, Wd1 = _moe_case("int4", "int4", "bf16", T=1, E=8, k=8, seed=6)
    _check_moe(x1, ids1, w1, Wgu1, Wd1, "bf16")


def test_moe_single_expert_equals_dense():
    rng = np.random.default_rng(8)
    T, H, I = 77, 256, 128
    W = _w("q8_0", rng, 1, 2 * I, H)
    x = synth.activations(rng, T, H, "f16")
    dw = upload(W)
    xd = torch_act(x, "f16")
    ids = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    plan = qm.moe_plan(ids, 1, 80)
    y_moe = qm.moe_gather_qmm(dw, plan, T, 1, xd, epilogue=qm.EPI_STORE, out_dtype=qm.F32)
    y_dense = qm.qmm_dense(dw, xd, qm.EPI_STORE, qm.F32)
    torch.cuda.synchronize()
    assert torch.equal(y_moe, y_dense)


@pytest.mark.parametrize("N,ydt", [(2048, "bf16"), (2048, "f32"), (1004, "bf16")])
def test_moe_combine_paths(N, ydt):
    # the deterministic top-k combine over sorted rows, with a base, dropped
    # pairs, 16-byte row loads (N % 8 == 0) and the element-wise path
    rng = np.random.default_rng(N + len(ydt))
    T, k, E = 300, 8, 32
    ids, w = synth.routing_softmax(rng, T, E, k)
    ids[5, 2] = -1
    ids[7, 0] = E
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    plan = qm.moe_plan(ids_d, E, 80)
    y64 = rng.standard_normal((T * k, N))
    y = torch.from_numpy(y64.astype(np.float32)).cuda()
    if ydt == "bf16":
        y = y.to(torch.bfloat16)
    base = torch.from_numpy(rng.standard_normal((T, N)).astype(np.float32)).cuda()
    out = qm.moe_combine(y, plan, T, k, E, w_d, base=base, out_dtype=qm.F32)
    out2 = qm.moe_combine(y, plan, T, k, E, w_d, base=base, out_dtype=qm.F32)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    yv = to_f64(y)
    inv = qm.plan_views(plan, T, k, E)["inv"].cpu().numpy().reshape(T, k)
    ref = base.cpu().numpy().astype(np.float64)
    for j in range(k):
        ok = inv[:, j] >= 0
        ref[ok] += w[ok, j, None].astype(np.float64) * yv[inv[ok, j]]
    assert normwise_err(to_f64(out), ref, "f32") <= 1e-6


@pytest.mark.parametrize("N,ydt,rdt,odt,gated,inplace", [
    (2048, "bf16", "bf16", "bf16", True, True),   # 16-byte path, residual updated in place
    (2048, "f32", "f32", "f32", True, False),
    (1004, "bf16", "bf16", "bf16", True, False),  # element-wise path
    (2048, "bf16", None, "f32", False, False),    # ungated shared expert, no residual
    (2048, "bf16", "f16", "bf16", True, False),   # residual in another dtype
    (1000, "f32", None, "bf16", True, False),
])
def test_moe_combine_shared(N, ydt, rdt, odt, gated, inplace):
    # combine + sigmoid-gated shared expert + residual against the oracle's
    # pair combine and post-MoE epilogue
    rng = np.random.default_rng(N + 3 * len(ydt) + (rdt is None))
    T, k, E = 300, 8, 32
    ids, w = synth.routing_softmax(rng, T, E, k)
    ids[5, 2] = -1
    ids[9, 7] = E
    pl = oracle.plan(ids, E, 80)
    ys = rng.standard_normal((len(pl["sorted"]), N)).astype(np.float32)   # rows in expert-sorted order
    shared = rng.standard_normal((T, N)).astype(np.float32)
    glog = (3.0 * rng.standard_normal(T)).astype(np.float32)
    glog[:4] = [0.0, 40.0, -40.0, -200.0]
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    y = torch.from_numpy(ys).cuda().to(dt[ydt])
    res = None if rdt is None else torch.from_numpy(rng.standard_normal((T, N)).astype(np.float32)).cuda().to(dt[rdt])
    plan = qm.moe_plan(torch.from_numpy(ids).cuda(), E, 80)
    args = dict(shared=torch.from_numpy(shared).cuda(), shared_gate=torch.from_numpy(glog).cuda() if gated else None,
                residual=res, out_dtype={"bf16": qm.BF16, "f32": qm.F32}[odt])
    res64 = None if res is None else to_f64(res)
    if inplace:
        args["out"] = res
    out = qm.moe_combine_shared(y, plan, T, k, E, torch.from_numpy(w).cuda(), **args)
    torch.cuda.synchronize()
    yp = np.zeros((T * k, N))
    yp[pl["sorted"]] = to_f64(y)
    ref = oracle.gated_shared_residual(oracle.combine_pairs(yp, ids, w, E), shared, glog if gated else None, res64)
    assert normwise_err(to_f64(out), ref, odt) <= (1e-6 if odt == "f32" else TOL)
    if inplace:
        assert out.data_ptr() == res.data_ptr()


def test_empty_inputs_launch_nothing():
    # T = 0 / M = 0 through the C ABI: every entry point returns QMOE_OK
    # without launching and leaves its output untouched
    import ctypes
    L = qm.lib()
    rng = np.random.default_rng(7)
    dw = upload(_w("int4", rng, 4, 64, 256))
    ws = dw.struct()
    buf = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")      # plan / ids / weights
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    out = torch.full((4, 64), 7.0, dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s = qm._stream()
    assert L.qmoe_moe_plan(P(buf), 0, 2, 4, 80, P(buf), buf.numel() * 4, s) == 0
    assert L.qmoe_moe_gather_qmm(ctypes.byref(ws), P(buf), 0, 2, 80, P(x), qm.BF16, qm.A_GATHER_TOKENS,
                                 None, qm.EPI_STORE, P(out), qm.F32, s) == 0
    wd = upload(_w("int4", rng, 1, 64, 256)).struct()    # dense: one expert
    assert L.qmoe_qmm_dense(ctypes.byref(wd), P(x), qm.BF16, 0, qm.EPI_STORE, P(out), qm.F32, s) == 0
    assert L.qmoe_moe_combine(P(y), qm.F32, P(buf), 0, 2, 4, P(buf), 64, None, P(out), qm.F32, s) == 0
    assert L.qmoe_moe_gemv(ctypes.byref(ws), P(x), qm.BF16, 0, P(buf), None, 2, qm.EPI_STORE, P(out), qm.F32, s) == 0
    assert L.qmoe_router_topk(P(y), qm.F32, 0, 64, 2, qm.ROUTER_SOFTMAX, None, 1.0, P(buf), P(buf), s) == 0
    torch.cuda.synchronize()
    assert float(out.min()) == 7.0 and float(out.max()) == 7.0


@pytest.mark.parametrize("planted", [None, 141, 113, 255])
def test_dense_mxfp4_f16_scale_ranges(planted):
    # fp16 activations: a workgroup whose block scales all lie in 2^-13 .. 2^13
    # folds them into the fp16 operands; one exponent outside that range (or
    # NaN, 0xFF) in the first 256 rows sends that workgroup down the fp32-scale
    # path while the second keeps folding
    rng = np.random.default_rng(33)
    M, N, K = 40, 512, 512
    W = synth.mxfp4(rng, 1, N, K)
    if planted is not None:
        W.blocks[0, 3, 5, 0] = planted
    x = synth.activations(rng, M, K, "f16")
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.qmm(oracle.act_to_f64(x, "f16"), W)
    y = qm.qmm_dense(upload(W), torch_act(x, "f16"), qm.EPI_STORE, qm.F32)
    torch.cuda.synchronize()
    got = to_f64(y)
    if planted == 255:   # a NaN scale poisons exactly the outputs of row 3
        assert np.isnan(got[:, 3]).all() and np.isfinite(np.delete(got, 3, axis=1)).all()
        got, ref = np.delete(got, 3, axis=1), np.delete(ref, 3, axis=1)
    err = normwise_err(got, ref, "f32")
    assert err <= TOL, (err, report(got, ref))


@pytest.mark.parametrize("fmt", ["int4", "q8_0", "mxfp4", "fp8", "q2_k", "iq2_xxs", "q4_k", "q6_k"])
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("epi", ["store", "swiglu"])
def test_two_byte_outputs_whole_rows(fmt, act, epi):
    # 2-byte outputs of the prefill kernels leave through LDS as whole rows:
    # ragged rows and a partial column tile against the oracle, and bit for
    # bit the kernel's own fp32 output rounded to nearest even
    rng = np.random.default_rng(17 + len(act) + len(epi) + len(fmt))
    M, K = 173, 512
    N = 800 if epi == "store" else 704  # 3 full 256-column tiles + 32 / 2 full 128-column tiles + 96
    if fmt == "fp8":
        N = 896 if epi == "store" else 640  # multiples of the 128-row scale blocks
    W = _w(fmt, rng, 1, N, K)
    x = synth.activations(rng, M, K, act)
    code = qm.F16 if act == "f16" else qm.BF16
    ep = qm.EPI_STORE if epi == "store" else qm.EPI_SWIGLU
    z = oracle.qmm(oracle.act_to_f64(x, act), W)
    ref = z if epi == "store" else oracle.silu(z[:, :N // 2]) * z[:, N // 2:]
    Wd, xd = upload(W), torch_act(x, act)
    y = qm.qmm_dense(Wd, xd, ep, code)
    y32 = qm.qmm_dense(Wd, xd, ep, qm.F32)
    torch.cuda.synchronize()
    err = normwise_err(to_f64(y), ref, act)
    assert err <= TOL, (err, report(to_f64(y), ref))
    bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits, oracle.round_out(y32.cpu().numpy(), act))
