"""Benchmark of the block-quantized MoE expert matmul on one MI355X.

Step (the timed unit of `value`): one pass of the whole prefill MoE hot path
over the Qwen3.6-A3B-shaped int4 workload -- routing plan, gathered gate/up
GEMM with the SwiGLU epilogue, gathered down GEMM into per-pair rows, and the
deterministic top-k weighted combine -- for T = 2048 tokens, hidden 2048, 256
experts, top-8, expert intermediate 512, bf16 activations, int4 affine
weights (group 64).  The weights rotate over R copies so no step finds them
in the 256 MB Infinity Cache.  `value` is algorithmic TFLOP/s of that step
(routed pairs only; padding is not counted), from the wall clock over K
steps; per-step and per-kernel times (HIP events on the launch stream) are
reported as p10 / p50 / p90.

Also in the same JSON line:
  * roofline       the headline workload's dominant kernel (int4 gate/up);
  * rooflines      every workload's kernels against their own bound: the
                   Qwen-shaped down GEMM and combine, the DSv4-flash-shaped
                   prefill (IQ2_XXS gate/up, Q2_K down, fp16; also with MXFP4
                   and FP8 block experts), the mixed-format FFN block
                   (T = 8192, Zipf routing, Q8_0 shared expert and four Q8_0
                   4096 x 4096 projections) and the decode kernels;
  * dense_q8_0     the M=32 N=256 K=2048 dense Q8_0 cell (launch-bound);
  * decode         the Qwen-shaped decode GEMV (B in {1, 4, 8}, 40 layers
                   with their own weight copies) as graph replays;
  * imbalance      per-expert row statistics of the Zipf-routed block;
  * cpu_baseline   the oracle on the headline workload, and cpu_oracle on
                   bounded samples of the others (1-core and all-core C1).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-extra]
                    [--only {qwen,dense,decode,dsv4,dsv4-mxfp4,dsv4-fp8,dsv4-kquant,mixed,router}]

Counter calibration and traffic records (see profiles/):
    python bench.py --copy-probe MIB
    python bench.py --summarize-traffic NAME KERNEL ALG_BYTES FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR MIB
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16 = 2.5166e15   # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
PEAK_HBM = 8.0e12            # bytes/s
N_CU = 256


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(values, scale=1.0):
    v = np.asarray(values, dtype=np.float64) * scale
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.median(v)), "p90": float(np.percentile(v, 90))}


def act_tensor(torch, bits, dtype="bf16"):
    """uint16 bit patterns -> an fp16 / bf16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to("cuda")


def upload(qm, W):
    if W.fmt == "int4":
        return qm.upload("int4", W.E, W.N, W.K, qs=W.qs, scale=W.scale, bias=W.bias, group=W.group)
    if W.fmt == "fp8":
        return qm.upload("fp8", W.E, W.N, W.K, qs=W.qs, scale=W.scale)
    return qm.upload(W.fmt, W.E, W.N, W.K, blocks=W.blocks, grid=W.grid)


def roof(kernel, workload, flops, nbytes, t, traffic=None, note=None):
    """A kernel against its own roofline: algorithmic bytes and flops per
    launch over the launch's duration; the bound is whichever peak the work
    needs longer on."""
    hbm = nbytes / t / PEAK_HBM
    mfma = flops / t / PEAK_MFMA_BF16
    bound = "hbm" if nbytes / PEAK_HBM >= flops / PEAK_MFMA_BF16 else "mfma"
    r = {"kernel": kernel, "workload": workload, "bound": bound,
         "achieved": nbytes / t / 1e9 if bound == "hbm" else flops / t / 1e12,
         "peak": PEAK_HBM / 1e9 if bound == "hbm" else PEAK_MFMA_BF16 / 1e12,
         "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
         "frac": hbm if bound == "hbm" else mfma, "traffic": traffic,
         "algorithmic_bytes_per_launch": int(nbytes), "algorithmic_flops_per_launch": float(flops),
         "launch_us": t * 1e6, "hbm_frac": hbm, "mfma_frac": mfma}
    if note:
        r["note"] = note
    return r


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def prefill_inputs(T):
    import synth
    return synth.qwen_a3b_prefill(T)


def algorithmic(inp, wbytes_gu=None, wbytes_dn=None):
    """Flops and bytes of one prefill step (routed pairs only), and of each
    kernel as launched (the down GEMM writes per-pair rows that the combine
    reads back)."""
    P = int(((inp.ids >= 0) & (inp.ids < inp.E)).sum())
    H, I, T = inp.H, inp.I, inp.T
    act = 2
    wgu = inp.w_gate_up.nbytes if wbytes_gu is None else wbytes_gu
    wdn = inp.w_down.nbytes if wbytes_dn is None else wbytes_dn
    flops_gu = 2.0 * P * (2 * I) * H
    flops_dn = 2.0 * P * H * I
    ob = 2 if inp.out in ("f16", "bf16") else 4
    base = T * H * 4 if inp.shared_gate_up is not None else 0  # the shared expert's fp32 rows, read by the combine
    return dict(P=P, flops=flops_gu + flops_dn, flops_gu=flops_gu, flops_dn=flops_dn,
                # the method's bytes: weights, x, h written and read once, out
                bytes=wgu + wdn + T * H * act + 2 * P * I * act + T * H * ob,
                bytes_gu=wgu + T * H * act + P * I * act,                 # weights + x read + h write
                bytes_dn=wdn + P * I * act + P * H * act,                 # weights + h read + y rows write
                bytes_cb=P * H * act + T * inp.k * 8 + base + T * H * ob)  # y rows + plan/w (+ base) read, out write


def run_prefill(args, torch, qm, inp, R, steps, warmup, bm=80):
    """The prefill step of a workload: plan, gate/up with SwiGLU, down into
    per-pair rows, the deterministic combine (plus the shared expert into the
    combine's fp32 base when the workload has one).  Returns the wall time per
    step over `steps` launched back to back and event timings per step and
    per kernel over another `steps`."""
    dev = "cuda"
    codes = {"f16": qm.F16, "bf16": qm.BF16}
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    x = act_tensor(torch, inp.x, inp.act)
    ids = torch.from_numpy(inp.ids).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    gu0, dn0 = upload(qm, inp.w_gate_up), upload(qm, inp.w_down)
    gus = [gu0] + [gu0.clone() for _ in range(R - 1)]
    dns = [dn0] + [dn0.clone() for _ in range(R - 1)]
    T, k, E, H, I = inp.T, inp.k, inp.E, inp.H, inp.I
    plan = torch.empty(qm.plan_bytes(T, k, E, bm) // 4, dtype=torch.int32, device=dev)
    h = torch.empty((T * k, I), dtype=tdt[inp.act], device=dev)
    y = torch.empty((T * k, H), dtype=tdt[inp.act], device=dev)
    out = torch.empty((T, H), dtype=tdt[inp.out], device=dev)
    shared = inp.shared_gate_up is not None
    base = None
    if shared:
        sgu, sdn = upload(qm, inp.shared_gate_up), upload(qm, inp.shared_down)
        hs = torch.empty((T, inp.shared_down.K), dtype=tdt[inp.act], device=dev)
        base = torch.empty((T, H), dtype=torch.float32, device=dev)
    names = ["plan", "gate_up", "down"] + (["shared"] if shared else []) + ["combine"]

    def step(i, timed):
        marks = []

        def mark():
            if timed:
                marks.append(torch.cuda.Event(enable_timing=True))
                marks[-1].record()

        mark()
        qm.moe_plan(ids, E, bm, plan=plan)
        mark()
        qm.moe_gather_qmm(gus[i % R], plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU, out=h)
        mark()
        qm.moe_gather_qmm(dns[i % R], plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, epilogue=qm.EPI_STORE, out=y)
        mark()
        if shared:
            qm.qmm_dense(sgu, x, qm.EPI_SWIGLU, codes[inp.act], out=hs)
            qm.qmm_dense(sdn, hs, qm.EPI_STORE, qm.F32, out=base)
            mark()
        qm.moe_combine(y, plan, T, k, E, w, base=base, out=out)
        mark()
        return marks

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    # K steps launched from the host back to back, wall clock (a HIP graph of
    # the step measured slower here than the four host launches it replaces)
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, False)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    all_marks = [step(i, True) for i in range(steps)]
    torch.cuda.synchronize()
    kern = {n: [m[j].elapsed_time(m[j + 1]) * 1e-3 for m in all_marks] for j, n in enumerate(names)}
    step_t = [m[0].elapsed_time(m[-1]) * 1e-3 for m in all_marks]
    res = dict(wall=wall, kern=kern, step=step_t, wbytes_gu=gu0.nbytes, wbytes_dn=dn0.nbytes)
    if inp.projections:
        ps = [upload(qm, Wp) for Wp in inp.projections]
        yp = torch.empty((T, H), dtype=tdt[inp.act], device=dev)
        for Wp in ps:
            qm.qmm_dense(Wp, x, qm.EPI_STORE, codes[inp.act], out=yp)
        torch.cuda.synchronize()
        per = []
        for _ in range(steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(len(ps) + 1)]
            e[0].record()
            for j, Wp in enumerate(ps):
                qm.qmm_dense(Wp, x, qm.EPI_STORE, codes[inp.act], out=yp)
                e[j + 1].record()
            per.append(e)
        torch.cuda.synchronize()
        res["projection"] = [p[j].elapsed_time(p[j + 1]) * 1e-3 for p in per for j in range(len(ps))]
        res["projection_bytes"] = ps[0].nbytes
        del ps
    del gus, dns
    torch.cuda.empty_cache()
    return res


def imbalance(inp, bm=80, bn_gu=128, bn_dn=256):
    """Per-expert row statistics of a routing, and what they do to the
    gathered matmuls' launches (tiles of at most bm rows; gate/up workgroups
    cover bn_gu output columns, down workgroups bn_dn)."""
    flat = inp.ids.reshape(-1)
    c = np.bincount(flat[(flat >= 0) & (flat < inp.E)], minlength=inp.E)
    tiles = int(np.sum((c + bm - 1) // bm))
    rows16 = int(np.sum((c + 15) // 16 * 16))
    wg_gu = tiles * -(-inp.I // bn_gu)
    wg_dn = tiles * -(-inp.H // bn_dn)
    return {"rows_per_expert": {"max": int(c.max()), "median": float(np.median(c)), "min": int(c.min()),
                                "mean": float(c.mean()), "empty_experts": int((c == 0).sum())},
            "hottest_expert_share": float(c.max() / c.sum()),
            "tiles_bm80": tiles, "hottest_expert_tiles": int(-(-c.max() // bm)),
            "rows_padded_to_16_over_routed": rows16 / float(c.sum()),
            "gate_up_workgroups": wg_gu, "gate_up_workgroups_per_cu": wg_gu / N_CU,
            "down_workgroups": wg_dn, "down_workgroups_per_cu": wg_dn / N_CU}


def prefill_line(name, inp, res, R):
    alg = algorithmic(inp, res["wbytes_gu"], res["wbytes_dn"])
    kern = res["kern"]
    t_step = float(np.median(res["step"]))
    flops = alg["flops"]
    if inp.shared_gate_up is not None:
        flops += 2.0 * inp.T * 3 * inp.shared_down.K * inp.H
    out = dict(workload=inp.name, tokens=inp.T, hidden=inp.H, intermediate=inp.I, experts=inp.E, top_k=inp.k,
               weights=f"gate/up {inp.w_gate_up.fmt}, down {inp.w_down.fmt}"
                       + (", shared expert q8_0" if inp.shared_gate_up is not None else ""),
               activations=inp.act, weight_copies_rotated=R, ms_per_step=t_step * 1e3,
               step_us=pct(res["step"], 1e6), tflops=flops / t_step / 1e12, mfma_frac=flops / t_step / PEAK_MFMA_BF16,
               tokens_per_s=inp.T / t_step,
               kernels_us={n: pct(v, 1e6) for n, v in kern.items()})
    rl = [roof(f"gate/up {inp.w_gate_up.fmt} SWIGLU", name, alg["flops_gu"], alg["bytes_gu"],
               float(np.median(kern["gate_up"])), traffic_from_profiles(f"gate_up_{name}")),
          roof(f"down {inp.w_down.fmt} STORE (per-pair rows)", name, alg["flops_dn"], alg["bytes_dn"],
               float(np.median(kern["down"])), traffic_from_profiles(f"down_{name}")),
          roof("combine (deterministic, fp32)", name, 2.0 * alg["P"] * inp.H, alg["bytes_cb"],
               float(np.median(kern["combine"])))]
    if "projection" in res:
        pf = 2.0 * inp.T * inp.H * inp.H
        pb = res["projection_bytes"] + 2 * inp.T * inp.H * 2
        tp = float(np.median(res["projection"]))
        out["projections"] = dict(count=len(inp.projections), us_each=pct(res["projection"], 1e6),
                                  tflops=pf / tp / 1e12, mfma_frac=pf / tp / PEAK_MFMA_BF16)
        rl.append(roof("dense q8_0 projection 4096x4096", name, pf, pb, tp))
    return out, rl


# ---------------------------------------------------------------------------
# dense Q8_0 cell, router, decode
# ---------------------------------------------------------------------------

def graph_time(torch, fn, n, reps=5):
    """Seconds per call of fn, from a captured graph of n calls replayed reps
    times (no host launch gaps); events on the replay stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (reps * n)
    del g
    return t


def run_launch_floor(torch, layers):
    """The floor a decode layer's two dependent launches sit on: per-launch
    time of a graph of 2 x layers trivial fills (16 floats), and of a graph of
    2 x layers gathers of 8 rows (32 KB) from a different cold 8 MB matrix
    each time, the smallest kernel that, like a decode GEMV, waits on HBM."""
    n = 2 * layers
    small = torch.zeros(16, device="cuda")
    big = [torch.randn(256, 8192, device="cuda") for _ in range(n)]
    ids = torch.randint(0, 256, (8,), device="cuda")
    out = torch.empty(8, 8192, device="cuda")
    t_fill = graph_time(torch, lambda i: small.fill_(1.0), n, reps=10)
    t_gather = graph_time(torch, lambda i: torch.index_select(big[i], 0, ids, out=out), n, reps=10)
    del big
    return {"us_per_launch_fill": t_fill * 1e6, "us_per_launch_cold_gather_8_rows": t_gather * 1e6,
            "us_per_layer_two_dependent_launches": 2 * t_gather * 1e6,
            "note": "graph replays on one stream; a decode layer (gate/up GEMV, then down GEMV) cannot go below "
                    "two dependent launches that each wait on HBM"}


def run_dense_cell(torch, qm):
    """Dense Q8_0 qmm M=32 N=256 K=2048, fp16 in / out: a launch-bound
    correctness cell, timed as graph-replayed launches and as single event-
    timed launches."""
    import synth
    x, W = synth.dense_q8_0()
    dw = upload(qm, W)
    xd = act_tensor(torch, x, "f16")
    y = torch.empty((32, 256), dtype=torch.float16, device="cuda")
    for _ in range(3):
        qm.qmm_dense(dw, xd, qm.EPI_STORE, qm.F16, out=y)
    torch.cuda.synchronize()
    t = graph_time(torch, lambda i: qm.qmm_dense(dw, xd, qm.EPI_STORE, qm.F16, out=y), 200)
    ev = []
    for _ in range(20):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        qm.qmm_dense(dw, xd, qm.EPI_STORE, qm.F16, out=y)
        e[1].record()
        ev.append(e)
    torch.cuda.synchronize()
    flops = 2.0 * 32 * 256 * 2048
    nbytes = dw.nbytes + 32 * 2048 * 2 + 32 * 256 * 2
    te = [e[0].elapsed_time(e[1]) * 1e-3 for e in ev]
    return {"workload": "dense q8_0 qmm M=32 N=256 K=2048 fp16", "bound": "launch",
            "us_per_launch_graph": t * 1e6, "us_per_launch_event": pct(te, 1e6),
            "tflops": flops / t / 1e12, "GBps": nbytes / t / 1e9,
            "mfma_frac": flops / t / PEAK_MFMA_BF16, "hbm_frac": nbytes / t / PEAK_HBM,
            "algorithmic_flops": flops, "algorithmic_bytes": int(nbytes),
            "note": "33.6 MFLOP and 0.7 MB take 13 ns on the matrix cores and 88 ns of HBM at peak; "
                    "the launch and the kernel's fixed latency set its time"}


def run_router(torch, qm):
    """Device router top-k ahead of the plan: per-launch time from a replayed
    graph of launches, and the HBM rate of its algorithmic bytes (logits and
    bias read, ids and weights written)."""
    import synth
    rows = []
    for name, T, E, k, dt, scoring in (("qwen3.6-a3b-shaped softmax top-8", 2048, 256, 8, "bf16", qm.ROUTER_SOFTMAX),
                                       ("qwen3.6-a3b-shaped softmax top-8, decode batch", 8, 256, 8, "bf16",
                                        qm.ROUTER_SOFTMAX),
                                       ("dsv4-flash-shaped sqrtsoftplus top-6", 2048, 288, 6, "f32",
                                        qm.ROUTER_SQRTSOFTPLUS)):
        rng = np.random.default_rng(E)
        x = synth.router_logits(rng, T, E, dt, 2.0)
        L = torch.from_numpy(x).cuda() if dt == "f32" else act_tensor(torch, x)
        bias = torch.from_numpy((0.1 * rng.standard_normal(E)).astype(np.float32)).cuda() \
            if scoring == qm.ROUTER_SQRTSOFTPLUS else None
        scale = 1.5 if bias is not None else 1.0
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        for _ in range(3):
            qm.router_topk(L, k, scoring, bias, scale, ids, w)
        torch.cuda.synchronize()
        t = graph_time(torch, lambda i: qm.router_topk(L, k, scoring, bias, scale, ids, w), 100)
        nbytes = L.numel() * L.element_size() + T * k * 8 + (E * 4 if bias is not None else 0)
        rows.append({"workload": name, "tokens": T, "experts": E, "top_k": k, "logits": dt,
                     "us_per_launch": t * 1e6, "GBps": nbytes / t / 1e9, "hbm_frac": nbytes / t / PEAK_HBM,
                     "bytes_per_launch": nbytes})
    return rows


def run_decode(args, torch, qm, B, layers, inp=None):
    """One decode layer step (gate/up SwiGLU GEMV, then the sum-folded down
    GEMV) over `layers` copies of the weights, each read cold: the layer time
    from a graph replay of all layers, each kernel alone from graphs of its
    launches only, plus eager and event-timed figures."""
    import synth
    inp = synth.qwen_a3b_decode(B) if inp is None else inp
    dev = "cuda"
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[inp.act]
    x = act_tensor(torch, inp.x, inp.act)
    ids = torch.from_numpy(inp.ids).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    gu0, dn0 = upload(qm, inp.w_gate_up), upload(qm, inp.w_down)
    gus = [gu0] + [gu0.clone() for _ in range(layers - 1)]
    dns = [dn0] + [dn0.clone() for _ in range(layers - 1)]
    h = torch.empty((B, inp.k, inp.I), dtype=tdt, device=dev)
    out = torch.empty((B, inp.H), dtype=tdt, device=dev)
    uniq = np.unique(inp.ids)
    pe_gu, pe_dn = gu0.nbytes // inp.E, dn0.nbytes // inp.E
    bytes_gu = len(uniq) * pe_gu + B * inp.H * 2 + B * inp.k * inp.I * 2
    bytes_dn = len(uniq) * pe_dn + B * inp.k * inp.I * 2 + B * inp.H * 2
    nbytes = bytes_gu + bytes_dn   # the layer: weights, x, h written and read, out

    def gate_up(l):
        qm.moe_gemv(gus[l], x, ids, epilogue=qm.EPI_SWIGLU, out=h)

    def down(l):
        qm.moe_gemv(dns[l], h, ids, w, epilogue=qm.EPI_WEIGHTED_COMBINE, out=out)

    def layer(l):
        gate_up(l)
        down(l)

    for _ in range(2):
        for l in range(layers):
            layer(l)
    torch.cuda.synchronize()
    reps = max(1, args.decode_reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for l in range(layers):
            layer(l)
    e1.record()
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) * 1e-3 / (reps * layers)
    t_graph = graph_time(torch, layer, layers, reps)
    t_gu = graph_time(torch, gate_up, layers, reps)
    t_dn = graph_time(torch, down, layers, reps)
    del gus, dns
    torch.cuda.empty_cache()
    f_gu = 2.0 * B * inp.k * 2 * inp.I * inp.H
    f_dn = 2.0 * B * inp.k * inp.I * inp.H
    # traffic records: decode_gate_up_b{B} for the int4 Qwen-shaped layer, decode_gate_up_<fmt>_b{B} for others
    tkey = "" if inp.w_gate_up.fmt == "int4" else "_" + inp.w_gate_up.fmt
    rl = [roof("decode gate/up SWIGLU GEMV", inp.name, f_gu, bytes_gu, t_gu,
               traffic_from_profiles(f"decode_gate_up{tkey}_b{B}"), note="graph of the layers' gate/up launches only"),
          roof("decode down sum-folded GEMV", inp.name, f_dn, bytes_dn, t_dn,
               traffic_from_profiles(f"decode_down{tkey}_b{B}"), note="graph of the layers' down launches only")]
    return dict(workload=inp.name, B=B, layers=layers, unique_experts=int(len(uniq)), bytes_per_layer=int(nbytes),
                us_per_layer_graph=t_graph * 1e6, us_per_layer_eager=t_eager * 1e6,
                us_gate_up_graph=t_gu * 1e6, us_down_graph=t_dn * 1e6,
                GBps=nbytes / t_graph / 1e9, hbm_frac=nbytes / t_graph / PEAK_HBM,
                GBps_eager=nbytes / t_eager / 1e9, tokens_per_s_per_layer=B / t_graph), rl


# ---------------------------------------------------------------------------
# CPU oracle baselines
# ---------------------------------------------------------------------------

def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_usable": aff}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(inp, n_tokens):
    """The oracle, as it stands, on a bounded sample of the headline workload:
    the full MoE FFN (gate/up + SwiGLU, down, weighted combine) for the first
    n_tokens tokens, in fp64."""
    import oracle
    ids, w = inp.ids[:n_tokens], inp.w[:n_tokens]
    x64 = oracle.act_to_f64(inp.x[:n_tokens], inp.act)
    t0 = time.perf_counter()
    oracle.moe_ffn(x64, ids, w, inp.w_gate_up, inp.w_down, h_dtype=inp.act)
    dt = time.perf_counter() - t0
    P = ids.size
    flops = 2.0 * P * (3 * inp.I * inp.H)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(_blas_threads()), kind="oracle",
                sample=f"first {n_tokens} of {inp.T} tokens ({P} routed pairs) of the prefill workload, "
                       f"fp64 oracle, {dt:.1f} s", tokens_per_s=n_tokens / dt, seconds=dt)


def cpu_sample_experts(inp, experts):
    """The oracle's MoE FFN on the routed pairs of a few experts only (every
    token with such a pair, its other pairs dropped): the oracle's cost is
    per expert decoded plus the pairs' fp64 products, so a handful of experts
    bounds the run."""
    import oracle
    keep = np.isin(inp.ids, experts)
    rows = np.nonzero(keep.any(axis=1))[0]
    ids = np.where(keep, inp.ids, -1)[rows]
    x64 = oracle.act_to_f64(inp.x[rows], inp.act)
    t0 = time.perf_counter()
    oracle.moe_ffn(x64, ids, inp.w[rows], inp.w_gate_up, inp.w_down, h_dtype=inp.act)
    dt = time.perf_counter() - t0
    P = int(keep.sum())
    flops = 2.0 * P * 3 * inp.I * inp.H
    return dict(workload=inp.name, kind="oracle", gflops=flops / dt / 1e9, seconds=dt, routed_pairs=P,
                cores=int(_blas_threads()),
                sample=f"the {P} routed pairs of experts {list(map(int, experts))} ({len(rows)} tokens), fp64 oracle")


def cpu_dense_cell():
    """The oracle's dense Q8_0 qmm M=32 N=256 K=2048 on all cores and on one."""
    import oracle
    import synth
    x, W = synth.dense_q8_0()
    x64 = oracle.act_to_f64(x, "f16")
    flops = 2.0 * 32 * 256 * 2048

    def timed():
        oracle.qmm(x64, W)
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            oracle.qmm(x64, W)
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    res = []
    t = timed()
    res.append(dict(workload="dense q8_0 qmm M=32 N=256 K=2048", kind="oracle", cores=int(_blas_threads()),
                    seconds=t, gflops=flops / t / 1e9, sample="whole cell, median of 5 after one warm-up"))
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t = timed()
        res.append(dict(workload="dense q8_0 qmm M=32 N=256 K=2048", kind="oracle", cores=1, seconds=t,
                        gflops=flops / t / 1e9, sample="whole cell, median of 5 after one warm-up"))
    except Exception as e:  # threadpoolctl missing: report what ran
        res.append(dict(kind="oracle", cores=1, error=str(e)))
    return res


# ---------------------------------------------------------------------------
# counter records
# ---------------------------------------------------------------------------

def copy_probe(mb, reps=20):
    """A plain device copy of known size (the runtime's copy kernel), run under
    rocprofv3 --pmc to calibrate FETCH_SIZE / WRITE_SIZE against true bytes."""
    import torch
    a = torch.ones(mb << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {mb} MiB")


def _pmc_median_kib(run_dir, counter, name_part):
    """Median per-dispatch value (summed over the counter's instances) of one
    counter for the kernels whose name contains name_part (``name@grid``:
    only dispatches of that grid size, e.g. one decode batch size)."""
    import csv
    import glob
    name_part, _, grid = name_part.partition("@")
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"] and (not grid or r["Grid_Size"] == grid):
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} samples for '{name_part}' under {run_dir}")
    return float(np.median(list(per.values()))), len(per)


KERNEL_SOURCES = {"gemm": ("common.h", "gemm.hip"), "gemv": ("common.h", "gemv.hip")}


def _source_hash(kind):
    """sha256 of a kernel family's sources with comments and blank lines
    removed, so a traffic record stays valid across comment-only edits."""
    import hashlib
    import re
    code = []
    for f in KERNEL_SOURCES[kind]:
        src = open(os.path.join(ROOT, "block_quantized_moe_amd", "csrc", f)).read()
        code += [re.sub(r"//.*", "", l).rstrip() for l in src.splitlines()]
    return hashlib.sha256("\n".join(l for l in code if l).encode()).hexdigest()


def summarize_traffic(name, kernel, alg_bytes, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mb,
                      bench_args=None):
    """Turn four rocprofv3 --pmc runs (the kernel's FETCH_SIZE and WRITE_SIZE;
    the copy probe's FETCH_SIZE and WRITE_SIZE) into HBM bytes per launch,
    written to profiles/<name>_traffic.json."""
    f_kib, nf = _pmc_median_kib(fetch_dir, "FETCH_SIZE", kernel)
    w_kib, nw = _pmc_median_kib(write_dir, "WRITE_SIZE", kernel)
    cf_kib, _ = _pmc_median_kib(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw_kib, _ = _pmc_median_kib(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    true = float(copy_mb << 20)
    k_fetch, k_write = true / (cf_kib * 1024), true / (cw_kib * 1024)
    kind = "gemv" if "gemv" in kernel else "gemm"
    rec = {"name": name, "kernel": kernel,
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
           "copy_probe_mib": copy_mb, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
           "fetch_scale": k_fetch, "write_scale": k_write,
           "bytes_per_launch": f_kib * 1024 * k_fetch + w_kib * 1024 * k_write,
           "algorithmic_bytes_per_launch": alg_bytes, "code_sha256": _source_hash(kind), "code": kind}
    rec["traffic_over_algorithmic"] = rec["bytes_per_launch"] / alg_bytes
    rec["note"] = ("FETCH_SIZE and WRITE_SIZE are KiB per dispatch summed over instances, scaled by "
                   "true bytes / counter bytes of a device copy of known size.")
    if bench_args:
        pmc = "cd /tmp && export TMPDIR=/tmp && cd - && timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python3 bench.py {a}"
        rec["commands"] = [pmc.format(c="FETCH_SIZE", d=fetch_dir, a=bench_args),
                           pmc.format(c="WRITE_SIZE", d=write_dir, a=bench_args),
                           pmc.format(c="FETCH_SIZE", d=copy_fetch_dir, a=f"--copy-probe {copy_mb}"),
                           pmc.format(c="WRITE_SIZE", d=copy_write_dir, a=f"--copy-probe {copy_mb}"),
                           f"python3 bench.py --summarize-traffic {name} '{kernel}' {alg_bytes} {fetch_dir} {write_dir} "
                           f"{copy_fetch_dir} {copy_write_dir} {copy_mb} '{bench_args}'"]
    out = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


PMC_PASSES = (
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU2 SQ_WAIT_INST_LDS SQ_ACTIVE_INST_SCA "
    "SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_MISC SQ_INSTS_MFMA GRBM_GUI_ACTIVE",
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_INSTS_LDS SQ_INST_LEVEL_LDS "
    "SQ_INSTS_VALU SQ_INSTS_SALU GRBM_GUI_ACTIVE",
)


def _csv_rows(run_dir, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(run_dir, "**", "*" + suffix), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_stats(run_dir, name, command, note, out_dir):
    """profiles/<name>.md from a rocprofv3 --kernel-trace run: per kernel the
    launch count and the median / mean / min / max duration (from the kernel
    trace), and the share of GPU time."""
    per = {}
    for r in _csv_rows(run_dir, "kernel_trace.csv"):
        per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    if not per:
        raise SystemExit(f"no kernel trace under {run_dir}")
    total = sum(sum(v) for v in per.values())
    lines = [f"# Kernel durations: {name}", "", "Command (MI355X, one GPU, from the repository root):", "", "```",
             "cd /tmp && export TMPDIR=/tmp && cd -", command, "```", "", note, "",
             "| kernel | calls | median us | mean us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        short = k if len(k) < 90 else k[:87] + "..."
        lines.append(f"| `{short}` | {len(v)} | {v[len(v) // 2]:.1f} | {sum(v) / len(v):.1f} | {v[0]:.1f} | "
                     f"{v[-1]:.1f} | {100 * sum(v) / total:.2f} |")
    lines += ["", "Template arguments: `qmm_int4_kernel<act, epilogue>`, `qmm_{iq2,q2k,mxfp4,q4k,q6k,fp8}_ring_kernel<epilogue>` (fp16), "
              "`qmm_kernel<format, act, epilogue>`, "
              "`gemv_int4_split_kernel<act, epilogue>`: act 0 = fp16, 1 = bf16; epilogue 0 = STORE, 1 = SWIGLU, "
              "2 = WEIGHTED_COMBINE, 3 = ACCUMULATE; format 0 = Q8_0, 1 = Q2_K, 2 = IQ2_XXS, 3 = int4, 4 = MXFP4, "
              "5 = FP8 E4M3 block, 6 = Q4_K, 7 = Q6_K."]
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, f"{name}.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(run_dirs, name, kernel, command, note, out_dir):
    """profiles/<name>_counters.md from rocprofv3 --pmc passes (one directory
    per pass, the PMC_PASSES sets): totals over the kernel's dispatches and
    the ratios that say what bounds it.  Per-SIMD counters are summed over
    the chip's 1024 SIMDs, per-SE ones over its CUs; GRBM_GUI_ACTIVE over
    its 8 XCDs."""
    tot, disp = {}, {}
    for d in run_dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if kernel not in r["Kernel_Name"]:
                continue
            c = r["Counter_Name"]
            tot[(d, c)] = tot.get((d, c), 0.0) + float(r["Counter_Value"])
            disp.setdefault(d, set()).add(r["Dispatch_Id"])
    if not tot:
        raise SystemExit(f"no counters for '{kernel}'")
    v = {}
    for (d, c), x in tot.items():   # per dispatch, averaged over the passes that have the counter
        v.setdefault(c, []).append(x / len(disp[d]))
    v = {c: float(np.mean(x)) for c, x in v.items()}
    n_simd, n_cu, n_xcd = 1024, 256, 8
    cyc = v["GRBM_GUI_ACTIVE"] / n_xcd           # cycles per dispatch
    ratios = {
        "kernel cycles per dispatch (GRBM_GUI_ACTIVE / 8 XCDs)": cyc,
        "MFMA busy, % of cycles per SIMD": 100 * v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / n_simd / cyc,
        "VALU instructions per MFMA (SQ_INSTS_VALU - MFMA) / MFMA": (v.get("SQ_INSTS_VALU", 0) - v.get("SQ_INSTS_MFMA", 0))
        / max(v.get("SQ_INSTS_MFMA", 1), 1),
        "VALU busy, % of cycles per SIMD (4 cycles per wave64 VALU instruction)":
            100 * 4 * (v.get("SQ_INSTS_VALU", 0) - v.get("SQ_INSTS_MFMA", 0)) / n_simd / cyc,
        "MFMA and VALU co-executing, % of MFMA busy cycles": 100 * v.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0)
        / max(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 1), 1),
        "LDS active, % of cycles per CU (SQ_LDS_IDX_ACTIVE)": 100 * v.get("SQ_LDS_IDX_ACTIVE", 0) / n_cu / cyc,
        "LDS bank-conflict cycles, % of LDS active": 100 * v.get("SQ_LDS_BANK_CONFLICT", 0)
        / max(v.get("SQ_LDS_IDX_ACTIVE", 1), 1),
        "wave time waiting on anything (s_waitcnt etc.), %": 100 * v.get("SQ_WAIT_ANY", 0) / v["SQ_WAVE_CYCLES"],
        "wave time ready but not issued, %": 100 * v.get("SQ_WAIT_INST_ANY", 0) / v["SQ_WAVE_CYCLES"],
        "wave time issuing, %": 100 * v.get("SQ_ACTIVE_INST_ANY", 0) / v["SQ_WAVE_CYCLES"],
    }
    lines = [f"# Counters: {name}", "", f"Kernel: `{kernel}` (dispatches whose name contains it).", "",
             "Commands (MI355X, one GPU, from the repository root; one rocprofv3 run per counter set):", "", "```",
             "cd /tmp && export TMPDIR=/tmp && cd -"]
    lines += [command.format(counters=c, i=i + 1) for i, c in enumerate(PMC_PASSES)]
    lines += [f"python3 bench.py --summarize-counters {name} '{kernel}' " + " ".join(run_dirs), "```", "", note, "",
              "| ratio | value |", "|---|---:|"]
    lines += [f"| {k} | {x:.3g} |" for k, x in ratios.items()]
    lines += ["", "Raw counters, per dispatch:", "", "| counter | value |", "|---|---:|"]
    lines += [f"| {c} | {x:.4g} |" for c, x in sorted(v.items())]
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, f"{name}_counters.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_from_profiles(name):
    """HBM bytes per launch measured with rocprofv3 counters, if a record
    exists and was taken on the current kernel code."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    return rec.get("bytes_per_launch") if rec.get("code_sha256") == _source_hash(rec.get("code", "gemm")) else None


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps before the timed ones: on MI355X the kernels keep speeding
    # up over the first tens of milliseconds of load (C2 step 244 us after 5
    # steps, 223 after 50, 216 after 200), so the default runs about 65 ms
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--decode-layers", type=int, default=40)
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the DSv4-shaped and mixed-format prefill lines")
    ap.add_argument("--only", choices=["qwen", "dense", "decode", "dsv4", "dsv4-mxfp4", "dsv4-fp8", "dsv4-kquant",
                                       "mixed", "router"],
                    help="run one workload (for per-workload profiles); prints its own JSON, not the bench line")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--summarize-stats", nargs=4, metavar=("RUN_DIR", "NAME", "COMMAND", "NOTE"),
                    help="write profiles/NAME.md from a rocprofv3 --kernel-trace run")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="NAME KERNEL COMMAND NOTE DIR...: write profiles/NAME_counters.md from --pmc passes")
    ap.add_argument("--summarize-traffic", nargs="+", metavar="ARG",
                    help="NAME KERNEL ALG_BYTES FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR COPY_MIB [BENCH_ARGS]: "
                         "write profiles/NAME_traffic.json")
    args = ap.parse_args()
    if args.summarize_stats:
        d = args.summarize_stats
        summarize_stats(d[0], d[1], d[2], d[3], os.path.join(ROOT, "profiles"))
        return
    if args.summarize_counters:
        d = args.summarize_counters
        summarize_counters(d[4:], d[0], d[1], d[2], d[3], os.path.join(ROOT, "profiles"))
        return
    if args.summarize_traffic:
        d = args.summarize_traffic
        summarize_traffic(d[0], d[1], int(d[2]), d[3], d[4], d[5], d[6], int(d[7]), d[8] if len(d) > 8 else None)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU layout is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_moe_amd as qm
    import synth

    qm.check_device()
    only = args.only
    want = lambda w: only is None or only == w
    others, rooflines, cpu_other, decode = [], [], [], []
    dense = router = imb = None
    decode_inputs = {}
    extra = not args.no_extra and only != "qwen"

    if want("qwen"):
        log("prefill (qwen): building inputs")
        inp = prefill_inputs(2048)
        res = run_prefill(args, torch, qm, inp, args.rotate, args.steps, args.warmup)
        alg = algorithmic(inp, res["wbytes_gu"], res["wbytes_dn"])
        t_step = res["wall"]
        value = alg["flops"] / t_step / 1e12
        t_gu = float(np.median(res["kern"]["gate_up"]))
        roofline = roof("qmm_int4_kernel<bf16, SWIGLU> (int4 gate/up)", "qwen3.6-a3b-int4-prefill",
                        alg["flops_gu"], alg["bytes_gu"], t_gu, traffic_from_profiles("gate_up_qwen"))
        roofline["bound"], roofline["unit"] = "hbm", "GB/s"   # HBM-bound by its own work (41 vs 27 us at peak)
        roofline["achieved"], roofline["peak"] = alg["bytes_gu"] / t_gu / 1e9, PEAK_HBM / 1e9
        roofline["frac"] = alg["bytes_gu"] / t_gu / PEAK_HBM
        qline, qrl = prefill_line("qwen", inp, res, args.rotate)
        rooflines += qrl
        log(f"prefill: step {t_step*1e6:.1f} us, {value:.1f} TFLOP/s; {json.dumps(qline['kernels_us'])}")
        cpu = None
        if not args.no_cpu and only is None:
            log("cpu baseline: oracle sample")
            cpu = cpu_baseline(inp, args.cpu_tokens)
        del inp
    if (extra or only == "dense") and want("dense"):
        log("dense q8_0 cell")
        dense = run_dense_cell(torch, qm)
        log(json.dumps(dense))
        if not args.no_cpu and only is None:
            cpu_other += cpu_dense_cell()
    if extra:
        for name, make, R in (("dsv4", lambda: synth.dsv4_flash_prefill(2048), 2),
                              ("dsv4-mxfp4", lambda: synth.dsv4_flash_mxfp4_prefill(2048), 2),
                              ("dsv4-fp8", lambda: synth.dsv4_flash_fp8_prefill(2048), 2),
                              ("dsv4-kquant", lambda: synth.dsv4_flash_kquant_prefill(2048), 2),
                              ("mixed", lambda: synth.mixed_ffn(8192), 2)):
            if not want(name):
                continue
            log(f"prefill ({name}): building inputs")
            inp_o = make()
            # a fifth of the warm-up: 60 steps by default (66 ms of the
            # DSv4-shaped step, 265 ms of the mixed block)
            res = run_prefill(args, torch, qm, inp_o, R, max(3, args.steps // 4), max(2, args.warmup // 5))
            line_o, rl = prefill_line(name, inp_o, res, R)
            if name == "mixed":
                imb = imbalance(inp_o)
                line_o["imbalance"] = imb
            others.append(line_o)
            rooflines += rl
            log(json.dumps(line_o))
            if not args.no_cpu and only is None and name in ("dsv4", "mixed"):
                log(f"cpu oracle sample ({name})")
                cpu_other.append(cpu_sample_experts(inp_o, np.arange(8)))
            if name in ("dsv4-mxfp4", "dsv4-fp8", "dsv4-kquant"):
                decode_inputs[name] = inp_o  # its weights also serve the decode lines of the format
            else:
                del inp_o
    if (extra or only == "router") and want("router"):
        log("router top-k")
        router = run_router(torch, qm)
        log(json.dumps(router))
    decode_floor = None
    if not args.no_decode and want("decode"):
        decode_floor = run_launch_floor(torch, args.decode_layers)
        log(f"decode launch floor: {json.dumps(decode_floor)}")
        for B in (1, 4, 8):
            log(f"decode: B={B}")
            d, rl = run_decode(args, torch, qm, B, args.decode_layers)
            decode.append(d)
            rooflines += rl
            log(json.dumps(d))
    if not args.no_decode and extra and only is None:
        import dataclasses
        for name, src in decode_inputs.items():
            fmt = name.split("-")[1]
            for B in (1, 4):
                log(f"decode ({name}): B={B}")
                dec = dataclasses.replace(src, name=f"dsv4-flash-{fmt}-decode-b{B}", T=B, x=src.x[:B],
                                          ids=src.ids[:B], w=src.w[:B])
                d, rl = run_decode(args, torch, qm, B, max(2, args.decode_layers // 5), dec)
                decode.append(d)
                rooflines += rl
                log(json.dumps(d))

    if only is not None and only != "qwen":
        print(json.dumps({"only": only, "other_prefill_workloads": others, "decode": decode,
                          "decode_launch_floor": decode_floor, "dense_q8_0": dense,
                          "router": router, "rooflines": rooflines}), flush=True)
        return
    line = {
        "metric": "MoE qGEMM prefill TFLOP/s (% MFMA peak) + decode GEMV GB/s (% HBM peak)",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3.6-a3b-shaped int4 MoE prefill", "tokens": 2048, "hidden": 2048,
                   "experts": 256, "top_k": 8, "intermediate": 512,
                   "weights": "int4 affine, group 64, fp16 scale+bias", "activations": "bf16",
                   "weight_copies_rotated": args.rotate},
        "mfma_frac": value * 1e12 / PEAK_MFMA_BF16,
        "tokens_per_s": 2048 / t_step,
        "step_us": qline["step_us"],
        "kernels_us": qline["kernels_us"],
        "algorithmic": {"flops": alg["flops"], "bytes": alg["bytes"]},
        "roofline": roofline,
        "rooflines": rooflines,
        "dense_q8_0": dense,
        "decode": decode,
        "decode_launch_floor": decode_floor,
        "other_prefill_workloads": others,
        "imbalance": imb,
        "router": router,
        "cpu_baseline": cpu,
        "cpu_oracle": cpu_other,
        "host": host_info(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
