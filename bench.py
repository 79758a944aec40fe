"""Benchmark of the block-quantized MoE expert matmul on one MI355X.

Step (the timed unit): one pass of the whole prefill MoE hot path over the
Qwen3.6-A3B-shaped int4 workload -- routing plan, gathered gate/up GEMM with
the SwiGLU epilogue, gathered down GEMM into per-pair rows, and the
deterministic top-k weighted combine -- for T = 2048 tokens, hidden 2048, 256 experts, top-8,
expert intermediate 512, bf16 activations, int4 affine weights (group 64).
The weights rotate over R copies so no step finds them in the 256 MB
Infinity Cache.  `value` is algorithmic TFLOP/s of that step (routed pairs
only; padding is not counted).

The decode GEMV leg (same model, B in {1, 4, 8}, 40 layers, each with its own
copy of the weights) is timed as a captured HIP graph replay and eagerly; its
GB/s are weight + activation bytes per layer over graph time per layer.  The
DSv4-flash-shaped prefill (IQ2_XXS gate/up, Q2_K down, fp16, T = 2048) and the
mixed-format FFN block (T = 8192, plus a Q8_0 shared expert; its four Q8_0
projections timed apart) are reported under other_prefill_workloads.  The
CPU oracle baseline is reported in the same JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-extra]

Counter calibration and the traffic record (see profiles/):
    python bench.py --copy-probe MIB
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR MIB
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def act_tensor(torch, bits):
    """uint16 bf16 bit patterns -> a bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def upload(qm, W):
    if W.fmt == "int4":
        return qm.upload("int4", W.E, W.N, W.K, qs=W.qs, scale=W.scale, bias=W.bias, group=W.group)
    if W.fmt == "fp8":
        return qm.upload("fp8", W.E, W.N, W.K, qs=W.qs, scale=W.scale)
    return qm.upload(W.fmt, W.E, W.N, W.K, blocks=W.blocks, grid=W.grid)


def prefill_inputs(T):
    import synth
    return synth.qwen_a3b_prefill(T)


def algorithmic(inp):
    """Flops and bytes of one prefill step (routed pairs only)."""
    P = int(inp.ids.size)
    H, I = inp.H, inp.I
    flops_gu = 2.0 * P * (2 * I) * H
    flops_dn = 2.0 * P * H * I
    wbytes_gu = inp.w_gate_up.nbytes
    wbytes_dn = inp.w_down.nbytes
    act = 2  # bf16
    bytes_gu = wbytes_gu + inp.T * H * act + P * I * act    # weights + x read + h write
    bytes_dn = wbytes_dn + P * I * act + inp.T * H * act    # weights + h read + out write
    return dict(P=P, flops=flops_gu + flops_dn, flops_gu=flops_gu, flops_dn=flops_dn,
                bytes=bytes_gu + bytes_dn, bytes_gu=bytes_gu, bytes_dn=bytes_dn)


def run_prefill(args, torch, qm):
    inp = prefill_inputs(2048)
    alg = algorithmic(inp)
    dev = "cuda"
    x = act_tensor(torch, inp.x)
    ids = torch.from_numpy(inp.ids).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    gu0, dn0 = upload(qm, inp.w_gate_up), upload(qm, inp.w_down)
    R = args.rotate
    gus = [gu0] + [gu0.clone() for _ in range(R - 1)]
    dns = [dn0] + [dn0.clone() for _ in range(R - 1)]
    T, k, E, I = inp.T, inp.k, inp.E, inp.I
    bm = 80
    plan = torch.empty(qm.plan_bytes(T, k, E, bm) // 4, dtype=torch.int32, device=dev)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T * k, inp.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, inp.H), dtype=torch.bfloat16, device=dev)

    ev = {name: [] for name in ("plan", "gate_up", "down", "combine")}

    def step(i, timed):
        gu, dn = gus[i % R], dns[i % R]
        marks = []
        if timed:
            marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record()
        qm.moe_plan(ids, E, bm, plan=plan)
        if timed:
            marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record()
        qm.moe_gather_qmm(gu, plan, T, k, x, bm=bm, epilogue=qm.EPI_SWIGLU, out=h)
        if timed:
            marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record()
        qm.moe_gather_qmm(dn, plan, T, k, h, bm=bm, a_mode=qm.A_SORTED_ROWS, epilogue=qm.EPI_STORE, out=y)
        if timed:
            marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record()
        qm.moe_combine(y, plan, T, k, E, w, out=out)
        if timed:
            marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record()
        return marks

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # K steps launched from the host, wall clock.  (A HIP graph of the step
    # measured slower here: 320 against 294 us, the graph launch costing more
    # than the four host launches it replaces.)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, False)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    # per-kernel durations (events on the launch stream) over another K steps
    all_marks = [step(i, True) for i in range(args.steps)]
    torch.cuda.synchronize()
    for m in all_marks:
        for j, name in enumerate(("plan", "gate_up", "down", "combine")):
            ev[name].append(m[j].elapsed_time(m[j + 1]) * 1e-3)
    kern = {n: float(np.median(v)) for n, v in ev.items()}
    return inp, alg, wall, kern


def run_prefill_other(args, torch, qm, inp, R, steps):
    """Another prefill workload, the same step as run_prefill (plan, gate/up
    with SwiGLU, down with the weighted scatter-add, cast), plus the shared
    expert (added into the same accumulator) when the workload has one; its
    dense projections are timed separately."""
    dev = "cuda"
    codes = {"f16": qm.F16, "bf16": qm.BF16}
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    x = act_tensor(torch, inp.x) if inp.act == "bf16" else \
        torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.float16)
    ids = torch.from_numpy(inp.ids).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    gu0, dn0 = upload(qm, inp.w_gate_up), upload(qm, inp.w_down)
    gus = [gu0] + [gu0.clone() for _ in range(R - 1)]
    dns = [dn0] + [dn0.clone() for _ in range(R - 1)]
    T, k, E, H, I = inp.T, inp.k, inp.E, inp.H, inp.I
    bm = 80
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

    for i in range(2):
        step(i, False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i, False)
    e1.record()
    torch.cuda.synchronize()
    t_step = e0.elapsed_time(e1) * 1e-3 / steps
    all_marks = [step(i, True) for i in range(steps)]
    torch.cuda.synchronize()
    kern = {n: float(np.median([m[j].elapsed_time(m[j + 1]) for m in all_marks])) * 1e-3
            for j, n in enumerate(names)}
    P = int(inp.ids.size)
    flops = 2.0 * P * 3 * I * H
    if shared:
        SI = inp.shared_down.K
        flops += 2.0 * T * 3 * SI * H
    res = dict(workload=inp.name, tokens=T, hidden=H, intermediate=I, experts=E, top_k=k,
               weights=f"gate/up {inp.w_gate_up.fmt}, down {inp.w_down.fmt}" + (", shared expert q8_0" if shared else ""),
               activations=inp.act, weight_copies_rotated=R, ms_per_step=t_step * 1e3,
               tflops=flops / t_step / 1e12, mfma_frac=flops / t_step / PEAK_MFMA_BF16,
               kernels_us={n: v * 1e6 for n, v in kern.items()})
    if inp.projections:
        ps = [upload(qm, Wp) for Wp in inp.projections]
        y = torch.empty((T, H), dtype=tdt[inp.act], device=dev)
        for Wp in ps:
            qm.qmm_dense(Wp, x, qm.EPI_STORE, codes[inp.act], out=y)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            for Wp in ps:
                qm.qmm_dense(Wp, x, qm.EPI_STORE, codes[inp.act], out=y)
        e1.record()
        torch.cuda.synchronize()
        tp = e0.elapsed_time(e1) * 1e-3 / steps
        pf = 2.0 * T * H * H * len(ps)
        res["projections"] = dict(count=len(ps), ms=tp * 1e3, tflops=pf / tp / 1e12, mfma_frac=pf / tp / PEAK_MFMA_BF16)
        del ps
    del gus, dns
    torch.cuda.empty_cache()
    return res


def run_router(args, torch, qm):
    """Device router top-k ahead of the plan: per-launch time from a replayed
    graph of launches (events on the replay stream), and the HBM rate of its
    algorithmic bytes (logits and bias read, ids and weights written)."""
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
        # launches captured in a graph and replayed, so host launch cost does
        # not hide the kernel's own time
        n = 100
        for _ in range(3):
            qm.router_topk(L, k, scoring, bias, scale, ids, w)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(n):
                    qm.router_topk(L, k, scoring, bias, scale, ids, w)
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / (5 * n)
        nbytes = L.numel() * L.element_size() + T * k * 8 + (E * 4 if bias is not None else 0)
        rows.append({"workload": name, "tokens": T, "experts": E, "top_k": k, "logits": dt,
                     "us_per_launch": t * 1e6, "GBps": nbytes / t / 1e9, "hbm_frac": nbytes / t / PEAK_HBM,
                     "bytes_per_launch": nbytes})
    return rows


def run_decode(args, torch, qm, B, layers, inp=None):
    import synth
    inp = synth.qwen_a3b_decode(B) if inp is None else inp
    dev = "cuda"
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[inp.act]
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).to(dev).view(tdt)
    ids = torch.from_numpy(inp.ids).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    gu0, dn0 = upload(qm, inp.w_gate_up), upload(qm, inp.w_down)
    gus = [gu0] + [gu0.clone() for _ in range(layers - 1)]
    dns = [dn0] + [dn0.clone() for _ in range(layers - 1)]
    h = torch.empty((B, inp.k, inp.I), dtype=tdt, device=dev)
    out = torch.empty((B, inp.H), dtype=tdt, device=dev)
    uniq = np.unique(inp.ids)
    per_expert = (inp.w_gate_up.nbytes + inp.w_down.nbytes) // inp.E
    nbytes = len(uniq) * per_expert + B * inp.H * 2 * 2 + B * inp.k * inp.I * 2 * 2
    def layer(l):
        qm.moe_gemv(gus[l], x, ids, epilogue=qm.EPI_SWIGLU, out=h)
        qm.moe_gemv(dns[l], h, ids, w, epilogue=qm.EPI_WEIGHTED_COMBINE, out=out)

    for _ in range(2):
        for l in range(layers):
            layer(l)
    torch.cuda.synchronize()
    reps = max(1, args.decode_reps)
    # eager: every layer launched from the host, events around the whole run
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for l in range(layers):
            layer(l)
    e1.record()
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) * 1e-3 / (reps * layers)
    # graph: the same layers captured once into a HIP graph and replayed
    # (no launch gaps from the host; the kernels allocate nothing and issue
    # no memset, so they replay as captured)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for l in range(layers):
                layer(l)
    torch.cuda.current_stream().wait_stream(stream)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t_graph = e0.elapsed_time(e1) * 1e-3 / (reps * layers)
    # per-launch durations with events around each launch (upper bounds: an
    # event pair adds its own gap to a launch this short)
    marks = []
    for l in range(layers):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        qm.moe_gemv(gus[l], x, ids, epilogue=qm.EPI_SWIGLU, out=h)
        e[1].record()
        qm.moe_gemv(dns[l], h, ids, w, epilogue=qm.EPI_WEIGHTED_COMBINE, out=out)
        e[2].record()
        marks.append(e)
    torch.cuda.synchronize()
    t_gu = float(np.median([m[0].elapsed_time(m[1]) for m in marks])) * 1e-3
    t_dn = float(np.median([m[1].elapsed_time(m[2]) for m in marks])) * 1e-3
    del graph, gus, dns
    torch.cuda.empty_cache()
    return dict(workload=inp.name, B=B, layers=layers, unique_experts=int(len(uniq)), bytes_per_layer=int(nbytes),
                s_per_layer_graph=t_graph, s_per_layer_eager=t_eager,
                gate_up_s_event=t_gu, down_s_event=t_dn,
                GBps=nbytes / t_graph / 1e9, hbm_frac=nbytes / t_graph / PEAK_HBM,
                GBps_eager=nbytes / t_eager / 1e9, tokens_per_s_per_layer=B / t_graph)


def cpu_baseline(n_tokens):
    """The oracle, as it stands, on a bounded sample of the prefill workload:
    the full MoE FFN (gate/up + SwiGLU, down, weighted combine) for the first
    n_tokens tokens, in fp64."""
    import oracle
    inp = prefill_inputs(2048)
    ids = inp.ids[:n_tokens]
    w = inp.w[:n_tokens]
    x64 = oracle.act_to_f64(inp.x[:n_tokens], "bf16")
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.moe_ffn(x64, ids, w, inp.w_gate_up, inp.w_down, h_dtype="bf16")
    dt = time.perf_counter() - t0
    P = ids.size
    flops = 2.0 * P * (3 * inp.I * inp.H)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"first {n_tokens} of 2048 tokens ({P} routed pairs) of the prefill workload, "
                       f"fp64 oracle, {dt:.1f} s", tokens_per_s=n_tokens / dt, seconds=dt)


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
    counter for the kernels whose name contains name_part."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} samples for '{name_part}' under {run_dir}")
    return float(np.median(list(per.values()))), len(per)


def _gemm_source_hash():
    """sha256 of the GEMM kernel sources (gemm.hip and the shared device
    helpers) with comments and blank lines removed, so the traffic record
    stays valid across comment-only edits."""
    import hashlib
    import re
    code = []
    for f in ("common.h", "gemm.hip"):
        src = open(os.path.join(ROOT, "block_quantized_moe_amd", "csrc", f)).read()
        code += [re.sub(r"//.*", "", l).rstrip() for l in src.splitlines()]
    return hashlib.sha256("\n".join(l for l in code if l).encode()).hexdigest()


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mb, out):
    """Turn four rocprofv3 --pmc runs (gate/up FETCH_SIZE, WRITE_SIZE; copy
    probe FETCH_SIZE, WRITE_SIZE) into HBM bytes per gate/up launch."""
    kern = "qmm_int4_kernel<1, 1>"
    f_kib, nf = _pmc_median_kib(fetch_dir, "FETCH_SIZE", kern)
    w_kib, nw = _pmc_median_kib(write_dir, "WRITE_SIZE", kern)
    cf_kib, _ = _pmc_median_kib(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw_kib, _ = _pmc_median_kib(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    true = float(copy_mb << 20)
    k_fetch, k_write = true / (cf_kib * 1024), true / (cw_kib * 1024)
    inp = prefill_inputs(2048)
    alg = algorithmic(inp)
    rec = {
        "kernel": "qmm_int4_kernel<bf16, SWIGLU> (int4 gate/up), qwen3.6-a3b-shaped prefill",
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
        "copy_probe_mib": copy_mb, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
        "fetch_scale": k_fetch, "write_scale": k_write,
        "bytes_per_launch": f_kib * 1024 * k_fetch + w_kib * 1024 * k_write,
        "algorithmic_bytes_per_launch": alg["bytes_gu"],
        "gemm_code_sha256": _gemm_source_hash(),
    }
    rec["traffic_over_algorithmic"] = rec["bytes_per_launch"] / alg["bytes_gu"]
    pm = "rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python3 bench.py {a}"
    prefill = "--steps 3 --warmup 1 --no-decode --no-cpu --no-extra"
    rec["commands"] = [pm.format(c="FETCH_SIZE", d=fetch_dir, a=prefill),
                       pm.format(c="WRITE_SIZE", d=write_dir, a=prefill),
                       pm.format(c="FETCH_SIZE", d=copy_fetch_dir, a=f"--copy-probe {copy_mb}"),
                       pm.format(c="WRITE_SIZE", d=copy_write_dir, a=f"--copy-probe {copy_mb}"),
                       f"python3 bench.py --summarize-traffic {fetch_dir} {write_dir} {copy_fetch_dir} "
                       f"{copy_write_dir} {copy_mb}"]
    rec["note"] = ("FETCH_SIZE and WRITE_SIZE are KiB per dispatch summed over instances, scaled by "
                   "true bytes / counter bytes of a device copy of known size.")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def traffic_from_profiles():
    """HBM bytes per gate/up launch measured with rocprofv3 counters, if the
    committed measurement was taken on the current kernel code."""
    p = os.path.join(ROOT, "profiles", "gate_up_qwen_prefill_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    return rec.get("bytes_per_launch") if rec.get("gemm_code_sha256") == _gemm_source_hash() else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--decode-layers", type=int, default=40)
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the DSv4-shaped and mixed-format prefill lines")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--summarize-traffic", nargs=5,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "COPY_MIB"),
                    help="write profiles/gate_up_qwen_prefill_traffic.json from rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.summarize_traffic:
        d = args.summarize_traffic
        summarize_traffic(d[0], d[1], d[2], d[3], int(d[4]),
                          os.path.join(ROOT, "profiles", "gate_up_qwen_prefill_traffic.json"))
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

    qm.check_device()
    log("prefill: building inputs")
    inp, alg, wall, kern = run_prefill(args, torch, qm)
    t_step = wall
    value = alg["flops"] / t_step / 1e12
    t_gu = kern["gate_up"]
    roofline = {
        "kernel": "qmm_int4_kernel<bf16, SWIGLU> (int4 gate/up)",
        "bound": "hbm",
        "achieved": alg["bytes_gu"] / t_gu / 1e9,
        "peak": PEAK_HBM / 1e9,
        "unit": "GB/s",
        "frac": alg["bytes_gu"] / t_gu / PEAK_HBM,
        "traffic": traffic_from_profiles(),
        "algorithmic_bytes_per_launch": alg["bytes_gu"],
        "launch_s": t_gu,
        "mfma_tflops": alg["flops_gu"] / t_gu / 1e12,
        "mfma_frac": alg["flops_gu"] / t_gu / PEAK_MFMA_BF16,
    }
    log(f"prefill: step {t_step*1e6:.1f} us, {value:.1f} TFLOP/s; kernels {json.dumps(kern)}")
    others = []
    decode_inputs = {}
    if not args.no_extra:
        import synth
        for name, make, R in (("dsv4", lambda: synth.dsv4_flash_prefill(2048), 2),
                              ("dsv4 mxfp4", lambda: synth.dsv4_flash_mxfp4_prefill(2048), 2),
                              ("dsv4 fp8", lambda: synth.dsv4_flash_fp8_prefill(2048), 2),
                              ("mixed", lambda: synth.mixed_ffn(8192), 2)):
            log(f"prefill ({name}): building inputs")
            inp_o = make()
            others.append(run_prefill_other(args, torch, qm, inp_o, R, max(3, args.steps // 4)))
            log(json.dumps(others[-1]))
            if name in ("dsv4 mxfp4", "dsv4 fp8"):
                decode_inputs[name] = inp_o  # its weights also serve the decode lines of the format
            del inp_o
    log("router top-k")
    router = run_router(args, torch, qm)
    log(json.dumps(router))
    decode = []
    if not args.no_decode:
        for B in (1, 4, 8):
            log(f"decode: B={B}")
            decode.append(run_decode(args, torch, qm, B, args.decode_layers))
            log(json.dumps(decode[-1]))
        if not args.no_extra:
            import dataclasses
            for name, src in decode_inputs.items():
                fmt = name.split()[1]
                for B in (1, 4):
                    log(f"decode ({name}): B={B}")
                    dec = dataclasses.replace(src, name=f"dsv4-flash-{fmt}-decode-b{B}", T=B, x=src.x[:B],
                                              ids=src.ids[:B], w=src.w[:B])
                    decode.append(run_decode(args, torch, qm, B, max(2, args.decode_layers // 5), dec))
                    log(json.dumps(decode[-1]))
    cpu = None
    if not args.no_cpu:
        log("cpu baseline: oracle sample")
        cpu = cpu_baseline(args.cpu_tokens)
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
        "config": {"workload": "qwen3.6-a3b-shaped int4 MoE prefill", "tokens": inp.T, "hidden": inp.H,
                   "experts": inp.E, "top_k": inp.k, "intermediate": inp.I,
                   "weights": "int4 affine, group 64, fp16 scale+bias", "activations": "bf16",
                   "weight_copies_rotated": args.rotate},
        "mfma_frac": value * 1e12 / PEAK_MFMA_BF16,
        "tokens_per_s": inp.T / t_step,
        "kernels_s": kern,
        "algorithmic": {"flops": alg["flops"], "bytes": alg["bytes"]},
        "roofline": roofline,
        "decode": [{"workload": d["workload"], "B": d["B"], "layers": d["layers"], "GBps": d["GBps"], "hbm_frac": d["hbm_frac"], "GBps_eager": d["GBps_eager"],
                    "us_per_layer_graph": d["s_per_layer_graph"] * 1e6,
                    "us_per_layer_eager": d["s_per_layer_eager"] * 1e6,
                    "us_gate_up_event": d["gate_up_s_event"] * 1e6, "us_down_event": d["down_s_event"] * 1e6,
                    "unique_experts": d["unique_experts"], "bytes_per_layer": d["bytes_per_layer"]}
                   for d in decode],
        "other_prefill_workloads": others,
        "router": router,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
