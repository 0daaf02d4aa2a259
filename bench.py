#!/usr/bin/env python3
"""Throughput of the CacheBlend KV-fusion step on one MI355X.

A step is one pass of the whole hot path -- for every layer of the workload:
re-rotate the cached keys, score and select the candidates, fuse the
recomputed rows, and run the selected rows' causal GQA attention -- over one
batch of seeded synthetic input already resident in HBM.  Every step gets its
own copy of the inputs (the blend works in place), so nothing is restored
inside the timed region and no step is served from the 256 MB Infinity Cache.

Metric: blended context tokens per second per layer = tokens * layers / time.

Printed: one JSON line with the metric, a roofline entry for the dominant
kernel (algorithmic work per launch / its average launch time, measured with
HIP events on the launch stream, against the published peak and against the
peak measured by the in-tree probe `cb_peaks`), the whole-step roofline
fraction (streaming bytes at 8 TB/s plus attention flops at the MFMA peak,
over the step time), per-kernel figures (each stage's rate and its fraction of
the published and the measured peak; the top-k also timed on its own) and the
CPU oracle timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # fp32 vector
DEFAULT_STEPS = {"tiny": (200, 20), "mistral7b-layer": (200, 20), "7b-32layer-6k": (20, 3),
                 "7b-32layer-32k": (4, 1), "70b-80layer-8req": (2, 1)}
STAGES = ("rerotate", "deviation_topk", "fuse_scatter", "partial_attn")
# the order that scores and selects first, then rotates-or-replaces in one pass
STAGES_AFTER = ("deviation_topk", "rerotate_fuse", "partial_attn")
PROFILES = os.path.join(ROOT, "profiles")


def source_fingerprint():
    """sha256 over the library's sources (its compiled files, their headers and
    the public header): a recorded byte count is only valid for the kernels it
    was measured on."""
    import hashlib
    from selective_recompute_amd import build as BLD
    csrc = os.path.join(ROOT, "selective_recompute_amd", "csrc")
    files = [os.path.join(csrc, n) for n in BLD.SOURCES]
    files += sorted(os.path.join(csrc, n) for n in os.listdir(csrc) if n.endswith(".hpp"))
    files += sorted(os.path.join(ROOT, "include", n) for n in os.listdir(os.path.join(ROOT, "include")))
    h = hashlib.sha256()
    for path in files:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def attainable_peaks():
    """Run the in-tree probe (built next to the library) in a child process
    before this process touches the GPU; None if it is not built."""
    import subprocess
    from selective_recompute_amd import build as BLD
    if not os.path.exists(BLD.PEAKS):
        return None
    res = subprocess.run([BLD.PEAKS], capture_output=True, text=True, timeout=120)
    if res.returncode != 0:
        log(f"[bench] peak probe failed: {res.stderr.strip()}")
        return None
    return json.loads(res.stdout.strip().splitlines()[-1])


def recorded_traffic(stage, workload):
    """HBM bytes per launch of `stage` from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary under profiles/, or None when there is none for this workload or
    the sources changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{stage}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != source_fingerprint():
        return None
    return float(rec["hbm_bytes_per_launch"])


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="mistral7b-layer", choices=list(DEFAULT_STEPS))
    ap.add_argument("--schedule", default="pool", choices=["pool", "chain"])
    ap.add_argument("--dev-source", default="v", choices=["v", "k", "kv"],
                    help="what the token deviation measures: V (default), K at the new "
                         "position, or the K and V rows as one vector")
    ap.add_argument("--order", default="auto", choices=["auto", "rotate-first", "select-first"],
                    help="step order of cb_blend_layer: select-first scores V and selects "
                         "first, then one launch writes the rows of S and re-rotates only the "
                         "others; auto lets the library choose")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--attainable", type=int, default=1,
                    help="1: measure attainable MFMA / HBM peaks first and report "
                         "fractions against them too")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: capture the timed steps' launches in one HIP graph and "
                         "time its replay (same kernels, no host launch cost)")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the blend step: dense causal attention of every "
                         "row (layer-1 full prefill) at the workload's shape")
    ap.add_argument("--print-source-sha", action="store_true",
                    help="print the sources' fingerprint and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB device to device once (a "
                         "plain copy of known size that calibrates byte counters)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_work(wl, runner, selected_per_layer, dev_tensors=1):
    """Per-layer algorithmic bytes / flops of each stage (what the method must
    move or compute), from the selection actually made.  dev_tensors: 2 when
    the deviation reads both K and V."""
    import numpy as np
    elem = 2 if wl.dtype == "bf16" else 4
    row = wl.n_kv_heads * wl.head_dim * elem
    t_count = wl.n_tokens
    delta = wl.delta()
    nz = int(np.count_nonzero(delta))
    tok_off = wl.tok_off
    work = []
    for layer in range(wl.n_layers):
        m = runner.batches[layer].n_cand
        sel = selected_per_layer[layer]
        k = len(sel)
        req = np.searchsorted(tok_off, sel, side="right") - 1
        pos = sel - tok_off[req]
        flops = 4.0 * wl.head_dim * wl.n_q_heads * float(np.sum(pos + 1))
        work.append({
            "rerotate": 2.0 * row * nz + 4.0 * t_count,
            "deviation_topk": 2.0 * dev_tensors * row * m + 8.0 * m,
            "fuse_scatter": 4.0 * row * k + 8.0 * k,
            # rotate-or-replace: kept rows with delta != 0 turned, rows of S written
            "rerotate_fuse": 2.0 * row * (nz - int(np.count_nonzero(delta[sel]))) + 4.0 * t_count
                             + 4.0 * row * k + 8.0 * k,
            "partial_attn": flops,
        })
    return work


def cpu_baseline(wl, seconds, dev_source="v"):
    """The CPU oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import cacheblend_oracle as O
    from selective_recompute_amd import workloads as W

    sets = W.PlantedSets(wl)
    x = W.layer_inputs(wl, sets, 0, device="cpu")
    f64 = lambda t: t.to(torch.float64).numpy()
    args = dict(k_old=f64(x["k_old"]), v_old=f64(x["v_old"]), delta=wl.delta(),
                k_new_c=f64(x["k_new_c"]), v_new_c=f64(x["v_new_c"]), q_c=f64(x["q_c"]),
                cand_idx=x["cand_idx"].numpy(), tok_off=wl.tok_off, cand_off=x["h_cand_off"],
                sel_counts=[(wl.r1_pct * n + 99) // 100 for n in wl.request_lengths],
                n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, theta=wl.rope_theta,
                scale=1.0 / math.sqrt(wl.head_dim))
    # Large layers: time re-rotation/deviation/top-k/fuse in full and the
    # attention on an evenly spaced 1/frac of the selected rows, then scale.
    frac = 1 if wl.n_tokens <= 8192 else 16
    reps, t_total = 0, 0.0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        res = O.blend_layer(**args, attend=(frac == 1), dev_source=dev_source)
        t1 = time.perf_counter()
        t_layer = t1 - t0
        if frac > 1:
            rows = np.arange(0, len(res["sel_global"]), frac)
            O.attention_rows(args["q_c"], res["sel_local"][rows], res["sel_global"][rows],
                             res["row_start"][rows], res["k_fused"], res["v_fused"],
                             wl.n_q_heads, wl.n_kv_heads, args["scale"])
            t_layer += (time.perf_counter() - t1) * frac
        t_total += t_layer
        reps += 1
        if time.perf_counter() - t_start >= seconds:
            break
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    sample = (f"layer 1 of {wl.name} ({wl.n_tokens} tokens, {sum(args['sel_counts'])} selected), "
              f"{reps} repetition(s) of the full oracle pipeline in float64 numpy")
    if frac > 1:
        sample += f"; attention timed on every {frac}th selected row and scaled by {frac}"
    sample += "; element-wise numpy runs on one thread, matrix-vector products on the BLAS pool"
    return {"value": wl.n_tokens * reps / t_total, "unit": "tokens/s/layer", "cores": cores,
            "kind": "oracle", "sample": sample}


def prefill_main(a, peaks):
    """Layer-1 full prefill: every row of every request attends causally over
    its request, through the same cb_partial_attn entry point (all rows
    selected).  Prints one JSON line in TFLOP/s."""
    import numpy as np
    import torch

    from selective_recompute_amd import binding as B
    from selective_recompute_amd import pipeline as PL
    from selective_recompute_amd import workloads as W

    wl = W.make_workload(a.workload)
    if wl.dtype != "bf16":
        raise SystemExit("--prefill measures the bf16 MFMA path")
    steps = a.steps if a.steps is not None else 5
    warmup = a.warmup if a.warmup is not None else 1
    lens = wl.request_lengths
    t_count = int(sum(lens))
    tok_off = PL.offsets(lens)
    gen = torch.Generator(device="cuda").manual_seed(0xCB10 + t_count)
    mk = lambda h: torch.randn(t_count, h, wl.head_dim, generator=gen, device="cuda").to(torch.bfloat16)
    q, k, v = mk(wl.n_q_heads), mk(wl.n_kv_heads), mk(wl.n_kv_heads)
    idx = torch.arange(t_count, dtype=torch.int32, device="cuda")
    rb = B.RaggedBatch(tok_off, tok_off, tok_off, "cuda")
    g = B.geom(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, torch.bfloat16)
    ws = B.workspace_tensor(B.attn_workspace_bytes(g, rb), "cuda")
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(wl.head_dim)
    stream = torch.cuda.Stream()
    run = lambda: B.partial_attn(g, rb, out, q, idx, idx, k, v, scale, workspace=ws, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 4.0 * wl.head_dim * wl.n_q_heads * sum(n * (n + 1) / 2 for n in lens)
    tf = flops / (ms * 1e-3) / 1e12
    roof = {"kernel": "partial_attn (all rows)", "bound": "mfma", "achieved": round(tf, 3),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 5),
            "traffic": None}
    if peaks:
        roof["attainable_peak"] = peaks["mfma_bf16_32x32x16_tflops"]
        roof["frac_attainable"] = round(tf / peaks["mfma_bf16_32x32x16_tflops"], 5)
    print(json.dumps({
        "metric": "dense causal attention TFLOP/s (layer-1 full prefill)", "value": round(tf, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} shape, every row selected", "tokens": t_count,
                   "requests": len(lens), "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "gflop_per_launch": round(flops / 1e9, 3)},
        "roofline": roof, "attainable": peaks}), flush=True)


def main():
    a = parse_args()
    if a.print_source_sha:
        print(source_fingerprint())
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported (the library "
              "has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    peaks = attainable_peaks() if a.attainable else None
    if a.prefill:
        return prefill_main(a, peaks)
    import numpy as np
    import torch

    from selective_recompute_amd import binding as B
    from selective_recompute_amd import pipeline as PL
    from selective_recompute_amd import workloads as W

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    B.lib()
    wl = W.make_workload(a.workload)
    steps, warmup = DEFAULT_STEPS[wl.name]
    steps = a.steps if a.steps is not None else steps
    warmup = a.warmup if a.warmup is not None else warmup
    L = wl.n_layers
    sets = W.PlantedSets(wl, a.schedule)
    runner = PL.BlendRunner(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.torch_dtype,
                            wl.request_lengths, wl.r1_pct, wl.r2_pct, L, wl.rope_theta,
                            schedule=a.schedule, dev_source=a.dev_source, device="cuda",
                            order=a.order)
    if a.order == "select-first" and a.dev_source != "v":
        raise SystemExit("--order select-first scores V only (a key deviation reads the "
                         "re-rotated keys)")
    stream = torch.cuda.Stream()
    h = stream.cuda_stream

    def make_copies(n, first_draw):
        cps = []
        for c in range(n):
            cps.append([W.layer_inputs(wl, sets, l, device="cuda", draw=first_draw + c)
                        for l in range(L)])
        torch.cuda.synchronize()
        return cps

    # ---- timed pass: whole layers through cb_blend_layer --------------------
    log(f"[bench] {wl.name}: generating {steps + warmup} input copies")
    copies = make_copies(steps + warmup, 0)
    prepared = []
    for cp in copies:
        row = []
        for l, x in enumerate(cp):
            o = runner.outs[l]
            row.append(B.PreparedLayer(runner.geom, runner.batches[l], k=x["k_old"], v=x["v_old"],
                                       k_new_c=x["k_new_c"], v_new_c=x["v_new_c"], q_c=x["q_c"],
                                       delta=x["delta"], cand_idx=runner.candidates(l),
                                       rope_theta=wl.rope_theta, rope_style=B.ROPE_HALF,
                                       softmax_scale=runner.scale, dev=o["dev"],
                                       sel_local=o["sel_local"], sel_global=o["sel_global"],
                                       out=o["out"], workspace=runner.workspace,
                                       dev_source=runner.dev_source,
                                       order=runner.order))
        prepared.append(row)
    # the attribution pass times the entry points of the order the library runs
    # (the same for every layer: it depends on the cache size and the source)
    select_first = prepared[0][0].resolved_order() == B.CB_ORDER_SELECT_FIRST
    stages = STAGES_AFTER if select_first else STAGES
    graph = None
    with torch.cuda.stream(stream):
        for c in range(warmup):
            for p in prepared[c]:
                p.launch(h)
        torch.cuda.synchronize()
        if a.graph:
            # capture records the launches without running them: the timed
            # copies are still pristine when the graph is replayed
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for c in range(warmup, warmup + steps):
                    for p in prepared[c]:
                        p.launch(h)
            torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for c in range(warmup, warmup + steps):
                for p in prepared[c]:
                    p.launch(h)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    del graph
    ms_per_step = ev0.elapsed_time(ev1) / steps
    wall_ms_per_step = (t1 - t0) * 1e3 / steps
    log(f"[bench] timed {steps} steps: {ms_per_step:.4f} ms/step (wall {wall_ms_per_step:.4f})")
    # The inputs plant the deviation tiers in V: a V score must select the
    # planted rows.  K-based scores select other rows; the attention work is
    # then counted on the last step's selection.
    selected = [runner.outs[l]["sel_global"].cpu().numpy() for l in range(L)]
    if a.dev_source == "v":
        for l in range(L):
            if not np.array_equal(selected[l], sets.layer(l).planted):
                raise RuntimeError(f"layer {l}: selection differs from the planted set")
    del prepared, copies
    torch.cuda.empty_cache()

    # ---- attribution pass: each entry point timed over all its launches -----
    lib = B.lib()
    copies = make_copies(steps, 10_000)
    gref = ctypes.byref(runner.geom)
    rgs = [rb.struct() for rb in runner.batches]
    stage_calls = {s: [[] for _ in range(L)] for s in STAGES + STAGES_AFTER}
    topk_calls = [[] for _ in range(L)]   # the selection half alone, for its own time
    keep = []
    # The attention is timed as the launch cb_blend_layer makes: the plan
    # cb_partial_attn chooses, pinned, on a workspace zero-filled once per
    # distinct plan (every call leaves its counters at zero), so no call
    # needs the launch that clears them.
    ws_bytes = 0 if runner.workspace is None else runner.workspace.numel()
    attn_plans, plan_ws = [], {}
    for l in range(L):
        pd = B.attn_plan(runner.geom, runner.batches[l], ws_bytes)
        key = (pd["mfma"], pd["key_split"], pd["key_chunk"])
        if key not in plan_ws:
            plan_ws[key] = B.workspace_tensor(pd["workspace_bytes"], "cuda")
            if plan_ws[key] is not None:
                plan_ws[key].zero_()
        attn_plans.append((B.AttnPlan(key[0], key[1], 0, key[2], 0, 0, 0),
                           *B._ws(plan_ws[key])))
    for cp in copies:
        sels = []
        for l, x in enumerate(cp):
            rb = runner.batches[l]
            dev_t = torch.empty(rb.n_cand, dtype=torch.float32, device="cuda")
            sl = torch.empty(rb.n_sel, dtype=torch.int32, device="cuda")
            sg = torch.empty(rb.n_sel, dtype=torch.int32, device="cuda")
            sels.append(sg)
            src = runner.filter.cand_source(l)
            cand = runner.all_tokens if src is None else sels[src]
            keep += [dev_t, sl, sg]
            k_ptr, v_ptr = x["k_old"].data_ptr(), x["v_old"].data_ptr()
            stage_calls["rerotate"][l].append(
                (lib.cb_rerotate, (gref, k_ptr, k_ptr, x["delta"].data_ptr(), wl.n_tokens, 1,
                                   wl.rope_theta, B.ROPE_HALF, h)))
            stage_calls["deviation_topk"][l].append(
                (lib.cb_kv_deviation_topk, (gref, ctypes.byref(rgs[l]), runner.dev_source,
                                            x["k_new_c"].data_ptr(), k_ptr,
                                            x["v_new_c"].data_ptr(), v_ptr, cand.data_ptr(),
                                            dev_t.data_ptr(), sl.data_ptr(), sg.data_ptr(), h)))
            topk_calls[l].append(
                (lib.cb_topk, (ctypes.byref(rgs[l]), dev_t.data_ptr(), cand.data_ptr(),
                               sl.data_ptr(), sg.data_ptr(), h)))
            stage_calls["fuse_scatter"][l].append(
                (lib.cb_fuse_scatter, (gref, k_ptr, v_ptr, x["k_new_c"].data_ptr(),
                                       x["v_new_c"].data_ptr(), sl.data_ptr(), sg.data_ptr(),
                                       rb.n_sel, h)))
            stage_calls["rerotate_fuse"][l].append(
                (lib.cb_rerotate_fuse, (gref, k_ptr, v_ptr, x["k_new_c"].data_ptr(),
                                        x["v_new_c"].data_ptr(), x["delta"].data_ptr(),
                                        sl.data_ptr(), sg.data_ptr(), rb.n_sel, wl.n_tokens,
                                        wl.rope_theta, B.ROPE_HALF, h)))
            plan, pws_ptr, pws_bytes = attn_plans[l]
            stage_calls["partial_attn"][l].append(
                (lib.cb_partial_attn_with_plan,
                 (gref, ctypes.byref(rgs[l]), ctypes.byref(plan),
                  runner.outs[l]["out"].data_ptr(), x["q_c"].data_ptr(), sl.data_ptr(),
                  sg.data_ptr(), k_ptr, v_ptr, runner.scale, pws_ptr, pws_bytes,
                  B.CB_ATTN_COUNTERS_ZERO, h)))
    events = {}
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        for l in range(L):
            for s in stages:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for fn, args in stage_calls[s][l]:
                    st = fn(*args)
                    if st != 0:
                        B.check(st)
                e1.record(stream)
                events[(l, s)] = (e0, e1)
            # the top-k again on the scores just computed (same outputs)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for fn, args in topk_calls[l]:
                st = fn(*args)
                if st != 0:
                    B.check(st)
            e1.record(stream)
            events[(l, "topk")] = (e0, e1)
        torch.cuda.synchronize()
    stage_ms = {s: sum(events[(l, s)][0].elapsed_time(events[(l, s)][1]) for l in range(L))
                for s in stages}
    launches = steps * L
    work = algorithmic_work(wl, runner, selected, 2 if a.dev_source == "kv" else 1)
    # every layer of every step was launched once
    stage_work = {s: steps * sum(w[s] for w in work) for s in stages}
    kernels = {}
    for s in stages:
        avg_us = stage_ms[s] * 1e3 / launches
        if s == "partial_attn":
            rate = stage_work[s] / (stage_ms[s] * 1e-3) / 1e12
            kernels[s] = {"avg_us": round(avg_us, 3), "tflops": round(rate, 3),
                          "gflop_per_launch": round(stage_work[s] / launches / 1e9, 4)}
        else:
            rate = stage_work[s] / (stage_ms[s] * 1e-3) / 1e9
            kernels[s] = {"avg_us": round(avg_us, 3), "gbs": round(rate, 1),
                          "mb_per_launch": round(stage_work[s] / launches / 1e6, 4)}
    # each class against its published peak and, when measured, the attainable one
    # (MFMA probe for the attention, streaming-read probe for the HBM stages)
    flop_peak_t = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    for s in stages:
        kk = kernels[s]
        if "tflops" in kk:
            kk["frac"] = round(kk["tflops"] / flop_peak_t, 5)
            if peaks and wl.dtype == "bf16":
                kk["frac_attainable"] = round(kk["tflops"] / peaks["mfma_bf16_32x32x16_tflops"], 5)
        else:
            kk["frac"] = round(kk["gbs"] / HBM_PEAK_GBS, 5)
            if peaks:
                kk["frac_attainable"] = round(kk["gbs"] / peaks["read_gbs"], 5)
    topk_ms = sum(events[(l, "topk")][0].elapsed_time(events[(l, "topk")][1]) for l in range(L))
    kernels["topk"] = {"avg_us": round(topk_ms * 1e3 / launches, 3), "bound": "latency"}
    dominant = max(stages, key=lambda s: stage_ms[s])
    if dominant == "partial_attn":
        bf16 = wl.dtype == "bf16"
        peak = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
        achieved = kernels[dominant]["tflops"]
        roof = {"kernel": "partial_attn", "bound": "mfma" if bf16 else "alu",
                "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 5),
                "traffic": recorded_traffic(dominant, wl.name)}
    else:
        achieved = kernels[dominant]["gbs"]
        roof = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                "traffic": recorded_traffic(dominant, wl.name)}
    if peaks:
        att = peaks["mfma_bf16_32x32x16_tflops"] if roof["unit"] == "TFLOP/s" else peaks["read_gbs"]
        if roof["bound"] in ("mfma", "hbm"):
            roof["attainable_peak"] = att
            roof["frac_attainable"] = round(roof["achieved"] / att, 5)
    del stage_calls, copies, keep
    torch.cuda.empty_cache()

    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if a.cpu_seconds > 0:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(wl, a.cpu_seconds, a.dev_source)

    value = wl.n_tokens * L / (ms_per_step * 1e-3)
    # whole-step roofline: streaming bytes at the HBM peak plus attention flops
    # at the MFMA (bf16) or vector (fp32) peak, over the measured step time
    flop_peak = (BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12
    t_star = sum((w["rerotate"] + w["deviation_topk"] + w["fuse_scatter"]) / (HBM_PEAK_GBS * 1e9)
                 + w["partial_attn"] / flop_peak for w in work)
    step_roofline = {"t_star_ms": round(t_star * 1e3, 6),
                     "frac": round(t_star / (ms_per_step * 1e-3), 5)}
    ratio = (f"r={wl.r1_pct}%" if wl.n_layers == 1
             else f"r1={wl.r1_pct}% -> r2={wl.r2_pct}%")
    line = {
        "metric": "blended context tokens/s per layer (1 GPU) + % HBM / MFMA roofline",
        "value": round(value, 1), "unit": "tokens/s/layer", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "tokens": wl.n_tokens,
                   "layers": L, "requests": wl.n_requests, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "selection": ratio,
                   "hkvd_pct": wl.hkvd_pct, "schedule": a.schedule,
                   "dev_source": a.dev_source,
                   "order": f"{a.order}: " + ("select, then rotate-or-replace" if select_first
                                              else "rotate, select, fuse"),
                   "launch": "hip graph replay" if a.graph else "stream launches"},
        "roofline": roof,
        "step_roofline": step_roofline,
        "attainable": peaks,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "wall_ms_per_step": round(wall_ms_per_step, 5),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
