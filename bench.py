#!/usr/bin/env python3
"""Throughput of the CacheBlend KV-fusion step on one MI355X.

A step is one pass of the whole hot path -- for every layer of the workload:
re-rotate the cached keys, score and select the candidates, fuse the
recomputed rows, and run the selected rows' causal GQA attention -- over one
batch of seeded synthetic input already resident in HBM.  The blend works in
place on the cached K/V, so the run keeps one pristine and one working copy
of every layer's K/V: before each step (untimed) the working copy is restored
from the pristine one and the 256 MB Infinity Cache is flushed by reading
512 MiB, so no step reads another step's results or starts from a warm MALL;
then a bounded spin kernel keeps the GPU busy while the host enqueues the
step, so the events time the GPU's work rather than the host's launch rate.
Each step's L-layer loop is timed with its own pair of HIP events on the
launch stream; ms_per_step is the median over the timed steps.

Default workload: the batched 70B-layer blend (8 ragged requests, 67 100
tokens, 80 layers, 64 Q / 8 KV heads), the largest single-GPU configuration.

Metric: blended context tokens per second per layer = tokens * layers / time.

Printed: one JSON line with the metric, a roofline entry for the dominant
kernel (algorithmic work per launch / its average launch time, measured with
HIP events on the launch stream, against the published peak and against the
peak measured by the in-tree probe `cb_peaks`), the whole-step roofline
fraction (streaming bytes at 8 TB/s plus attention flops at the MFMA peak,
over the step time), per-kernel figures (each stage's rate and its fraction of
the published and the measured peak; the top-k also timed on its own), the
selection objective of the deviation top-k against random selections, and the
CPU oracle timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # fp32 vector
DEFAULT_WORKLOAD = "70b-80layer-8req"
DEFAULT_STEPS = {"tiny": (200, 20), "mistral7b-layer": (200, 20), "7b-32layer-6k": (20, 5),
                 "7b-32layer-32k": (20, 5), "70b-80layer-8req": (20, 5)}
STAGES = ("rerotate", "deviation_topk", "fuse_scatter", "partial_attn")
# the order that scores and selects first, then rotates-or-replaces in one pass
STAGES_AFTER = ("deviation_topk", "rerotate_fuse", "partial_attn")
PROFILES = os.path.join(ROOT, "profiles")
FLUSH_BYTES = 512 << 20        # twice the Infinity Cache
CPU_WORKERS_MAX = 16           # host CPU share of one GPU


def source_fingerprint():
    """sha256 over the library sources (its compiled files, their headers and
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
    from selective_recompute_amd import build as BLD
    if not os.path.exists(BLD.PEAKS):
        return None
    res = subprocess.run([BLD.PEAKS], capture_output=True, text=True, timeout=120)
    if res.returncode != 0:
        log(f"[bench] peak probe failed: {res.stderr.strip()}")
        return None
    return json.loads(res.stdout.strip().splitlines()[-1])


def mfma_attainable(peaks):
    """The attainable bf16 MFMA rate for real data: the probe's figure on
    pseudo-random operands (the chip clocks lower when more operand bits
    toggle), or its smooth-operand figure where an older probe lacks it."""
    return peaks.get("mfma_bf16_32x32x16_random_tflops") or peaks["mfma_bf16_32x32x16_tflops"]


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


def parse_args(argv=None):
    from selective_recompute_amd import workloads as W
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(W.WORKLOADS))
    ap.add_argument("--schedule", default="pool", choices=["pool", "chain"])
    ap.add_argument("--dev-source", default="v", choices=["v", "k", "kv"],
                    help="what the token deviation measures: V (default), K at the new "
                         "position, or the K and V rows as one vector")
    ap.add_argument("--order", default="auto", choices=["auto", "rotate-first", "select-first"],
                    help="step order of cb_blend_layer: select-first scores V and selects "
                         "first, then one launch writes the rows of S and re-rotates only the "
                         "others; auto lets the library choose")
    ap.add_argument("--select-in-launch", type=int, default=0,
                    help="1: the top-k runs inside the deviation launch (a zero-filled "
                         "workspace, CB_LAYER_WORKSPACE_ZEROED); 0: its own launch")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="rough budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--attainable", type=int, default=1,
                    help="1: measure attainable MFMA / HBM peaks first and report "
                         "fractions against them too")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: capture one step's launches in a HIP graph and time its "
                         "replay (same kernels, no host launch cost)")
    ap.add_argument("--attribution", type=int, default=1,
                    help="1: also time every entry point on its own (per-kernel figures "
                         "and the roofline entry)")
    ap.add_argument("--objective", type=int, default=1,
                    help="1: also report the selection objective of the deviation top-k "
                         "against random selections (library kernels, c1's shape)")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the blend step: dense causal attention of every "
                         "row (layer-1 full prefill) at the workload's shape")
    ap.add_argument("--print-source-sha", action="store_true",
                    help="print the sources' fingerprint and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB device to device once (a "
                         "plain copy of known size that calibrates byte counters)")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help=argparse.SUPPRESS)  # the child process that times the oracle
    return ap.parse_args(argv)


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


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the workload.
# It runs in a child process started before this process touches the GPU.
# --------------------------------------------------------------------------
_POOL_ARGS = None


def _pool_init(args):
    global _POOL_ARGS
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)          # one thread per process: the pool is the parallelism
    _POOL_ARGS = args


def _pool_rows(rows):
    from oracle import cacheblend_oracle as O
    a = _POOL_ARGS
    O.attention_rows(a["q_c"], a["sel_local"][rows], a["sel_global"][rows], a["row_start"][rows],
                     a["k_fused"], a["v_fused"], a["n_q_heads"], a["n_kv_heads"], a["scale"])
    return len(rows)


def _oracle_layer_time(wl, sets, layer, frac, workers, dev_source):
    """Seconds the oracle takes for one layer: every step but the attention in
    full (plain numpy, one thread), the attention on every frac-th selected
    row over a pool of `workers` processes, its wall time scaled by frac."""
    import multiprocessing as mp

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import cacheblend_oracle as O
    from selective_recompute_amd import workloads as W

    x = W.layer_inputs(wl, sets, layer, device="cpu")
    f64 = lambda t: t.to(torch.float64).numpy()
    pct = wl.r1_pct if layer == 0 else wl.r2_pct
    args = dict(k_old=f64(x["k_old"]), v_old=f64(x["v_old"]), delta=wl.delta(),
                k_new_c=f64(x["k_new_c"]), v_new_c=f64(x["v_new_c"]), q_c=f64(x["q_c"]),
                cand_idx=x["cand_idx"].numpy(), tok_off=wl.tok_off, cand_off=x["h_cand_off"],
                sel_counts=[(pct * n + 99) // 100 for n in wl.request_lengths],
                n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, theta=wl.rope_theta,
                scale=1.0 / math.sqrt(wl.head_dim))
    del x
    with threadpool_limits(1):
        # repeated while short (about 1 s), so one cold pass does not decide it
        reps, t0 = 0, time.perf_counter()
        while True:
            res = O.blend_layer(**args, attend=False, dev_source=dev_source)
            reps += 1
            if time.perf_counter() - t0 >= 1.0:
                break
        t_steps = (time.perf_counter() - t0) / reps
    n_sel = len(res["sel_global"])
    rows = np.arange(0, n_sel, frac)
    blocks = [b for b in np.array_split(rows, max(1, min(len(rows), workers * 8))) if len(b)]
    pool_args = dict(q_c=args["q_c"], sel_local=res["sel_local"], sel_global=res["sel_global"],
                     row_start=res["row_start"], k_fused=res["k_fused"], v_fused=res["v_fused"],
                     n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, scale=args["scale"])
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init, initargs=(pool_args,)) as pool:
        t0 = time.perf_counter()
        done = sum(pool.map(_pool_rows, blocks, chunksize=1))
        t_attn = time.perf_counter() - t0
    assert done == len(rows)
    return t_steps + t_attn * frac, t_steps, t_attn, n_sel, len(rows)


def cpu_baseline(wl, seconds, dev_source="v"):
    """Oracle tokens/s per layer on this host: layer 1 (every token a
    candidate) and, for multi-layer workloads, layer 2 (the later layers'
    shape), extrapolated to the whole stack."""
    workers = max(1, min(CPU_WORKERS_MAX, len(os.sched_getaffinity(0))))
    from selective_recompute_amd import workloads as W
    sets = W.PlantedSets(wl)
    # attention sample: aim at about `seconds` of attention work on the pool
    # (about 4 s per 64 heads of the 32k-token rows and 1k sampled rows)
    k1 = sum((wl.r1_pct * n + 99) // 100 for n in wl.request_lengths)
    avg_keys = sum(n * n / 2 for n in wl.request_lengths) / max(1, wl.n_tokens)
    est_per_row = 2.0e-9 * wl.n_q_heads * avg_keys * wl.head_dim + 2e-5 * wl.n_q_heads
    frac = max(1, int(math.ceil(k1 * est_per_row / workers / max(seconds, 1.0) * 2)))
    layers = [0] if wl.n_layers == 1 else [0, 1]
    times, parts = [], []
    for layer in layers:
        t, t_steps, t_attn, n_sel, n_rows = _oracle_layer_time(wl, sets, layer, frac, workers,
                                                               dev_source)
        times.append(t)
        parts.append(f"layer {layer + 1}: {n_sel} selected rows, re-rotation/deviation/"
                     f"top-k/fuse {t_steps:.2f} s on one thread, attention of {n_rows} rows "
                     f"(every {frac}th) {t_attn:.2f} s on {workers} processes")
    total = times[0] + (wl.n_layers - 1) * (times[1] if len(times) > 1 else times[0])
    sample = (f"{wl.name}, the unchanged float64 numpy oracle; " + "; ".join(parts)
              + (f"; attention wall time scaled by {frac}" if frac > 1 else ""))
    if wl.n_layers > 1:
        sample += (f"; stack time = layer 1 + {wl.n_layers - 1} x layer 2 (later layers share "
                   "layer 2's candidate and selection counts)")
    return {"value": wl.n_tokens * wl.n_layers / total, "unit": "tokens/s/layer",
            "cores": workers, "kind": "oracle", "sample": sample}


def run_cpu_baseline_child(a):
    """The CPU baseline in a child process (started before this process
    initialises the GPU); None if it fails."""
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", "--workload",
           a.workload, "--cpu-seconds", str(a.cpu_seconds), "--dev-source", a.dev_source]
    log("[bench] timing the CPU oracle")
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    if res.returncode != 0:
        log(f"[bench] CPU baseline failed: {res.stderr.strip()[-2000:]}")
        return None
    out = json.loads(res.stdout.strip().splitlines()[-1])
    log(f"[bench] CPU oracle: {out['value']:.4g} tokens/s/layer on {out['cores']} processes")
    return out


def prefill_main(a, peaks):
    """Layer-1 full prefill: every row of every request attends causally over
    its request, through the same cb_partial_attn entry point (all rows
    selected).  Prints one JSON line in TFLOP/s."""
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
        roof["attainable_peak"] = mfma_attainable(peaks)
        roof["frac_attainable"] = round(tf / mfma_attainable(peaks), 5)
    print(json.dumps({
        "metric": "dense causal attention TFLOP/s (layer-1 full prefill)", "value": round(tf, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} shape, every row selected", "tokens": t_count,
                   "requests": len(lens), "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "gflop_per_launch": round(flops / 1e9, 3)},
        "roofline": roof, "attainable": peaks}), flush=True)


def selection_objective():
    """[Derivations, "形式化"] objective at the Mistral-7B-shaped layer (4 chunks
    of 512 tokens, 32 / 8 heads, bf16), through the library only: the norm of
    the difference between every row's attention over the fused cache and
    over full recompute, for the deviation top-k ([Derivations, "近似解"]), for
    8 random selections of the same size, for no recompute and for the top-k
    over a cache that is not re-rotated.  Keys: one content rotated (by the
    library) to chunk-local cached and global recomputed positions; values
    deviate strongly on 15% of the tokens."""
    import torch

    from selective_recompute_amd import binding as B
    from selective_recompute_amd import pipeline as PL

    hq, hkv, d, theta, chunk, n_chunks = 32, 8, 128, 10000.0, 512, 4
    t = chunk * n_chunks
    k_sel = PL.select_count(15, t)
    gen = torch.Generator(device="cuda").manual_seed(0xCB0E)
    rnd = lambda *shape: torch.randn(*shape, generator=gen, device="cuda")
    p_old = torch.arange(chunk, dtype=torch.int32, device="cuda").repeat(n_chunks)
    p_new = torch.arange(t, dtype=torch.int32, device="cuda")
    g_kv, g_q, g = B.geom(hkv, hkv, d, torch.bfloat16), B.geom(hq, hq, d, torch.bfloat16), \
        B.geom(hq, hkv, d, torch.bfloat16)

    def rotated(x, pos, geom):
        out = torch.empty_like(x)
        B.rerotate(geom, out, x, pos, t, 1, theta)
        return out

    k_base = rnd(t, hkv, d)
    k_old = rotated(k_base.to(torch.bfloat16), p_old, g_kv)
    k_new = rotated((k_base + 0.01 * rnd(t, hkv, d)).to(torch.bfloat16), p_new, g_kv)
    q = rotated(rnd(t, hq, d).to(torch.bfloat16), p_new, g_q)
    v_old = rnd(t, hkv, d).to(torch.bfloat16)
    hot = torch.randperm(t, generator=gen, device="cuda")[:k_sel]
    sigma = torch.full((t, 1, 1), 0.01, device="cuda")
    sigma[hot] = 1.0
    v_new = (v_old.float() + sigma * rnd(t, hkv, d)).to(torch.bfloat16)
    delta = p_new - p_old
    every = torch.arange(t, dtype=torch.int32, device="cuda")
    rb_all = B.RaggedBatch([0, t], [0, t], [0, t], "cuda")
    ws = B.workspace_tensor(B.attn_workspace_bytes(g, rb_all))
    scale = 1.0 / math.sqrt(d)

    def attend(keys, vals):
        out = torch.empty((t, hq, d), dtype=torch.bfloat16, device="cuda")
        B.partial_attn(g, rb_all, out, q, every, every, keys, vals, scale, ws)
        return out

    full = attend(k_new, v_new).float()

    def error(sel, rerotate_cache=True):
        sel = torch.sort(sel.to(torch.int32)).values
        keys, vals = k_old.clone(), v_old.clone()
        if rerotate_cache:
            B.rerotate(g_kv, keys, keys, delta, t, 1, theta)
        B.fuse_scatter(g, keys, vals, k_new, v_new, sel, sel, len(sel))
        return float(torch.linalg.vector_norm(attend(keys, vals).float() - full))

    rb = B.RaggedBatch([0, t], [0, t], [0, k_sel], "cuda")
    dev = torch.empty(t, dtype=torch.float32, device="cuda")
    sl = torch.empty(k_sel, dtype=torch.int32, device="cuda")
    sg = torch.empty(k_sel, dtype=torch.int32, device="cuda")
    B.deviation_topk(g, rb, v_new, v_old, every, dev, sl, sg)
    e_rand = [error(torch.randperm(t, generator=gen, device="cuda")[:k_sel]) for _ in range(8)]
    return {"objective": "||Attn(Q,K_fused,V_fused) - Attn(Q,K_new,V_new)|| over every row",
            "shape": "4x512 tokens, 32/8 heads, head_dim 128, bf16, 15% selected",
            "hkvd_topk": round(error(sg), 4),
            "random_min": round(min(e_rand), 4), "random_mean": round(sum(e_rand) / 8, 4),
            "random_max": round(max(e_rand), 4), "random_draws": 8,
            "no_recompute": round(error(sg[:0]), 4),
            "hkvd_topk_cache_not_rerotated": round(error(sg, rerotate_cache=False), 4)}


class Inputs:
    """Every layer's inputs on the device, generated once.  K and V of all
    layers live in one working and one pristine tensor each: restore() copies
    the pristine caches over the working ones and then reads FLUSH_BYTES of
    an unrelated buffer, so that nothing of the previous step (nor of the
    restore) stays in L2 or the Infinity Cache.  A read evicts with clean
    lines: a written flush would leave dirty lines whose write-back lands
    inside the next step."""

    def __init__(self, wl, sets):
        import torch

        from selective_recompute_amd import workloads as W
        L, T = wl.n_layers, wl.n_tokens
        shape = (L, T, wl.n_kv_heads, wl.head_dim)
        dt = wl.torch_dtype
        self.k_work = torch.empty(shape, dtype=dt, device="cuda")
        self.v_work = torch.empty(shape, dtype=dt, device="cuda")
        self.k_pristine = torch.empty(shape, dtype=dt, device="cuda")
        self.v_pristine = torch.empty(shape, dtype=dt, device="cuda")
        self.layers = []
        for layer in range(L):
            x = W.layer_inputs(wl, sets, layer, device="cuda")
            self.k_pristine[layer].copy_(x.pop("k_old"))
            self.v_pristine[layer].copy_(x.pop("v_old"))
            x["k_old"], x["v_old"] = self.k_work[layer], self.v_work[layer]
            self.layers.append(x)
        self.flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.flush_sum = torch.zeros((), dtype=torch.int64, device="cuda")
        self._sum = torch.sum
        self._i64 = torch.int64

    def restore(self):
        self.k_work.copy_(self.k_pristine)
        self.v_work.copy_(self.v_pristine)
        self._sum(self.flush, dim=0, dtype=self._i64, out=self.flush_sum)


class HeadStart:
    """Keeps the GPU busy while the host enqueues a step, so that the events
    around the step (or around each launch of the attribution pass) time the
    GPU's work and not the rate at which the host can launch.  Before each
    step, outside the events, it enqueues torch's bounded spin kernel
    (torch.cuda._sleep) for 1.5x the host's enqueue time of the previous
    step, at least 100 us and at most 50 ms."""

    MIN_US, MAX_US = 100.0, 50000.0

    def __init__(self, torch, stream):
        self._sleep = torch.cuda._sleep
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            self._sleep(1000)
            e0.record(stream)
            self._sleep(1 << 21)
            e1.record(stream)
        torch.cuda.synchronize()
        self.cycles_per_us = (1 << 21) / max(e0.elapsed_time(e1) * 1e3, 1.0)
        self.us = self.MIN_US
        self._t = None

    def __call__(self):
        """Enqueue the spin, then start the host clock of the step."""
        self._sleep(int(self.us * self.cycles_per_us))
        self._t = time.perf_counter()

    def done(self):
        """The step is enqueued: size the next spin to the host's time."""
        host_us = (time.perf_counter() - self._t) * 1e6
        self.us = min(self.MAX_US, max(self.MIN_US, 1.5 * host_us))


def main():
    a = parse_args()
    if a.print_source_sha:
        print(source_fingerprint())
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported (this build runs "
              "on one GPU only and has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if a.cpu_baseline_only:
        from selective_recompute_amd import workloads as W
        print(json.dumps(cpu_baseline(W.make_workload(a.workload), a.cpu_seconds, a.dev_source)),
              flush=True)
        return
    # child processes first: nothing below them has touched the GPU yet
    peaks = attainable_peaks() if a.attainable else None
    if a.prefill:
        return prefill_main(a, peaks)
    cpu = run_cpu_baseline_child(a) if a.cpu_seconds > 0 else None

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
    if steps < 1:
        raise SystemExit("--steps must be >= 1")
    L = wl.n_layers
    sets = W.PlantedSets(wl, a.schedule)
    runner = PL.BlendRunner(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.torch_dtype,
                            wl.request_lengths, wl.r1_pct, wl.r2_pct, L, wl.rope_theta,
                            schedule=a.schedule, dev_source=a.dev_source, device="cuda",
                            order=a.order, in_launch_select=bool(a.select_in_launch))
    if a.order == "select-first" and a.dev_source != "v":
        raise SystemExit("--order select-first scores V only (a key deviation reads the "
                         "re-rotated keys)")
    stream = torch.cuda.Stream()
    h = stream.cuda_stream

    log(f"[bench] {wl.name}: generating the inputs of {L} layer(s)")
    inp = Inputs(wl, sets)
    torch.cuda.synchronize()
    prepared = []
    for l, x in enumerate(inp.layers):
        o = runner.outs[l]
        prepared.append(B.PreparedLayer(runner.geom, runner.batches[l], k=x["k_old"],
                                        v=x["v_old"], k_new_c=x["k_new_c"], v_new_c=x["v_new_c"],
                                        q_c=x["q_c"], delta=x["delta"],
                                        cand_idx=runner.candidates(l), rope_theta=wl.rope_theta,
                                        rope_style=B.ROPE_HALF, softmax_scale=runner.scale,
                                        dev=o["dev"], sel_local=o["sel_local"],
                                        sel_global=o["sel_global"], out=o["out"],
                                        workspace=runner.workspace, dev_source=runner.dev_source,
                                        order=runner.order, flags=runner.flags))
    # the attribution pass times the entry points of the order the library runs
    # (the same for every layer: it depends on the cache size and the source)
    select_first = prepared[0].resolved_order() == B.CB_ORDER_SELECT_FIRST
    stages = STAGES_AFTER if select_first else STAGES

    def launch_step():
        for p in prepared:
            p.launch(h)

    # ---- timed pass: whole layers through cb_blend_layer --------------------
    graph = None
    step_events = []
    head = HeadStart(torch, stream)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            inp.restore()
            head()
            launch_step()
            head.done()
        torch.cuda.synchronize()
        if a.graph:
            # capture records the launches without running them
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                launch_step()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            inp.restore()                                   # untimed: outside the events
            head()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if graph is not None:
                graph.replay()
            else:
                launch_step()
            e1.record(stream)
            head.done()
            step_events.append((e0, e1))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    del graph
    step_ms = [e0.elapsed_time(e1) for e0, e1 in step_events]
    ms_per_step = statistics.median(step_ms)
    log(f"[bench] timed {steps} steps: median {ms_per_step:.4f} ms/step (min {min(step_ms):.4f}, "
        f"max {max(step_ms):.4f}); timed region with restores {t1 - t0:.2f} s")
    # The inputs plant the deviation tiers in V: a V score must select the
    # planted rows.  K-based scores select other rows; the attention work is
    # then counted on the last step's selection.
    selected = [runner.outs[l]["sel_global"].cpu().numpy() for l in range(L)]
    if a.dev_source == "v":
        for l in range(L):
            if not np.array_equal(selected[l], sets.layer(l).planted):
                raise RuntimeError(f"layer {l}: selection differs from the planted set")
    work = algorithmic_work(wl, runner, selected, 2 if a.dev_source == "kv" else 1)

    kernels, roof = {}, None
    if a.attribution:
        kernels, roof = attribution_pass(a, wl, runner, inp, stream, stages, steps, warmup, work,
                                         peaks)

    objective = selection_objective() if a.objective else None

    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

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
                   "launch": "hip graph replay" if a.graph else "stream launches",
                   "select": ("top-k inside the deviation launch" if runner.flags
                              else "top-k in its own launch"),
                   "step_timing": "median of per-step HIP event pairs; K/V restored from a "
                                  "pristine copy, 512 MiB read (L2 and MALL flush) and a spin "
                                  "that outlasts the host's enqueue of the step, before each "
                                  "step, outside the events"},
        "roofline": roof,
        "step_roofline": step_roofline,
        "attainable": peaks,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "selection_objective": objective,
        "step_ms": {"median": round(ms_per_step, 5), "mean": round(statistics.mean(step_ms), 5),
                    "min": round(min(step_ms), 5), "max": round(max(step_ms), 5)},
        "timed_region_s": round(t1 - t0, 3),
    }
    print(json.dumps(line), flush=True)


def attribution_pass(a, wl, runner, inp, stream, stages, steps, warmup, work, peaks):
    """Each entry point of the step timed on its own, layer by layer, over as
    many restored steps as the timed pass; returns (kernels, roofline entry of
    the dominant one)."""
    import torch

    from selective_recompute_amd import binding as B

    L = wl.n_layers
    h = stream.cuda_stream
    lib = B.lib()
    gref = ctypes.byref(runner.geom)
    rgs = [rb.struct() for rb in runner.batches]
    stage_calls = {s: [None] * L for s in STAGES + STAGES_AFTER}
    topk_calls = [None] * L   # the selection half alone, for its own time
    # The attention is timed as the launch cb_blend_layer makes: the plan
    # cb_partial_attn chooses, pinned, on a workspace zero-filled once per
    # distinct plan (every call leaves its counters at zero), so no call
    # needs the launch that clears them.
    ws_bytes = 0 if runner.workspace is None else runner.workspace.numel()
    if runner.flags & B.CB_LAYER_WORKSPACE_ZEROED and ws_bytes >= B.CB_SELECT_COUNTER_BYTES + 256:
        ws_bytes = (ws_bytes - B.CB_SELECT_COUNTER_BYTES) & ~255   # what the attention gets
    plan_ws, keep = {}, []
    for l, x in enumerate(inp.layers):
        rb, o = runner.batches[l], runner.outs[l]
        pd = B.attn_plan(runner.geom, rb, ws_bytes)
        key = (pd["mfma"], pd["key_split"], pd["key_chunk"], pd["stream_spans"])
        if key not in plan_ws:
            plan_ws[key] = B.workspace_tensor(pd["workspace_bytes"], "cuda")
        plan = B.AttnPlan(key[0], key[1], 0, key[2], 0, 0, 0, key[3])
        keep.append(plan)
        pws_ptr, pws_bytes = B._ws(plan_ws[key])
        cand = runner.candidates(l)
        dev_t, sl, sg = o["dev"], o["sel_local"], o["sel_global"]
        k_ptr, v_ptr = x["k_old"].data_ptr(), x["v_old"].data_ptr()
        stage_calls["rerotate"][l] = (lib.cb_rerotate, (gref, k_ptr, k_ptr, x["delta"].data_ptr(),
                                                         wl.n_tokens, 1, wl.rope_theta,
                                                         B.ROPE_HALF, h))
        stage_calls["deviation_topk"][l] = (
            lib.cb_kv_deviation_topk, (gref, ctypes.byref(rgs[l]), runner.dev_source,
                                       x["k_new_c"].data_ptr(), k_ptr, x["v_new_c"].data_ptr(),
                                       v_ptr, cand.data_ptr(), dev_t.data_ptr(), sl.data_ptr(),
                                       sg.data_ptr(), h))
        topk_calls[l] = (lib.cb_topk, (ctypes.byref(rgs[l]), dev_t.data_ptr(), cand.data_ptr(),
                                       sl.data_ptr(), sg.data_ptr(), h))
        stage_calls["fuse_scatter"][l] = (
            lib.cb_fuse_scatter, (gref, k_ptr, v_ptr, x["k_new_c"].data_ptr(),
                                  x["v_new_c"].data_ptr(), sl.data_ptr(), sg.data_ptr(), rb.n_sel,
                                  h))
        stage_calls["rerotate_fuse"][l] = (
            lib.cb_rerotate_fuse, (gref, k_ptr, v_ptr, x["k_new_c"].data_ptr(),
                                   x["v_new_c"].data_ptr(), x["delta"].data_ptr(), sl.data_ptr(),
                                   sg.data_ptr(), rb.n_sel, wl.n_tokens, wl.rope_theta,
                                   B.ROPE_HALF, h))
        stage_calls["partial_attn"][l] = (
            lib.cb_partial_attn_with_plan,
            (gref, ctypes.byref(rgs[l]), ctypes.byref(plan), o["out"].data_ptr(),
             x["q_c"].data_ptr(), sl.data_ptr(), sg.data_ptr(), k_ptr, v_ptr, runner.scale,
             pws_ptr, pws_bytes, B.CB_ATTN_COUNTERS_ZERO, h))

    def call(fn_args):
        fn, args = fn_args
        st = fn(*args)
        if st != 0:
            B.check(st)

    totals = {s: 0.0 for s in stages}
    topk_ms = 0.0
    head = HeadStart(torch, stream)
    with torch.cuda.stream(stream):
        for step in range(warmup + steps):
            inp.restore()
            head()
            evs = []
            for l in range(L):
                for s in stages:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    call(stage_calls[s][l])
                    e1.record(stream)
                    evs.append((s, e0, e1))
                # the top-k again on the scores just computed (same outputs)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call(topk_calls[l])
                e1.record(stream)
                evs.append(("topk", e0, e1))
            head.done()
            torch.cuda.synchronize()
            if step < warmup:
                continue
            for s, e0, e1 in evs:
                if s == "topk":
                    topk_ms += e0.elapsed_time(e1)
                else:
                    totals[s] += e0.elapsed_time(e1)
    launches = steps * L
    stage_work = {s: steps * sum(w[s] for w in work) for s in stages}
    kernels = {}
    for s in stages:
        avg_us = totals[s] * 1e3 / launches
        if s == "partial_attn":
            rate = stage_work[s] / (totals[s] * 1e-3) / 1e12
            kernels[s] = {"avg_us": round(avg_us, 3), "tflops": round(rate, 3),
                          "gflop_per_launch": round(stage_work[s] / launches / 1e9, 4)}
        else:
            rate = stage_work[s] / (totals[s] * 1e-3) / 1e9
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
                kk["frac_attainable"] = round(kk["tflops"] / mfma_attainable(peaks), 5)
        else:
            kk["frac"] = round(kk["gbs"] / HBM_PEAK_GBS, 5)
            if peaks:
                kk["frac_attainable"] = round(kk["gbs"] / peaks["read_gbs"], 5)
    kernels["topk"] = {"avg_us": round(topk_ms * 1e3 / launches, 3), "bound": "latency"}
    dominant = max(stages, key=lambda s: totals[s])
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
        att = mfma_attainable(peaks) if roof["unit"] == "TFLOP/s" else peaks["read_gbs"]
        if roof["bound"] in ("mfma", "hbm"):
            roof["attainable_peak"] = att
            roof["frac_attainable"] = round(roof["achieved"] / att, 5)
    del stage_calls, keep, plan_ws
    torch.cuda.empty_cache()
    return kernels, roof


if __name__ == "__main__":
    main()
