"""The selection objective on the GPU path, checked against the oracle.

[Derivations, "形式化"] scores a choice S of recomputed tokens by how far the
layer's attention over the fused cache lies from full recompute, and
[Derivations, "近似解"] approximates the best S by the tokens of largest KV
deviation.  Inputs (c1's shape: 4 chunks of 512 tokens, 32 / 8 heads, head
dimension 128, bf16): one key content rotated by the oracle to its
chunk-local (cached) and its global (recomputed) positions, values that
deviate strongly on 15% of the tokens.  The library then re-rotates the
cache (cb_rerotate), selects (cb_deviation_topk), fuses (cb_fuse_scatter)
and attends with every row (cb_partial_attn); the oracle does the same from
the same stored tensors.  Per selection -- full recompute, the deviation
top-k, eight random selections of the same size, none, and the top-k over
an unrotated cache -- the GPU rows must match the oracle's to 2e-2 on
sampled rows, and the objective on those rows (the norm of the difference
to full recompute) must agree between the two.  Both sides must rank the
deviation top-k far ahead of every random choice.
"""
import math

import numpy as np
import pytest
import torch

from oracle import cacheblend_oracle as O
from selective_recompute_amd import binding as B
from selective_recompute_amd import pipeline as PL

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATTN_ABS = 2e-2


def say(msg):
    print(f"\n[objective] {msg}", flush=True)


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def test_deviation_selection_beats_random_on_gpu_and_in_the_oracle():
    hq, hkv, d, theta = 32, 8, 128, 10000.0
    chunk, n_chunks = 512, 4
    t = chunk * n_chunks
    k_sel = PL.select_count(15, t)
    gen = torch.Generator().manual_seed(0xCB0F)
    rng = np.random.default_rng(0xCB0F)
    p_old = np.tile(np.arange(chunk), n_chunks)
    p_new = np.arange(t)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)
    # stored inputs (bf16): the same key content at chunk-local (cached) and
    # global (recomputed) positions; recomputed keys and values move a little
    # everywhere and the values a lot on 15% of the tokens
    k_base = torch.randn(t, hkv, d, generator=gen, dtype=torch.float64).numpy()
    k_old = bf(O.rotate(k_base, p_old, theta))
    k_new = bf(O.rotate(k_base + 0.01 * torch.randn(t, hkv, d, generator=gen,
                                                    dtype=torch.float64).numpy(), p_new, theta))
    q = bf(O.rotate(torch.randn(t, hq, d, generator=gen, dtype=torch.float64).numpy(), p_new, theta))
    v_old = torch.randn(t, hkv, d, generator=gen).to(torch.bfloat16)
    hot = np.sort(rng.choice(t, k_sel, replace=False))
    sigma = np.full((t, 1, 1), 0.01)
    sigma[hot] = 1.0
    v_new = bf(np64(v_old) + sigma * torch.randn(t, hkv, d, generator=gen,
                                                 dtype=torch.float64).numpy())
    delta = (p_new - p_old).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    random_sels = [np.sort(rng.choice(t, k_sel, replace=False)) for _ in range(8)]

    # ---- the library ----------------------------------------------------------
    g_kv = B.geom(hkv, hkv, d, torch.bfloat16)
    g = B.geom(hq, hkv, d, torch.bfloat16)
    kd_old, kd_new, qd, vd_old, vd_new = (x.to(DEV) for x in (k_old, k_new, q, v_old, v_new))
    deltad = torch.from_numpy(delta).to(DEV)
    every = torch.arange(t, dtype=torch.int32, device=DEV)
    rb_all = B.RaggedBatch([0, t], [0, t], [0, t], DEV)
    ws = B.workspace_tensor(B.attn_workspace_bytes(g, rb_all))

    def attend_all(keys, vals):
        out = torch.empty((t, hq, d), dtype=torch.bfloat16, device=DEV)
        B.partial_attn(g, rb_all, out, qd, every, every, keys, vals, scale, ws)
        return out

    def gpu_fused(sel, rerotate_cache=True):
        sel = torch.from_numpy(np.asarray(sel, np.int32)).to(DEV)
        keys, vals = kd_old.clone(), vd_old.clone()
        if rerotate_cache:
            B.rerotate(g_kv, keys, keys, deltad, t, 1, theta)
        B.fuse_scatter(g, keys, vals, kd_new, vd_new, sel, sel, len(sel))
        return attend_all(keys, vals)

    rb = B.RaggedBatch([0, t], [0, t], [0, k_sel], DEV)
    dev = torch.empty(t, dtype=torch.float32, device=DEV)
    sl = torch.empty(k_sel, dtype=torch.int32, device=DEV)
    sg = torch.empty(k_sel, dtype=torch.int32, device=DEV)
    B.deviation_topk(g, rb, vd_new, vd_old, every, dev, sl, sg)
    gpu_sel = sg.cpu().numpy().astype(np.int64)
    cases = {"full": attend_all(kd_new, vd_new), "top-k": gpu_fused(gpu_sel),
             "none": gpu_fused(np.zeros(0, np.int64)),
             "top-k, cache not re-rotated": gpu_fused(gpu_sel, rerotate_cache=False)}
    for i, s in enumerate(random_sels):
        cases[f"random {i}"] = gpu_fused(s)
    torch.cuda.synchronize()
    gpu = {name: np64(out) for name, out in cases.items()}

    # ---- the oracle, from the same stored tensors ------------------------------
    f64 = lambda x: np64(x)
    ko, kn, qo, vo, vn = f64(k_old), f64(k_new), f64(q), f64(v_old), f64(v_new)
    dev_o = O.deviation(vn, vo, np.arange(t))
    _, sel_o = O.topk_select(dev_o, np.arange(t), k_sel)
    assert np.array_equal(gpu_sel, sel_o)
    assert np.array_equal(sel_o, hot)
    k_rot = O.rerotate(ko, delta, theta)
    rows = np.unique(np.concatenate([[0, chunk - 1, chunk, t - 1],
                                     rng.choice(t, 44, replace=False)]))
    start = np.zeros(len(rows), np.int64)

    def oracle_attend(keys, vals):
        return O.attention_rows(qo[rows], np.arange(len(rows)), rows, start, keys, vals, hq, hkv,
                                scale)

    def oracle_fused(sel, keys=k_rot):
        sel = np.asarray(sel, np.int64)
        k_f, v_f = O.fuse(keys, vo, kn, vn, sel, sel)
        return oracle_attend(k_f, v_f)

    ref = {"full": oracle_attend(kn, vn), "top-k": oracle_fused(sel_o),
           "none": oracle_fused(np.zeros(0, np.int64)),
           "top-k, cache not re-rotated": oracle_fused(sel_o, keys=ko)}
    for i, s in enumerate(random_sels):
        ref[f"random {i}"] = oracle_fused(s)

    # ---- per-row parity and the objective on the sampled rows --------------------
    objective_gpu, objective_ref = {}, {}
    for name in ref:
        err = np.abs(gpu[name][rows] - ref[name]).max()
        assert err <= ATTN_ABS, f"{name}: attention max err {err}"
        objective_gpu[name] = float(np.linalg.norm(gpu[name][rows] - gpu["full"][rows]))
        objective_ref[name] = float(np.linalg.norm(ref[name] - ref["full"]))
    # the GPU's objective is the oracle's to the rounding of the outputs: each
    # element of both outputs lies within ATTN_ABS of the oracle's
    bound = 2 * ATTN_ABS * math.sqrt(gpu["full"][rows].size)
    for name in ref:
        assert abs(objective_gpu[name] - objective_ref[name]) <= bound, name
    e_rand = [objective_ref[f"random {i}"] for i in range(8)]
    g_rand = [objective_gpu[f"random {i}"] for i in range(8)]
    say("||attn(fused) - attn(full)|| on %d rows, oracle / GPU: deviation top-k %.3f / %.3f, "
        "random %.3f .. %.3f / %.3f .. %.3f, no recompute %.3f / %.3f, top-k without "
        "re-rotation %.3f / %.3f" % (len(rows), objective_ref["top-k"], objective_gpu["top-k"],
                                     min(e_rand), max(e_rand), min(g_rand), max(g_rand),
                                     objective_ref["none"], objective_gpu["none"],
                                     objective_ref["top-k, cache not re-rotated"],
                                     objective_gpu["top-k, cache not re-rotated"]))
    for side in (objective_ref, objective_gpu):
        rand = [side[f"random {i}"] for i in range(8)]
        assert side["top-k"] < 0.5 * min(rand)
        assert side["top-k"] < 0.5 * side["none"]
        assert side["top-k"] < 0.5 * side["top-k, cache not re-rotated"]   # re-rotation matters
    # every token recomputed is full recompute, bit for bit, on the GPU
    assert torch.equal(gpu_fused(np.arange(t)), cases["full"])
