"""The selection objective on the GPU path.

[Derivations, "形式化"] scores a choice S of recomputed tokens by how far the
layer's attention over the fused cache lies from full recompute, and
[Derivations, "近似解"] approximates the best S by the tokens of largest KV
deviation.  Here the whole check runs through the library: keys at their old
and new positions come from cb_rerotate of one base, the selection from
cb_deviation_topk, the fused cache from cb_rerotate + cb_fuse_scatter, and
every row's attention from cb_partial_attn.  The deviation top-k must leave
a much smaller attention error than random selections of the same size, and
re-rotating the reused keys must matter.  Nothing here uses the oracle: the
claim compares GPU results with each other.
"""
import math

import pytest
import torch

from selective_recompute_amd import binding as B
from selective_recompute_amd import pipeline as PL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"\n[objective] {msg}", flush=True)


def _randn(shape, gen):
    return torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)


def test_deviation_selection_beats_random_on_gpu():
    hq, hkv, d, theta = 32, 8, 128, 10000.0
    chunk, n_chunks = 512, 4
    t = chunk * n_chunks
    k_sel = PL.select_count(15, t)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(0xCB0F)
    p_old = torch.arange(chunk, dtype=torch.int32, device=DEV).repeat(n_chunks)
    p_new = torch.arange(t, dtype=torch.int32, device=DEV)
    g_kv = B.geom(hkv, hkv, d, torch.bfloat16)
    g_q = B.geom(hq, hq, d, torch.bfloat16)
    g = B.geom(hq, hkv, d, torch.bfloat16)

    def rotated(base, pos, geom):
        out = torch.empty_like(base)
        B.rerotate(geom, out, base, pos, t, 1, theta)
        return out

    # the same key content at chunk-local (cached) and global (recomputed)
    # positions; recomputed keys and values move a little everywhere and the
    # values a lot on 15% of the tokens
    k_base = _randn((t, hkv, d), gen)
    k_old = rotated(k_base.to(torch.bfloat16), p_old, g_kv)
    k_new = rotated((k_base + 0.01 * _randn((t, hkv, d), gen)).to(torch.bfloat16), p_new, g_kv)
    q = rotated(_randn((t, hq, d), gen).to(torch.bfloat16), p_new, g_q)
    v_old = _randn((t, hkv, d), gen).to(torch.bfloat16)
    hot = torch.randperm(t, generator=gen, device=DEV)[:k_sel]
    sigma = torch.full((t, 1, 1), 0.01, device=DEV)
    sigma[hot] = 1.0
    v_new = (v_old.float() + sigma * _randn((t, hkv, d), gen)).to(torch.bfloat16)
    delta = p_new - p_old
    scale = 1.0 / math.sqrt(d)
    every = torch.arange(t, dtype=torch.int32, device=DEV)
    rb_all = B.RaggedBatch([0, t], [0, t], [0, t], DEV)
    ws = B.workspace_tensor(B.attn_workspace_bytes(g, rb_all))

    def attend_all(keys, vals):
        out = torch.empty((t, hq, d), dtype=torch.bfloat16, device=DEV)
        B.partial_attn(g, rb_all, out, q, every, every, keys, vals, scale, ws)
        return out

    full = attend_all(k_new, v_new)

    def error(sel, rerotate_cache=True):
        sel = torch.sort(sel.to(torch.int32)).values
        keys, vals = k_old.clone(), v_old.clone()
        if rerotate_cache:
            B.rerotate(g_kv, keys, keys, delta, t, 1, theta)
        B.fuse_scatter(g, keys, vals, k_new, v_new, sel, sel, len(sel))
        return float(torch.linalg.vector_norm((attend_all(keys, vals).float() - full.float())))

    # the library's selection: deviation of every token's V, top 15%
    rb = B.RaggedBatch([0, t], [0, t], [0, k_sel], DEV)
    dev = torch.empty(t, dtype=torch.float32, device=DEV)
    sl = torch.empty(k_sel, dtype=torch.int32, device=DEV)
    sg = torch.empty(k_sel, dtype=torch.int32, device=DEV)
    B.deviation_topk(g, rb, v_new, v_old, every, dev, sl, sg)
    torch.cuda.synchronize()
    assert torch.equal(sg, torch.sort(hot.to(torch.int32)).values)

    e_top = error(sg)
    e_rand = [error(torch.randperm(t, generator=gen, device=DEV)[:k_sel]) for _ in range(8)]
    e_stale = error(sg, rerotate_cache=False)
    e_none = error(torch.zeros(0, dtype=torch.int32, device=DEV))
    e_all = error(every)
    torch.cuda.synchronize()
    say(f"||attn(fused) - attn(full)||: deviation top-k {e_top:.3f}, random "
        f"{min(e_rand):.3f} .. {max(e_rand):.3f}, no recompute {e_none:.3f}, "
        f"top-k without re-rotation {e_stale:.3f}, everything recomputed {e_all:.3f}")
    assert e_all == 0.0                          # S = all tokens is full recompute
    assert e_top < 0.5 * min(e_rand)
    assert e_top < 0.5 * e_none
    assert e_top < 0.5 * e_stale                 # the reused keys must be re-rotated
