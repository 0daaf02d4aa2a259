"""The top-k inside the deviation launch (cb_blend_layer with
CB_LAYER_WORKSPACE_ZEROED) against the top-k in its own launch.

[Derivations, "近似解"]: the k candidates of largest deviation, ties to the
lower row.  Both paths run the same selection code; here every output of a
layer -- deviations, selections, fused K/V, attention -- must be equal bit
for bit between them, in both step orders, on the workloads' layers and on a
ragged batch of many small requests (several requests per scoring workgroup,
requests with nothing to select, everything to select, ties at zero).  The
selection counters must be zero after every call, and a second call on the
same workspace must give the same results.  The top-k in its own launch is
itself checked against the oracle in tests/test_parity_gpu.py; the many-
request case also checks the selections against the oracle here.
"""
import math

import numpy as np
import pytest
import torch

from oracle import cacheblend_oracle as O
from selective_recompute_amd import binding as B
from selective_recompute_amd import pipeline as PL
from selective_recompute_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(f"\n[select-in-launch] {msg}", flush=True)


def _run(g, rb, x, cand_idx, theta, scale, order, ws, flags):
    dev = torch.full((rb.n_cand,), float("nan"), dtype=torch.float32, device=DEV)
    sl = torch.full((rb.n_sel,), -1, dtype=torch.int32, device=DEV)
    sg = torch.full((rb.n_sel,), -1, dtype=torch.int32, device=DEV)
    out = torch.full((rb.n_sel, g.n_q_heads, g.head_dim), float("nan"),
                     dtype=x["k_old"].dtype, device=DEV)
    k, v = x["k_old"].clone(), x["v_old"].clone()
    B.blend_layer(g, rb, k=k, v=v, k_new_c=x["k_new_c"], v_new_c=x["v_new_c"], q_c=x["q_c"],
                  delta=x["delta"], cand_idx=cand_idx, rope_theta=theta,
                  rope_style=B.ROPE_HALF, softmax_scale=scale, dev=dev, sel_local=sl,
                  sel_global=sg, out=out, workspace=ws, order=order, flags=flags)
    torch.cuda.synchronize()
    return [t.cpu() for t in (dev, sl, sg, k, v, out)]


def _counters_zero(ws):
    """The selection counters (the workspace's last CB_SELECT_COUNTER_BYTES,
    256-byte aligned) are all zero."""
    n = ws.numel()
    off = (n - B.CB_SELECT_COUNTER_BYTES) & ~255
    return not ws[off:off + B.CB_SELECT_COUNTER_BYTES].any().item()


def _compare(g, rb, x, cand_idx, theta, scale, order):
    """Own-launch top-k on a workspace of A bytes against the in-launch one on
    A + CB_SELECT_COUNTER_BYTES + 256 (the attention sees A bytes either way,
    so both choose the same plan); the in-launch path twice on its workspace."""
    attn = B.attn_workspace_bytes(g, rb)
    ws_a = B.workspace_tensor(max(attn, 256), DEV)
    ws_b = B.workspace_tensor(max(attn, 256) + B.CB_SELECT_COUNTER_BYTES + 256, DEV)
    ref = _run(g, rb, x, cand_idx, theta, scale, order, ws_a, 0)
    for call in range(2):
        got = _run(g, rb, x, cand_idx, theta, scale, order, ws_b, B.CB_LAYER_WORKSPACE_ZEROED)
        for name, a, b in zip(("dev", "sel_local", "sel_global", "k", "v", "out"), ref, got):
            assert torch.equal(a, b), f"call {call}: {name} differs"
        assert _counters_zero(ws_b), f"call {call}: selection counters left non-zero"
    return ref


@pytest.mark.parametrize("order", [B.CB_ORDER_ROTATE_FIRST, B.CB_ORDER_SELECT_FIRST])
@pytest.mark.parametrize("name,layer", [("tiny", 0), ("mistral7b-layer", 0),
                                        ("7b-32layer-6k", 0), ("7b-32layer-6k", 1),
                                        ("7b-32layer-32k", 1), ("70b-80layer-8req", 0),
                                        ("70b-80layer-8req", 1)])
def test_select_in_launch_is_bit_identical(name, layer, order):
    say(f"{name} layer {layer} order {order}")
    wl = W.make_workload(name)
    sets = W.PlantedSets(wl)
    counts = PL.GradualFilter(wl.request_lengths, wl.r1_pct, wl.r2_pct).counts(layer)
    gen = "cpu" if wl.n_tokens <= 8192 else DEV
    x = {k: (v.to(DEV) if torch.is_tensor(v) else v)
         for k, v in W.layer_inputs(wl, sets, layer, device=gen).items()}
    g = B.geom(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.torch_dtype)
    rb = B.RaggedBatch(x["h_tok_off"], x["h_cand_off"], PL.offsets(counts), DEV)
    ref = _compare(g, rb, x, x["cand_idx"], wl.rope_theta, 1.0 / math.sqrt(wl.head_dim), order)
    assert np.array_equal(ref[2].numpy().astype(np.int64), x["planted"])


def _many_requests(seed, n_req=70, hq=8, hkv=2, d=64):
    """A ragged batch of n_req small requests: 1..40 tokens each, every token
    a candidate, k from 0 to all; a third of the requests have V rows equal
    to the cache on most tokens (ties at exactly zero)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 41, n_req)
    ks = [int(rng.integers(0, n + 1)) if i % 5 else (0 if i % 10 == 0 else int(n))
          for i, n in enumerate(lens)]
    tok_off = PL.offsets(lens)
    t = int(tok_off[-1])
    gen = torch.Generator().manual_seed(seed)
    mk = lambda h: torch.randn(t, h, d, generator=gen).to(torch.bfloat16)
    k_old, v_old, k_new, q = mk(hkv), mk(hkv), mk(hkv), mk(hq)
    v_new = v_old.clone()
    change = torch.rand(t, generator=gen) < 0.4
    for r in range(n_req):
        if r % 3 == 0:      # mostly ties at zero
            change[tok_off[r]:tok_off[r + 1]] = torch.rand(int(lens[r]), generator=gen) < 0.1
    v_new[change] = mk(hkv)[change]
    delta = np.concatenate([np.full(n, (n // 2) * (r % 2)) for r, n in enumerate(lens)])
    x = dict(k_old=k_old.to(DEV), v_old=v_old.to(DEV), k_new_c=k_new.to(DEV),
             v_new_c=v_new.to(DEV), q_c=q.to(DEV),
             delta=torch.from_numpy(delta.astype(np.int32)).to(DEV))
    return lens, ks, tok_off, x


@pytest.mark.parametrize("order", [B.CB_ORDER_ROTATE_FIRST, B.CB_ORDER_SELECT_FIRST])
@pytest.mark.parametrize("seed", [3, 4])
def test_select_in_launch_many_small_requests(seed, order):
    say(f"70 small requests seed {seed} order {order}")
    lens, ks, tok_off, x = _many_requests(seed)
    hq, hkv, d = x["q_c"].shape[1], x["k_old"].shape[1], x["k_old"].shape[2]
    g = B.geom(hq, hkv, d, torch.bfloat16)
    rb = B.RaggedBatch(tok_off, tok_off, PL.offsets(ks), DEV)
    t = int(tok_off[-1])
    cand = torch.arange(t, dtype=torch.int32, device=DEV)
    ref = _compare(g, rb, x, cand, 10000.0, 1.0 / math.sqrt(d), order)
    # the selections against the oracle's top-k on the GPU's deviations
    dev = ref[0].numpy().astype(np.float64)
    sg = ref[2].numpy().astype(np.int64)
    sel_off = PL.offsets(ks)
    for r in range(len(lens)):
        c0, c1 = int(tok_off[r]), int(tok_off[r + 1])
        _, want = O.topk_select(dev[c0:c1], np.arange(c0, c1), ks[r])
        assert np.array_equal(sg[sel_off[r]:sel_off[r + 1]], want), f"request {r}"
