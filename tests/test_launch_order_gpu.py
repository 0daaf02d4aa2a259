"""The launch order of whole-row attention units does not change results.

A plan whose units are whole rows over several requests launches its query
tiles longest row first, in an order the host estimates from the request
sizes; a single request keeps the default order.  Every unit computes the
same numbers wherever it sits in the launch, so each request's rows of a
batched launch must equal, bit for bit, those of a launch over that request
alone ([Derivations, "形式化"]: each selected row attends over its own
request's keys only).  Cases: the 70B-shaped batch's ragged requests with
rows spread at random, many small requests (some with nothing selected), and
more query tiles than the order table holds (the default order).  The batched
outputs are also checked against the oracle on sampled rows.
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
ATTN_ABS = 2e-2
WHOLE_ROWS = dict(mfma=1, key_split=1, key_chunk=0)


def say(msg):
    print(f"\n[launch-order] {msg}", flush=True)


def _case(name):
    rng = np.random.default_rng(7)
    if name == "70b-8req":
        lens = list(W.make_workload("70b-80layer-8req").request_lengths)
        ks = [(15 * n + 99) // 100 for n in lens]
        return 64, 8, lens, ks
    if name == "40-small":
        lens = [int(x) for x in rng.integers(60, 3000, 40)]
        ks = [0 if r % 7 == 3 else int(rng.integers(1, n // 4 + 2)) for r, n in enumerate(lens)]
        return 32, 8, lens, ks
    if name == "1000-tiles":      # more query tiles than the order table holds
        lens = [64] * 1000
        ks = [8] * 1000
        return 64, 8, lens, ks
    raise KeyError(name)


@pytest.mark.parametrize("name", ["70b-8req", "40-small", "1000-tiles"])
def test_batched_rows_equal_single_request_launches(name):
    hq, hkv, lens, ks = _case(name)
    d = 128
    say(f"{name}: {len(lens)} requests, {sum(lens)} tokens, {sum(ks)} rows")
    rng = np.random.default_rng(11)
    tok_off, sel_off = PL.offsets(lens), PL.offsets(ks)
    sel = np.concatenate([np.sort(rng.choice(n, k, replace=False)) + tok_off[r]
                          for r, (n, k) in enumerate(zip(lens, ks))]).astype(np.int32)
    t_count, n_sel = int(tok_off[-1]), len(sel)
    gen = torch.Generator(device=DEV).manual_seed(5)
    q = torch.randn(n_sel, hq, d, generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn(t_count, hkv, d, generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn(t_count, hkv, d, generator=gen, device=DEV).to(torch.bfloat16)
    geo = B.geom(hq, hkv, d, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    rb = B.RaggedBatch(tok_off, tok_off, sel_off, DEV)
    sl = torch.arange(n_sel, dtype=torch.int32, device=DEV)
    sg = torch.from_numpy(sel).to(DEV)
    out = torch.full((n_sel, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.partial_attn_with_plan(geo, rb, WHOLE_ROWS, out, q, sl, sg, k, v, scale)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a row of the batched launch was not written"

    for r, (n, kr) in enumerate(zip(lens, ks)):
        if kr == 0:
            continue
        lo, s0, s1 = int(tok_off[r]), int(sel_off[r]), int(sel_off[r + 1])
        rb1 = B.RaggedBatch(np.array([0, n]), np.array([0, n]), np.array([0, kr]), DEV)
        out1 = torch.full((kr, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.partial_attn_with_plan(geo, rb1, WHOLE_ROWS, out1, q[s0:s1],
                                 torch.arange(kr, dtype=torch.int32, device=DEV),
                                 sg[s0:s1] - lo, k[lo:lo + n], v[lo:lo + n], scale)
        torch.cuda.synchronize()
        assert torch.equal(out[s0:s1], out1), f"request {r}: batched rows differ from its own launch"

    # the batched rows against the oracle on sampled rows (each request's last)
    pick = np.array([int(sel_off[r + 1]) - 1 for r in range(len(lens)) if ks[r]][:12])
    req = np.searchsorted(tok_off, sel[pick], side="right") - 1
    hi = int(sel[pick].max()) + 1
    kn = k[:hi].float().cpu().numpy()
    vn = v[:hi].float().cpu().numpy()
    ref = O.attention_rows(q.float().cpu().numpy(), pick, sel[pick], tok_off[req], kn, vn,
                           hq, hkv, scale)
    got = out[torch.from_numpy(pick).to(DEV)].float().cpu().numpy()
    err = np.abs(got - ref).max()
    assert err <= ATTN_ABS, f"attention max err {err}"
