"""The launch order of attention units does not change results.

Split plans launch their units longest piece first, in an order the host
estimates from the request sizes; unsplit plans keep the kernel's own order
(request by request, last tile first).  Every unit computes the same numbers
wherever it sits in the launch, and a split tile merges its pieces in piece
order whichever arrives last, so each request's rows of a batched launch
must equal, bit for bit, those of a launch over that request alone
([Derivations, "形式化"]: each selected row attends over its own request's
keys only) -- a launch whose units come in another order.  Cases: the
70B-shaped batch's ragged requests with rows spread at random, many small
requests (some with nothing selected), and more units than the order table
holds (the kernel's own order); whole rows, and rows split over key chunks
with either key split.  The batched outputs are also checked against the
oracle on sampled rows.
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


SPLIT_KS1 = dict(mfma=1, key_split=1, key_chunk=512)
SPLIT_KS2 = dict(mfma=1, key_split=2, key_chunk=768)
SPLIT_6K = dict(mfma=1, key_split=1, key_chunk=6144)


def _ws(geo, rb, plan):
    n = B.describe_plan(geo, rb, **plan)["workspace_bytes"]
    return B.workspace_tensor(max(n, 256), DEV)


@pytest.mark.parametrize("name,plan", [("70b-8req", WHOLE_ROWS), ("70b-8req", SPLIT_6K),
                                       ("40-small", WHOLE_ROWS), ("40-small", SPLIT_KS1),
                                       ("40-small", SPLIT_KS2), ("1000-tiles", WHOLE_ROWS)])
def test_batched_rows_equal_single_request_launches(name, plan):
    hq, hkv, lens, ks = _case(name)
    d = 128
    say(f"{name}: {len(lens)} requests, {sum(lens)} tokens, {sum(ks)} rows, plan {plan}")
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
    B.partial_attn_with_plan(geo, rb, plan, out, q, sl, sg, k, v, scale,
                             workspace=_ws(geo, rb, plan))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a row of the batched launch was not written"

    for r, (n, kr) in enumerate(zip(lens, ks)):
        if kr == 0:
            continue
        lo, s0, s1 = int(tok_off[r]), int(sel_off[r]), int(sel_off[r + 1])
        rb1 = B.RaggedBatch(np.array([0, n]), np.array([0, n]), np.array([0, kr]), DEV)
        out1 = torch.full((kr, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.partial_attn_with_plan(geo, rb1, plan, out1, q[s0:s1],
                                 torch.arange(kr, dtype=torch.int32, device=DEV),
                                 sg[s0:s1] - lo, k[lo:lo + n], v[lo:lo + n], scale,
                                 workspace=_ws(geo, rb1, plan))
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


SPLIT_256 = dict(mfma=1, key_split=1, key_chunk=256)


@pytest.mark.parametrize("units", [64, 65, 256, 257, 960, 961])
def test_order_table_sizes(units):
    """The launch order travels in a table sized to the launch (64, 256 or
    960 units; more keep the kernel's own order).  Requests of 512 tokens
    with 8 selected rows are one query tile (64 Q / 8 KV heads: 32 rows per
    tile) in two key chunks of 256, one request of 256 tokens a single
    chunk: units // 2 of the first and units % 2 of the second give each
    table size at its edge and one past it.  Every row is written, and
    sampled requests equal their own launches bit for bit."""
    hq, hkv, d = 64, 8, 128
    lens = [512] * (units // 2) + [256] * (units % 2)
    n_req = len(lens)
    ks = [8] * n_req
    say(f"order table: {units} units over {n_req} requests")
    rng = np.random.default_rng(units)
    tok_off, sel_off = PL.offsets(lens), PL.offsets(ks)
    sel = np.concatenate([np.sort(rng.choice(n, 8, replace=False)) + tok_off[r]
                          for r, n in enumerate(lens)]).astype(np.int32)
    gen = torch.Generator(device=DEV).manual_seed(units)
    q = torch.randn(len(sel), hq, d, generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn(int(tok_off[-1]), hkv, d, generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn(int(tok_off[-1]), hkv, d, generator=gen, device=DEV).to(torch.bfloat16)
    geo = B.geom(hq, hkv, d, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    rb = B.RaggedBatch(tok_off, tok_off, sel_off, DEV)
    assert B.describe_plan(geo, rb, **SPLIT_256)["workgroups"] == units * hkv
    sg = torch.from_numpy(sel).to(DEV)
    out = torch.full((len(sel), hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.partial_attn_with_plan(geo, rb, SPLIT_256, out, q,
                             torch.arange(len(sel), dtype=torch.int32, device=DEV), sg, k, v,
                             scale, workspace=_ws(geo, rb, SPLIT_256))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a row of the batched launch was not written"
    for r in sorted({0, n_req // 2, n_req - 1} | set(range(0, n_req, 97))):
        n, lo, s0 = lens[r], int(tok_off[r]), int(sel_off[r])
        rb1 = B.RaggedBatch(np.array([0, n]), np.array([0, n]), np.array([0, 8]), DEV)
        out1 = torch.full((8, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.partial_attn_with_plan(geo, rb1, SPLIT_256, out1, q[s0:s0 + 8],
                                 torch.arange(8, dtype=torch.int32, device=DEV),
                                 sg[s0:s0 + 8] - lo, k[lo:lo + n], v[lo:lo + n], scale,
                                 workspace=_ws(geo, rb1, SPLIT_256))
        torch.cuda.synchronize()
        assert torch.equal(out[s0:s0 + 8], out1), f"request {r}"
