"""Attention parity on long rows, with inputs whose outputs are O(1).

[Derivations, "形式化"]: the selected rows attend with Attention(Q, K_fused,
V_fused); [KV-blog, "transformer训练与推理并行计算的差异"]: causal mask.

Rows of 32k (the long-context blend), of the 70B-shaped batch's ragged
requests (4k-20k tokens) and of 128k keys, with the needle and peaked input
families of tests/needles.py, so that a lost key chunk, tile or diagonal
fails the 2e-2 bar (tests/test_attention_power.py shows that on the CPU).
Every case runs through cb_partial_attn with the planner's choice and through
every pinned decomposition that fits the rows (plain kernel, key split 1 / 2,
unsplit and over 2, 4 and 8 key chunks), each compared with the oracle on the
same sampled rows (each request's first and last selected row among them).
"""
import math

import numpy as np
import pytest
import torch

import needles as N
from oracle import cacheblend_oracle as O
from selective_recompute_amd import binding as B
from selective_recompute_amd import pipeline as PL
from selective_recompute_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _pct(p, n):
    return (p * n + 99) // 100


C4_LENS = W.make_workload("70b-80layer-8req").request_lengths
LONG_CASES = {
    # name: (hq, hkv, d, request lengths, selected per request, sampled rows)
    "32k-r10": (32, 8, 128, [32768], [3277], 12),
    "32k-r20": (32, 8, 128, [32768], [6554], 12),
    "70b-8req-r25": (64, 8, 128, C4_LENS, [_pct(25, n) for n in C4_LENS], 8),
    "70b-8req-r15": (64, 8, 128, C4_LENS, [_pct(15, n) for n in C4_LENS], 8),
    "128k-r1": (32, 8, 128, [131072], [1311], 6),
}


def _plans(lens, ks_list=(1, 2)):
    """Pinned plans that fit these requests: the plain kernel, and per key
    split unsplit and over 2, 4 and 8 key chunks of the longest request."""
    max_n = max(lens)
    plans = [dict(mfma=0)]
    for ks in ks_list:
        plans.append(dict(mfma=1, key_split=ks, key_chunk=0))
        for c in (2, 4, 8):
            kc = -(-max_n // c)
            kc = -(-kc // (64 * ks)) * (64 * ks)
            if kc < max_n:
                plans.append(dict(mfma=1, key_split=ks, key_chunk=kc))
    # the balanced decomposition: a span per CU, and coarse spans (fewer
    # cuts, so longer rows end in different spans' pieces)
    plans += [dict(mfma=1, key_split=1, stream_spans=32), dict(mfma=1, key_split=1, stream_spans=5)]
    return plans


def _selection(lens, ks, rng):
    tok_off = PL.offsets(lens)
    sel = []
    for r, (n, k) in enumerate(zip(lens, ks)):
        rows = np.sort(rng.choice(n, k, replace=False))
        if k and rows[-1] != n - 1:
            rows[-1] = n - 1                      # the longest row of the request
            rows = np.unique(rows)
            while len(rows) < k:
                rows = np.unique(np.concatenate([rows, rng.choice(n, 1)]))
        sel.append(rows + tok_off[r])
    return np.concatenate(sel).astype(np.int32)


def _sample_rows(sel_off, n_sel, n_rows, rng):
    ends = np.concatenate([[sel_off[r], sel_off[r + 1] - 1] for r in range(len(sel_off) - 1)
                           if sel_off[r + 1] > sel_off[r]])
    return np.unique(np.concatenate([ends, rng.choice(n_sel, min(n_sel, n_rows), replace=False)]))


def _run(g, rb, plan, q, sel, kf, vf, scale, hkv):
    """Output of cb_partial_attn (plan None) or cb_partial_attn_with_plan."""
    out = torch.full((rb.n_sel, q.shape[1], q.shape[2]), float("nan"), dtype=q.dtype, device=DEV)
    args = (out, q, sel, sel, kf, vf, scale)
    if plan is None:
        ws = B.workspace_tensor(B.attn_workspace_bytes(g, rb), DEV)
        if ws is not None:
            ws.fill_(0xFF)
        B.partial_attn(g, rb, *args, workspace=ws)
        used = B.attn_plan(g, rb, 0 if ws is None else ws.numel())
    else:
        used = B.describe_plan(g, rb, **plan)
        ws = B.workspace_tensor(used["workspace_bytes"], DEV)
        if ws is not None:
            ws.fill_(0xFF)
        B.partial_attn_with_plan(g, rb, plan, *args, workspace=ws)
    torch.cuda.synchronize()
    if used["key_chunk"]:
        n = used["tiles"] * hkv
        end = used["workspace_bytes"]
        assert not ws[end - 4 * n:end].view(torch.int32).any(), "arrival counters left non-zero"
    return np64(out), used


@pytest.mark.parametrize("family", ["needle", "peaked"])
@pytest.mark.parametrize("name", list(LONG_CASES))
def test_long_rows_every_plan(name, family):
    hq, hkv, d, lens, ks, n_rows = LONG_CASES[name]
    seed = sum(lens) + sum(ks) + len(family)
    rng = np.random.default_rng(seed)
    tok_off, sel_off = PL.offsets(lens), PL.offsets(ks)
    t_count = int(tok_off[-1])
    sel = _selection(lens, ks, rng)
    gen = torch.Generator().manual_seed(seed)
    # candidates = every token (q has one row per token; sel_local = sel_global)
    q = torch.randn(t_count, hq, d, generator=gen).to(torch.bfloat16)
    kf = torch.randn(t_count, hkv, d, generator=gen).to(torch.bfloat16)
    vf = torch.randn(t_count, hkv, d, generator=gen).to(torch.bfloat16)
    if family == "needle":
        q, kf, vf = N.plant_in_cache(q, kf, vf, N.needle_rows(sel, tok_off, sel_off), seed)
    else:
        q = N.peak_queries(q)
    rows = _sample_rows(sel_off, len(sel), n_rows, rng)
    row_start = np.repeat(tok_off[:-1], np.diff(sel_off))
    scale = 1.0 / math.sqrt(d)
    say(f"long rows {name} {family}: oracle on {len(rows)} rows")
    q_rows = np64(q[torch.from_numpy(sel[rows].astype(np.int64))])   # the sampled queries only
    ref = O.attention_rows(q_rows, np.arange(len(rows)), sel[rows], row_start[rows], np64(kf),
                           np64(vf), hq, hkv, scale)
    assert np.abs(ref).max() > 0.2                      # O(1) outputs: the bar has power
    g = B.geom(hq, hkv, d, torch.bfloat16)
    rb = B.RaggedBatch(tok_off, tok_off, sel_off, DEV)
    qd, sd, kd, vd = q.to(DEV), torch.from_numpy(sel).to(DEV), kf.to(DEV), vf.to(DEV)
    for plan in [None] + _plans(lens):
        say(f"long rows {name} {family}: plan {plan or 'chosen'}")
        got, used = _run(g, rb, plan, qd, sd, kd, vd, scale, hkv)
        assert np.isfinite(got).all()
        err = N.attention_error(got[rows], ref)
        assert err <= N.ATTN_ABS, f"plan {plan or used}: max err {err}"


DENSE_LONG = {
    # layer-1 full prefill: every row of every request selected
    "32k": (32, 8, 128, [32768], 12),
    "70b-8req": (64, 8, 128, C4_LENS, 8),
}


@pytest.mark.parametrize("family", ["needle", "peaked"])
@pytest.mark.parametrize("name", list(DENSE_LONG))
def test_dense_prefill_full_length(name, family):
    """[KV-blog, "渐进式过滤机制"]: layer 1 computes every token.  Dense causal
    attention of every row at 32k tokens and at the 70B-shaped batch's ragged
    lengths, through the planner's choice and key split 2 unsplit."""
    hq, hkv, d, lens, n_rows = DENSE_LONG[name]
    seed = 99 + sum(lens) + len(family)
    rng = np.random.default_rng(seed)
    tok_off = PL.offsets(lens)
    t_count = int(tok_off[-1])
    sel = np.arange(t_count, dtype=np.int32)
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(t_count, hq, d, generator=gen).to(torch.bfloat16)
    kf = torch.randn(t_count, hkv, d, generator=gen).to(torch.bfloat16)
    vf = torch.randn(t_count, hkv, d, generator=gen).to(torch.bfloat16)
    if family == "needle":
        q, kf, vf = N.plant_in_cache(q, kf, vf, N.needle_rows(sel, tok_off, tok_off), seed)
    else:
        q = N.peak_queries(q)
    rows = _sample_rows(tok_off, t_count, n_rows, rng)
    row_start = np.repeat(tok_off[:-1], lens)
    scale = 1.0 / math.sqrt(d)
    say(f"dense prefill {name} {family}: oracle on {len(rows)} rows")
    q_rows = np64(q[torch.from_numpy(sel[rows].astype(np.int64))])   # the sampled queries only
    ref = O.attention_rows(q_rows, np.arange(len(rows)), sel[rows], row_start[rows], np64(kf),
                           np64(vf), hq, hkv, scale)
    g = B.geom(hq, hkv, d, torch.bfloat16)
    rb = B.RaggedBatch(tok_off, tok_off, tok_off, DEV)
    qd, sd, kd, vd = q.to(DEV), torch.from_numpy(sel).to(DEV), kf.to(DEV), vf.to(DEV)
    for plan in (None, dict(mfma=1, key_split=2, key_chunk=0)):
        say(f"dense prefill {name} {family}: plan {plan or 'chosen'}")
        got, used = _run(g, rb, plan, qd, sd, kd, vd, scale, hkv)
        assert np.isfinite(got).all()
        err = N.attention_error(got[rows], ref)
        assert err <= N.ATTN_ABS, f"plan {plan or used}: max err {err}"
