"""Seeded synthetic inputs for the KV-fusion step (shared by tests and bench).

This module holds none of the method's arithmetic: no rotation, no deviation,
no ranking, no attention.  It draws Gaussian tensors, plants which tokens are
"hot" (high KV deviation), "warm" or "cold", adds tier-scaled noise to make
the recomputed V rows, and casts to the storage dtype.  Both the HIP path and
the CPU oracle consume the exact bytes it produces.

Structure of the pages the inputs mimic:

* [KV-blog] = the blog page "rag的kvcache问题": section "核心发现" (about 15% of
  tokens change a lot when the chunk sees its prefix, the rest barely move),
  section "跨层相关性" (a token that deviates strongly at one layer tends to do
  so at the next) and section "渐进式过滤机制" (ratio r1 over all tokens at
  layer 1, then r2 < r1 among the surviving candidates).

Recipe (per layer l, per request of N tokens):

* K_old, V_old ~ N(0, 1) for every token.  A RoPE rotation maps an isotropic
  Gaussian pair to an isotropic Gaussian pair, so N(0,1) cached keys have the
  distribution of keys rotated at their chunk-local positions.
* Recomputed rows exist only for the layer's candidates C_l (all tokens at
  layer 1; layer 1's planted selection afterwards, or the previous layer's in
  the "chain" schedule).  K_new_c and Q_c ~ N(0,1) (Q for every query head).
  V_new_c[j] = V_old[C_l[j]] + sigma * N(0,1) with sigma = 1 on the hot set,
  0.1 on the warm set and 0.01 on cold tokens.
* Hot set: ceil(hkvd% * N) tokens at layer 1; at each later layer a fraction
  ``persistence`` of the previous hot set is kept and the rest is refilled
  from layer 1's candidate pool.
* Warm set: wherever the layer's selected count k_l exceeds the number of hot
  candidates, k_l - |hot & C_l| cold candidates are promoted to the warm tier,
  so every selection boundary sits between two tiers whose deviations differ
  by about two orders of magnitude.  This is what makes the top-k index set
  unique beyond fp rounding.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np
import torch

SIGMA_HOT = 1.0
SIGMA_WARM = 0.1
SIGMA_COLD = 0.01

_TID = {"k_old": 1, "v_old": 2, "k_new": 3, "v_noise": 4, "q": 5, "k_noise": 6}


@dataclass(frozen=True)
class Workload:
    """One synthetic blend workload: request/chunk layout, model geometry and policy."""
    name: str
    n_layers: int
    chunks: Tuple[Tuple[int, ...], ...]     # per request, its chunk lengths
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    dtype: str                              # "f32" or "bf16"
    hkvd_pct: int                           # planted hot share of each request
    r1_pct: int                             # layer-1 selection ratio
    r2_pct: int                             # later-layer selection ratio
    persistence_pct: int                    # hot tokens kept from layer to layer
    seed: int
    description: str = ""

    @property
    def n_requests(self) -> int:
        return len(self.chunks)

    @property
    def request_lengths(self) -> List[int]:
        return [sum(c) for c in self.chunks]

    @property
    def n_tokens(self) -> int:
        return sum(self.request_lengths)

    @property
    def tok_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.request_lengths)]).astype(np.int64)

    def delta(self) -> np.ndarray:
        """p_new - p_old per packed token: the start of its chunk inside its request."""
        out = []
        for chunk_lens in self.chunks:
            start = 0
            for n in chunk_lens:
                out.append(np.full(n, start, dtype=np.int64))
                start += n
        return np.concatenate(out)

    def positions(self) -> np.ndarray:
        """p_new per packed token (request-local position)."""
        return np.concatenate([np.arange(n, dtype=np.int64) for n in self.request_lengths])

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def _count(pct: int, n: int) -> int:
    # smallest integer >= pct * n / 100
    return (pct * n + 99) // 100


def _draw_batched_chunks(seed: int, n_req=8, min_chunks=2, max_chunks=16,
                         min_len=256, max_len=4096, lo=57344, hi=73728):
    """First seeded draw of per-request chunk lengths whose total is ~64k."""
    rng = np.random.default_rng(seed)
    while True:
        counts = rng.integers(min_chunks, max_chunks + 1, size=n_req)
        lens = [tuple(int(x) for x in rng.integers(min_len, max_len + 1, size=c)) for c in counts]
        total = sum(sum(c) for c in lens)
        if lo <= total <= hi:
            return tuple(lens)


def make_workload(name: str) -> Workload:
    """The five synthetic workloads, by name (see WORKLOADS)."""
    if name == "tiny":
        return Workload("tiny", 1, ((64, 64),), 4, 2, 16, 10000.0, "f32", 15, 15, 15, 80, 0xCB00,
                        "tiny blend: 1 layer, 2x64 tokens, 4 Q / 2 KV heads, head_dim 16, fp32")
    if name == "mistral7b-layer":
        return Workload("mistral7b-layer", 1, ((512,) * 4,), 32, 8, 128, 10000.0, "bf16", 15, 15, 15, 80, 0xCB01,
                        "Mistral-7B-shaped layer: 4x512 tokens, 32 Q / 8 KV heads, head_dim 128, bf16")
    if name == "7b-32layer-6k":
        return Workload("7b-32layer-6k", 32, ((1024,) * 6,), 32, 8, 128, 10000.0, "bf16", 15, 30, 15, 80, 0xCB02,
                        "32-layer gradual filter at 7B shape: 6x1024 tokens, r1 30% -> r2 15%")
    if name == "7b-32layer-32k":
        return Workload("7b-32layer-32k", 32, ((2048,) * 16,), 32, 8, 128, 10000.0, "bf16", 10, 20, 10, 80, 0xCB03,
                        "long-context blend: 16x2048 tokens, 32 layers, r1 20% -> r2 10%")
    if name == "70b-80layer-8req":
        chunks = _draw_batched_chunks(0xCB04)
        return Workload("70b-80layer-8req", 80, chunks, 64, 8, 128, 10000.0, "bf16", 15, 25, 15, 80, 0xCB04,
                        "batched 70B-layer blend: 8 ragged requests of 2-16 chunks, ~64k tokens, 80 layers")
    raise KeyError(name)


WORKLOADS = ("tiny", "mistral7b-layer", "7b-32layer-6k", "7b-32layer-32k", "70b-80layer-8req")


@dataclass
class LayerSets:
    """Planted index structure of one layer (all indices are packed/global rows)."""
    cand_idx: np.ndarray          # [M] ascending within each request
    cand_off: np.ndarray          # [B+1]
    hot: np.ndarray               # bool [T]
    warm: np.ndarray              # bool [T]
    planted: np.ndarray           # [sum k] ascending within each request
    planted_off: np.ndarray       # [B+1]


class PlantedSets:
    """Per-layer hot/warm sets and candidate lists of a workload, from its seed."""

    def __init__(self, wl: Workload, schedule: str = "pool"):
        if schedule not in ("pool", "chain"):
            raise ValueError(schedule)
        self.wl, self.schedule = wl, schedule
        self._layers: List[LayerSets] = []
        self._hot_local: List[List[np.ndarray]] = []   # per layer, per request (local idx)
        self._sel_local: List[List[np.ndarray]] = []

    def layer(self, layer: int) -> LayerSets:
        """Sets of layer ``layer`` (0-based)."""
        while len(self._layers) <= layer:
            self._build(len(self._layers))
        return self._layers[layer]

    def _build(self, layer: int):
        wl = self.wl
        tok_off = wl.tok_off
        t_count = wl.n_tokens
        hot = np.zeros(t_count, bool)
        warm = np.zeros(t_count, bool)
        cands, planted, hot_loc, sel_loc = [], [], [], []
        for r, n in enumerate(wl.request_lengths):
            rng = np.random.default_rng([wl.seed, 7, layer, r])
            n_hot = _count(wl.hkvd_pct, n)
            if layer == 0:
                cand = np.arange(n)
                h = rng.choice(n, n_hot, replace=False)
                k = _count(wl.r1_pct, n)
            else:
                first = self._sel_local[0][r]
                prev_hot = self._hot_local[layer - 1][r]
                cand = first if (self.schedule == "pool" or layer == 1) else self._sel_local[layer - 1][r]
                keep = int(np.floor(wl.persistence_pct * len(prev_hot) / 100.0 + 0.5))
                kept = rng.choice(prev_hot, keep, replace=False)
                pool = np.setdiff1d(first, prev_hot)
                refill = rng.choice(pool, min(n_hot - keep, len(pool)), replace=False)
                h = np.concatenate([kept, refill])
                k = _count(wl.r2_pct, n)
            cand = np.sort(cand)
            hot_in_cand = np.intersect1d(h, cand)
            if len(hot_in_cand) > k:
                raise ValueError("planted hot set larger than the selection: no tier gap")
            rest = np.setdiff1d(cand, hot_in_cand)
            w = rng.choice(rest, k - len(hot_in_cand), replace=False)
            sel = np.sort(np.concatenate([hot_in_cand, w]))
            hot[tok_off[r] + h] = True
            warm[tok_off[r] + w] = True
            cands.append(cand + tok_off[r])
            planted.append(sel + tok_off[r])
            hot_loc.append(np.sort(h))
            sel_loc.append(sel)
        self._hot_local.append(hot_loc)
        self._sel_local.append(sel_loc)
        cand_off = np.concatenate([[0], np.cumsum([len(c) for c in cands])])
        planted_off = np.concatenate([[0], np.cumsum([len(p) for p in planted])])
        self._layers.append(LayerSets(np.concatenate(cands), cand_off, hot, warm,
                                      np.concatenate(planted), planted_off))


def _seed(wl: Workload, layer: int, tensor: str, draw: int) -> int:
    return int(np.random.SeedSequence([wl.seed, layer, _TID[tensor], draw]).generate_state(1)[0])


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def layer_inputs(wl: Workload, sets: PlantedSets, layer: int, device="cpu", draw: int = 0,
                 k_new: str = "independent") -> dict:
    """Tensors of one layer on ``device``: cached K/V, recomputed candidate rows,
    their queries and the index arrays.  ``draw`` selects an independent copy
    with the same planted structure.

    k_new "independent": K_new_c ~ N(0,1).  k_new "tied": K_new_c[j] =
    K_old[C[j]] + sigma * N(0,1) with the same tiers as V, i.e. the recomputed
    key sits next to the cached one: meant for caches whose keys already are
    at their new positions (no re-rotation), where a key-based deviation then
    has the same planted gap as the V one."""
    s = sets.layer(layer)
    t_count, m = wl.n_tokens, len(s.cand_idx)
    hkv, hq, d = wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    dt = wl.torch_dtype
    k_old = _randn((t_count, hkv, d), _seed(wl, layer, "k_old", draw), device).to(dt)
    v_old = _randn((t_count, hkv, d), _seed(wl, layer, "v_old", draw), device).to(dt)
    sigma = np.full(t_count, SIGMA_COLD, np.float32)
    sigma[s.warm] = SIGMA_WARM
    sigma[s.hot] = SIGMA_HOT
    cand_t = torch.from_numpy(s.cand_idx.astype(np.int64)).to(device)
    sig_c = torch.from_numpy(sigma[s.cand_idx]).to(device)[:, None, None]
    noise = _randn((m, hkv, d), _seed(wl, layer, "v_noise", draw), device)
    v_new_c = (v_old.index_select(0, cand_t).float() + sig_c * noise).to(dt)
    del noise
    if k_new == "independent":
        k_new_c = _randn((m, hkv, d), _seed(wl, layer, "k_new", draw), device).to(dt)
    elif k_new == "tied":
        noise = _randn((m, hkv, d), _seed(wl, layer, "k_noise", draw), device)
        k_new_c = (k_old.index_select(0, cand_t).float() + sig_c * noise).to(dt)
        del noise
    else:
        raise ValueError(k_new)
    q_c = _randn((m, hq, d), _seed(wl, layer, "q", draw), device).to(dt)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return dict(
        k_old=k_old, v_old=v_old, k_new_c=k_new_c, v_new_c=v_new_c, q_c=q_c,
        cand_idx=i32(s.cand_idx), cand_off=i32(s.cand_off), tok_off=i32(wl.tok_off),
        delta=i32(wl.delta()),
        h_cand_off=s.cand_off.astype(np.int64), h_tok_off=wl.tok_off.astype(np.int64),
        planted=s.planted.astype(np.int64), planted_off=s.planted_off.astype(np.int64),
    )
