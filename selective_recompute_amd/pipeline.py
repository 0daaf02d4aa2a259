"""Host driver of the per-layer blend with gradual filtering.

[KV-blog] = the blog page "rag的kvcache问题", section "渐进式过滤机制":
layer 1 scores every token and keeps a ratio r1; layer 2 recomputes only
those candidates and keeps r2 < r1; later layers keep rolling with the small
pool.  The candidate pool of layer l >= 2 is layer 1's selection ("pool",
default) or the previous layer's ("chain").  Per request the selected count
is ceil(ratio * N / 100) with N the request's token count.

The driver never reads device memory: counts are known on the host, and the
selected rows of one layer stay on the device as the next layer's candidates.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import binding as B


def select_count(percent: int, n_tokens: int) -> int:
    """Smallest integer k with 100 k >= percent * n_tokens."""
    return (percent * n_tokens + 99) // 100


class GradualFilter:
    """Selected counts and candidate sources of each layer (0-based)."""

    def __init__(self, request_lengths: Sequence[int], r1_pct: int, r2_pct: int,
                 schedule: str = "pool"):
        if schedule not in ("pool", "chain"):
            raise ValueError(schedule)
        self.lengths = [int(n) for n in request_lengths]
        self.r1, self.r2, self.schedule = r1_pct, r2_pct, schedule

    def counts(self, layer: int) -> List[int]:
        pct = self.r1 if layer == 0 else self.r2
        return [select_count(pct, n) for n in self.lengths]

    def cand_counts(self, layer: int) -> List[int]:
        if layer == 0:
            return list(self.lengths)
        src = 0 if (self.schedule == "pool" or layer == 1) else layer - 1
        return self.counts(src)

    def cand_source(self, layer: int) -> Optional[int]:
        """Layer whose selection is this layer's candidate list (None = all tokens)."""
        if layer == 0:
            return None
        return 0 if (self.schedule == "pool" or layer == 1) else layer - 1


def offsets(counts: Sequence[int]) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


class BlendRunner:
    """Runs L layers of the blend on one stream with preallocated outputs.

    The layers share one zero-filled workspace (the attention's split partials
    and counters).  in_launch_select=True also reserves the selection's
    arrival counters at its end and passes CB_LAYER_WORKSPACE_ZEROED, so each
    call selects inside the deviation launch; by default the top-k is a launch
    of its own, which measured as fast or faster on every workload."""

    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 request_lengths: Sequence[int], r1_pct: int, r2_pct: int, n_layers: int,
                 rope_theta: float, rope_style: int = B.ROPE_HALF, schedule: str = "pool",
                 dev_source: str = "v", device="cuda", order: str = "auto",
                 in_launch_select: bool = False):
        self.geom = B.geom(n_q_heads, n_kv_heads, head_dim, dtype)
        self.dev_source = B.DEV_SOURCES[dev_source]
        self.order = B.ORDERS[order]
        self.flags = B.CB_LAYER_WORKSPACE_ZEROED if in_launch_select else 0
        self.filter = GradualFilter(request_lengths, r1_pct, r2_pct, schedule)
        self.n_layers, self.theta, self.style = n_layers, rope_theta, rope_style
        self.scale = 1.0 / math.sqrt(head_dim)
        self.dtype, self.device = dtype, device
        self.n_q_heads, self.head_dim = n_q_heads, head_dim
        tok_off = offsets(request_lengths)
        t_count = int(tok_off[-1])
        self.all_tokens = torch.arange(t_count, dtype=torch.int32, device=device)
        self.batches, self.outs = [], []
        for layer in range(n_layers):
            cand_off = offsets(self.filter.cand_counts(layer))
            sel_off = offsets(self.filter.counts(layer))
            rb = B.RaggedBatch(tok_off, cand_off, sel_off, device)
            m, k = rb.n_cand, rb.n_sel
            self.batches.append(rb)
            self.outs.append(dict(
                dev=torch.empty(m, dtype=torch.float32, device=device),
                sel_local=torch.empty(k, dtype=torch.int32, device=device),
                sel_global=torch.empty(k, dtype=torch.int32, device=device),
                out=torch.empty((k, n_q_heads, head_dim), dtype=dtype, device=device)))
        # one workspace, sized for the largest layer's attention plus the
        # selection counters, zero-filled once and shared in stream order
        ws = max(B.attn_workspace_bytes(self.geom, rb) for rb in self.batches)
        if in_launch_select:
            ws += B.CB_SELECT_COUNTER_BYTES + 256
        self.workspace = B.workspace_tensor(ws, device)

    def candidates(self, layer: int) -> torch.Tensor:
        src = self.filter.cand_source(layer)
        return self.all_tokens if src is None else self.outs[src]["sel_global"]

    def run_layer(self, layer: int, x: dict, stream=None):
        """One layer on inputs x (k_old/v_old are fused in place)."""
        o = self.outs[layer]
        B.blend_layer(self.geom, self.batches[layer], k=x["k_old"], v=x["v_old"],
                      k_new_c=x["k_new_c"], v_new_c=x["v_new_c"], q_c=x["q_c"],
                      delta=x["delta"], cand_idx=self.candidates(layer),
                      rope_theta=self.theta, rope_style=self.style,
                      softmax_scale=self.scale, dev=o["dev"], sel_local=o["sel_local"],
                      sel_global=o["sel_global"], out=o["out"], workspace=self.workspace,
                      dev_source=self.dev_source, order=self.order, flags=self.flags,
                      stream=stream)
        return o

    def run(self, layers_inputs: Sequence[dict], stream=None):
        for layer, x in enumerate(layers_inputs):
            self.run_layer(layer, x, stream)
        return self.outs
