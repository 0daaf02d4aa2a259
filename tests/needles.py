"""Attention inputs whose outputs stay O(1) at any row length (tests only).

With iid N(0,1) queries and keys and the 1/sqrt(D) scale, the softmax of a
long row is almost flat and the output of a row of n keys shrinks like
sqrt(e/n): at 32k keys and more, an absolute bar of 2e-2 passes even when a
whole block of keys is lost.  Two input families keep the bar meaningful:

* needles -- every query of KV group g gets a large component alpha along a
  unit direction u_g, and a few "needle" rows per request carry the key
  beta * u_g (every KV head) with their own O(1) V row.  A needle's score is
  about 25 above the bulk of the keys, so a query's softmax mass sits on the
  needles it can see, and its output is close to the mean of their V rows.
  Needles are chosen among the selected rows, about evenly spaced, so every
  key chunk of a split (at most 8 per row) holds one, and a selected needle
  row sees itself: losing a chunk, the tile of a needle or the diagonal moves
  the output by O(1 / #needles seen).
* peaked -- the plain Gaussian inputs with the queries scaled up (x6): each
  row's softmax concentrates on a few keys spread over the whole row.

The attention itself is computed only by the oracle and by the library; this
module only shapes inputs.
"""
from __future__ import annotations

import numpy as np
import torch

ATTN_ABS = 2e-2          # attention bar against the oracle's fp64 values
NEEDLES_PER_REQUEST = 16
ALPHA = 16.0             # query component along u_g
BETA = 18.0              # needle key length along u_g
PEAK_Q_SCALE = 6.0


def attention_error(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def attention_close(got: np.ndarray, ref: np.ndarray) -> bool:
    """The parity bar: every output element within ATTN_ABS of the oracle."""
    return bool(np.isfinite(got).all()) and attention_error(got, ref) <= ATTN_ABS


def needle_rows(sel_global: np.ndarray, tok_off: np.ndarray, sel_off: np.ndarray,
                per_request: int = NEEDLES_PER_REQUEST) -> np.ndarray:
    """Packed rows of the needles: in each request, the selected rows nearest
    to `per_request` evenly spaced positions (its first and last selected row
    included)."""
    out = []
    for r in range(len(tok_off) - 1):
        rows = np.asarray(sel_global[sel_off[r]:sel_off[r + 1]], np.int64)
        if len(rows) == 0:
            continue
        lo, hi = int(tok_off[r]), int(tok_off[r + 1])
        targets = np.linspace(lo, hi - 1, per_request)
        idx = np.searchsorted(rows, targets)
        idx = np.clip(idx, 0, len(rows) - 1)
        prev = np.clip(idx - 1, 0, len(rows) - 1)
        pick = np.where(np.abs(rows[prev] - targets) < np.abs(rows[idx] - targets), prev, idx)
        out.append(np.unique(np.concatenate([rows[pick], rows[[0, -1]]])))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def directions(n_kv_heads: int, head_dim: int, seed: int) -> torch.Tensor:
    """One random unit vector per KV head, float32 [Hkv, D]."""
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(n_kv_heads, head_dim, generator=g, dtype=torch.float64)
    return (u / u.norm(dim=1, keepdim=True)).float()


def sharpen_queries(q: torch.Tensor, u: torch.Tensor, alpha: float = ALPHA) -> torch.Tensor:
    """q [rows, Hq, D] (any float dtype): every query head h of group
    g = h // (Hq / Hkv) gets alpha * u_g added; returned in q's dtype."""
    hq, hkv = q.shape[1], u.shape[0]
    grp = hq // hkv
    add = (alpha * u).repeat_interleave(grp, dim=0)          # [Hq, D]
    return (q.float() + add[None, :, :].to(q.device)).to(q.dtype)


def needle_key(u: torch.Tensor, dtype, beta: float = BETA) -> torch.Tensor:
    """The key row [Hkv, D] of a needle: beta * u_g for every KV head."""
    return (beta * u).to(dtype)


def plant_in_cache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rows: np.ndarray,
                   seed: int):
    """Needles in a plain (q, k, v) attention case, all on the CPU: q holds one
    row per query row, k and v one per packed token.  Returns the new
    (q, k, v); V rows of needles get a fresh N(0, 2^2) row of their own."""
    u = directions(k.shape[1], k.shape[2], seed)
    q = sharpen_queries(q, u)
    k, v = k.clone(), v.clone()
    ridx = torch.from_numpy(np.asarray(rows, np.int64))
    k[ridx] = needle_key(u, k.dtype)[None].expand(len(rows), -1, -1)
    g = torch.Generator().manual_seed(seed + 1)
    v[ridx] = (2.0 * torch.randn(len(rows), v.shape[1], v.shape[2], generator=g)).to(v.dtype)
    return q, k, v


def plant_in_blend(x: dict, needle_global: np.ndarray, cand_idx: np.ndarray, seed: int) -> dict:
    """Needles in one layer's blend inputs (tensors of ``layer_inputs``), on
    their device: needle rows must be candidates that the layer selects.
    Their recomputed keys become beta * u_g, their recomputed V rows move
    further from the cached ones (so they stay selected: a larger deviation)
    and every candidate's queries get alpha * u_g.  Returns a new dict."""
    y = dict(x)
    dev = x["q_c"].device
    u = directions(x["k_old"].shape[1], x["k_old"].shape[2], seed)
    local = np.searchsorted(cand_idx, needle_global)
    assert np.array_equal(cand_idx[local], needle_global), "needles must be candidates"
    li = torch.from_numpy(local.astype(np.int64)).to(dev)
    y["q_c"] = sharpen_queries(x["q_c"], u)
    kn = x["k_new_c"].clone()
    kn[li] = needle_key(u, kn.dtype).to(dev)[None].expand(len(local), -1, -1)
    y["k_new_c"] = kn
    g = torch.Generator().manual_seed(seed + 1)
    bump = 2.0 * torch.randn(len(local), kn.shape[1], kn.shape[2], generator=g)
    vn = x["v_new_c"].clone()
    vn[li] = (vn[li].float() + bump.to(dev)).to(vn.dtype)
    y["v_new_c"] = vn
    return y


def peak_queries(q: torch.Tensor, scale: float = PEAK_Q_SCALE) -> torch.Tensor:
    return (q.float() * scale).to(q.dtype)


def drop_keys(k: np.ndarray, v: np.ndarray, sel_global: np.ndarray, row_start: np.ndarray,
              lo: int, hi: int):
    """Inputs with the packed key rows [lo, hi) removed (a lost key chunk):
    returns (k', v', end', start') for the oracle's per-row attention, where a
    row's last visible key index and its request start move down past the
    removed range.  Rows inside the range keep the keys below it only."""
    keep = np.ones(k.shape[0], bool)
    keep[lo:hi] = False
    end = np.asarray(sel_global, np.int64)
    start = np.asarray(row_start, np.int64)
    end2 = np.where(end >= hi, end - (hi - lo), np.minimum(end, lo - 1))
    # a request that starts inside the range starts at its first key past it
    start2 = np.where(start >= hi, start - (hi - lo), np.where(start >= lo, lo, start))
    return k[keep], v[keep], end2, start2
