"""Plain fp64 CPU oracle for the CacheBlend KV-fusion step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, the smoke check in ``__graft_entry__`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library (no
kernels, headers, helpers or tables) and imports nothing from the
``selective_recompute_amd`` package.

Pages this module follows (cited by title and section):

* [Derivations] -- the page "数学推导" (math derivations) of the CacheBlend
  documentation, inference.lei6393.com/cacheblend/appendix/c-math-derivations/
* [KV-blog] -- the blog page "rag的kvcache问题",
  zxj-2023.github.io/2026/06/11/.../rag的kvcache问题/

Every value is computed in float64 from inputs that are exact up-casts of the
stored tensors (fp32 or bf16 widen to fp64 without rounding).  The code is
written for a reader to check against the pages by eye: no blocking, no fusion,
no reordering beyond what each definition states.  Library primitives used as
single steps: numpy's cos/sin, matrix-vector products, exp, lexsort.

Readings taken where the pages are silent or garbled (each restated where it
is used):

* The 2x2 block of [Derivations, "RoPE 位置编码的相对位置不变性证明"] is
  applied to D/2 coordinate pairs with the RoFormer frequency schedule
  ``omega_j = theta ** (-2 j / D)`` (RoFormer is the page's second reference).
  Pairs are ``(j, j + D/2)`` ("half" style, default) or ``(2j, 2j+1)``
  ("interleaved" style).
* The deviation is the squared L2 norm of the V difference over every KV head
  and every head dimension of a token ([Derivations, "近似解"]); the blog's
  absolute-difference form ranks tokens the same way.  The blog's deviation of
  a token's whole KV vector is also offered: on K alone, or on K and V read
  as one vector; cached keys enter it after re-rotation (at the new position).
* Ties in the top-k go to the lower global token index; NaN ranks above +inf.
* Attention is causal inside a request, uses scale ``1/sqrt(D)``, and maps
  query head h to KV head ``h // (Hq // Hkv)``.
* Gradual filtering: layer 1 picks ``ceil(r1 * N / 100)`` of all N tokens;
  every later layer picks ``ceil(r2 * N / 100)`` among layer 1's picks ("pool"
  schedule, default) or among the previous layer's picks ("chain").
"""
from __future__ import annotations

import numpy as np

ROPE_HALF = 0
ROPE_INTERLEAVED = 1


# --------------------------------------------------------------------------
# Re-rotation of cached keys.
# [Derivations, "RoPE 位置编码的相对位置不变性证明"]: a vector at position m is
# rotated by R_m, built from 2x2 blocks [[cos, -sin], [sin, cos]].
# [Derivations, "CacheBlend 中的应用"]: a key cached at p_old is moved to p_new
# by R_{p_new - p_old}, because R_{p_new} R_{p_old}^{-1} = R_{p_new - p_old}.
# --------------------------------------------------------------------------
def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """Angular speed of each coordinate pair (RoFormer schedule), float64 [D/2]."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / head_dim)


def rope_pairs(head_dim: int, style: int):
    """Index arrays (first, second) of the coordinate pairs each block rotates."""
    half = head_dim // 2
    if style == ROPE_HALF:
        return np.arange(half), np.arange(half) + half
    if style == ROPE_INTERLEAVED:
        return np.arange(0, head_dim, 2), np.arange(1, head_dim, 2)
    raise ValueError(f"unknown rope style {style}")


def rotate(x: np.ndarray, pos, theta: float, style: int = ROPE_HALF) -> np.ndarray:
    """Apply R_pos to every head vector of every token.

    x   : float64 [T, H, D]
    pos : [T] rotation position of each token (any real number)
    Each pair (a, b) becomes (a cos t - b sin t, a sin t + b cos t) with
    t = pos * omega_j for pair j.
    """
    x = np.asarray(x, dtype=np.float64)
    t_count, _, head_dim = x.shape
    pos = np.asarray(pos, dtype=np.float64).reshape(t_count)
    omega = rope_frequencies(head_dim, theta)
    angle = pos[:, None] * omega[None, :]               # [T, D/2]
    c = np.cos(angle)[:, None, :]                       # [T, 1, D/2]
    s = np.sin(angle)[:, None, :]
    first, second = rope_pairs(head_dim, style)
    a = x[:, :, first]
    b = x[:, :, second]
    out = np.empty_like(x)
    out[:, :, first] = a * c - b * s
    out[:, :, second] = a * s + b * c
    return out


def rerotate(k_old: np.ndarray, delta, theta: float, style: int = ROPE_HALF) -> np.ndarray:
    """K_rot[t] = R_{delta[t]} K_old[t], with delta = p_new - p_old per token."""
    return rotate(k_old, delta, theta, style)


# --------------------------------------------------------------------------
# KV deviation. [Derivations, "近似解"]: tokens are ranked by
# || V_new[i] - V_old[i] ||_2^2.  [KV-blog, "核心发现： KV 偏差"]: the deviation
# of token j at layer i compares its isolated-chunk KV with its full-prefill KV.
# --------------------------------------------------------------------------
def deviation(v_new_c: np.ndarray, v_old: np.ndarray, cand_idx) -> np.ndarray:
    """dev[j] = sum over heads and dims of (V_new_c[j] - V_old[cand_idx[j]])^2.

    v_new_c : float64 [M, Hkv, D]  recomputed rows of the candidates, in cand order
    v_old   : float64 [T, Hkv, D]  cached rows of every token
    returns float64 [M]
    """
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    m = cand_idx.shape[0]
    diff = np.asarray(v_new_c, np.float64).reshape(m, -1) - \
        np.asarray(v_old, np.float64)[cand_idx].reshape(m, -1)
    return np.sum(diff * diff, axis=1)


# --------------------------------------------------------------------------
# Which part of the token's KV the deviation looks at.  [KV-blog, "核心发现：
# KV 偏差"] measures the distance between a token's whole KV vector as cached
# (its chunk encoded alone) and as it would be with the full prefix;
# [Derivations, "近似解"] scores V alone.  Reading taken for K: the cached key
# is compared after re-rotation, i.e. both keys at the new position; the
# cached key at its old position would differ by the rotation alone.
# --------------------------------------------------------------------------
DEV_SOURCES = ("v", "k", "kv")


def store_as(x, dtype: str) -> np.ndarray:
    """x as a tensor of storage type ``dtype`` keeps it ("f32" or "bf16"):
    rounded to the nearest representable value, ties to even, as float64.
    bf16 keeps 8 significant bits (normal range; the keys here are far from
    its limits): x = m * 2**e with 1/2 <= |m| < 1 becomes rint(m * 2**8) * 2**(e-8)."""
    x = np.asarray(x, np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(x)
        return np.ldexp(np.rint(m * 256.0), e - 8)
    raise ValueError(dtype)


def kv_deviation(source: str, *, k_new_c=None, k_cached=None, v_new_c=None, v_old=None,
                 cand_idx=None) -> np.ndarray:
    """Squared distance between the recomputed and the cached rows of each candidate.

    source "v":  the V rows (the [Derivations] score, same as ``deviation``)
    source "k":  the K rows; k_cached holds the cached keys at the new positions
    source "kv": the token's K row and V row read as one vector (their concatenation)
    """
    if source == "v":
        new_rows, cached_rows = [v_new_c], [v_old]
    elif source == "k":
        new_rows, cached_rows = [k_new_c], [k_cached]
    elif source == "kv":
        new_rows, cached_rows = [k_new_c, v_new_c], [k_cached, v_old]
    else:
        raise ValueError(source)
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    m = cand_idx.shape[0]
    new_vec = np.concatenate([np.asarray(a, np.float64).reshape(m, -1) for a in new_rows], axis=1)
    old_vec = np.concatenate([np.asarray(a, np.float64)[cand_idx].reshape(m, -1)
                              for a in cached_rows], axis=1)
    diff = new_vec - old_vec
    return np.sum(diff * diff, axis=1)


# --------------------------------------------------------------------------
# Greedy selection. [Derivations, "近似解"]: S is the TopK of the deviation.
# Ties go to the lower global index; S is emitted in ascending global order.
# --------------------------------------------------------------------------
def topk_select(dev: np.ndarray, cand_idx, k: int):
    """Return (sel_local, sel_global), both ascending, of the k selected candidates.

    Order of preference: NaN first, then larger deviation, then lower global
    token index.  sel_local indexes the candidate list, sel_global = cand_idx[sel_local].
    """
    dev = np.asarray(dev, dtype=np.float64)
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    if not 0 <= k <= dev.shape[0]:
        raise ValueError("k out of range")
    is_nan = np.isnan(dev)
    value = np.where(is_nan, 0.0, dev)
    # lexsort sorts by the last key first: NaN flag (desc), value (desc), index (asc)
    order = np.lexsort((cand_idx, -value, -is_nan.astype(np.int64)))
    chosen = order[:k]
    chosen = chosen[np.argsort(cand_idx[chosen], kind="stable")]
    return chosen.astype(np.int64), cand_idx[chosen]


# --------------------------------------------------------------------------
# Fusion. [Derivations, "形式化"]: K_fused[i] is K_new[i] for i in S and the
# cached row otherwise; V_fused likewise.  [KV-blog, "渐进式过滤机制"]: the
# recomputed rows are spliced into the reused cache before attention.
# --------------------------------------------------------------------------
def fuse(k_rot, v_old, k_new_c, v_new_c, sel_local, sel_global):
    """Return (K_fused, V_fused) as new float64 arrays [T, Hkv, D]."""
    k_fused = np.array(k_rot, dtype=np.float64, copy=True)
    v_fused = np.array(v_old, dtype=np.float64, copy=True)
    sel_local = np.asarray(sel_local, dtype=np.int64)
    sel_global = np.asarray(sel_global, dtype=np.int64)
    k_fused[sel_global] = np.asarray(k_new_c, np.float64)[sel_local]
    v_fused[sel_global] = np.asarray(v_new_c, np.float64)[sel_local]
    return k_fused, v_fused


# --------------------------------------------------------------------------
# Attention of the selected rows over the fused cache.
# [Derivations, "形式化"]: the objective compares Attention(Q, K_fused, V_fused)
# with full recompute.  [KV-blog, "渐进式过滤机制"]: the selected rows run the
# layer's attention over the spliced cache.  [KV-blog, "阶段二：注意力分数计算阶段"]:
# each query row is independent of the others.  [KV-blog, "transformer训练与推理
# 并行计算的差异"]: the causal mask hides every later position.
# --------------------------------------------------------------------------
def attention_rows(q_c, sel_local, sel_global, row_start, k_fused, v_fused,
                   n_q_heads: int, n_kv_heads: int, scale: float) -> np.ndarray:
    """O[s, h] = softmax over keys u in [row_start[s], sel_global[s]] of
    <Q_c[sel_local[s], h], K_fused[u, g]> * scale, applied to V_fused[u, g],
    with g = h // (n_q_heads // n_kv_heads).

    q_c: float64 [M, Hq, D]; k_fused, v_fused: float64 [T, Hkv, D].
    row_start[s]: first packed row of the request that row s belongs to.
    returns float64 [k, Hq, D]
    """
    q_c = np.asarray(q_c, np.float64)
    k_fused = np.asarray(k_fused, np.float64)
    v_fused = np.asarray(v_fused, np.float64)
    group = n_q_heads // n_kv_heads
    n_sel = len(sel_global)
    head_dim = q_c.shape[2]
    out = np.zeros((n_sel, n_q_heads, head_dim), dtype=np.float64)
    for s in range(n_sel):
        lo, hi = int(row_start[s]), int(sel_global[s]) + 1
        for h in range(n_q_heads):
            g = h // group
            q = q_c[int(sel_local[s]), h]
            keys = k_fused[lo:hi, g, :]
            vals = v_fused[lo:hi, g, :]
            e = (keys @ q) * scale
            w = np.exp(e - e.max())
            out[s, h] = (w @ vals) / w.sum()
    return out


# --------------------------------------------------------------------------
# Gradual filtering. [KV-blog, "渐进式过滤机制"]: layer 1 computes every token
# and keeps a ratio r1 of them; layer 2 recomputes only those candidates and
# keeps r2 < r1; later layers keep rolling with the small pool.
# --------------------------------------------------------------------------
def select_count(percent: int, n_tokens: int) -> int:
    """ceil(percent * n_tokens / 100) in exact integer arithmetic."""
    return -((-percent * n_tokens) // 100)


def layer_plan(layer: int, n_tokens: int, r1: int, r2: int):
    """Percent ratio and selected count of a request at ``layer`` (1-based)."""
    pct = r1 if layer == 1 else r2
    return pct, select_count(pct, n_tokens)


def candidates_for_layer(layer: int, n_tokens: int, first_sel, prev_sel, schedule: str = "pool"):
    """Request-local candidate token list (ascending) for ``layer`` (1-based).

    Layer 1: every token.  Later layers: layer 1's selection ("pool") or the
    previous layer's selection ("chain").
    """
    if layer == 1:
        return np.arange(n_tokens, dtype=np.int64)
    if schedule == "pool":
        return np.asarray(first_sel, dtype=np.int64)
    if schedule == "chain":
        return np.asarray(prev_sel, dtype=np.int64)
    raise ValueError(schedule)


# --------------------------------------------------------------------------
# One layer of the blend over a ragged batch of independent requests.
# --------------------------------------------------------------------------
def blend_layer(*, k_old, v_old, delta, k_new_c, v_new_c, q_c, cand_idx,
                tok_off, cand_off, sel_counts, n_q_heads, n_kv_heads, theta,
                style=ROPE_HALF, scale=None, attend=True, dev_source="v", cache_dtype=None):
    """Run re-rotate, deviation, top-k, fuse and partial attention for one layer.

    Arrays are float64 (values exactly as stored) except the int index arrays.
    tok_off[B+1] / cand_off[B+1] split tokens and candidates by request;
    sel_counts[B] is each request's k.  cand_idx holds packed (global) rows.
    delta None means the cached keys already sit at their new positions.
    dev_source picks what the deviation measures (see ``kv_deviation``); a key
    deviation reads the re-rotated keys as the cache stores them (cache_dtype
    "f32" / "bf16", rounded to nearest even; None keeps float64).
    Returns a dict with k_rot, dev, sel_local, sel_global, k_fused, v_fused, out.
    """
    head_dim = np.asarray(k_old).shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    k_rot = np.asarray(k_old, np.float64) if delta is None else rerotate(k_old, delta, theta, style)
    if dev_source == "v":
        dev = deviation(v_new_c, v_old, cand_idx)
    else:
        k_cached = k_rot if cache_dtype is None else store_as(k_rot, cache_dtype)
        dev = kv_deviation(dev_source, k_new_c=k_new_c, k_cached=k_cached, v_new_c=v_new_c,
                           v_old=v_old, cand_idx=cand_idx)
    sel_local, sel_global, row_start = [], [], []
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    for r in range(len(tok_off) - 1):
        c0, c1 = int(cand_off[r]), int(cand_off[r + 1])
        loc, glob = topk_select(dev[c0:c1], cand_idx[c0:c1], int(sel_counts[r]))
        sel_local.append(loc + c0)
        sel_global.append(glob)
        row_start.append(np.full(len(glob), int(tok_off[r]), dtype=np.int64))
    sel_local = np.concatenate(sel_local) if sel_local else np.zeros(0, np.int64)
    sel_global = np.concatenate(sel_global) if sel_global else np.zeros(0, np.int64)
    row_start = np.concatenate(row_start) if row_start else np.zeros(0, np.int64)
    k_fused, v_fused = fuse(k_rot, v_old, k_new_c, v_new_c, sel_local, sel_global)
    out = None
    if attend:
        out = attention_rows(q_c, sel_local, sel_global, row_start, k_fused, v_fused,
                             n_q_heads, n_kv_heads, scale)
    return dict(k_rot=k_rot, dev=dev, sel_local=sel_local, sel_global=sel_global,
                row_start=row_start, k_fused=k_fused, v_fused=v_fused, out=out)
