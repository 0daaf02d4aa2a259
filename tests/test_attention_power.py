"""The attention parity bar has power on long rows (CPU, oracle only).

The GPU parity tests compare outputs with the oracle at 2e-2 absolute.  On
plain Gaussian inputs a long row's output is tiny and a lost block of keys
hides under that bar; the needle and peaked input families of tests/needles.py
are built so that it cannot.  Here the oracle itself plays the broken kernel:
the same rows are computed with one key chunk (an eighth of the row, the
largest chunk a split uses), one needle's 64-key tile, or a row's own key
removed, and the bar must reject every such output, at 32k and at 128k keys.
Rounding the true output to bf16 (what a correct kernel stores) must pass.
"""
import math

import numpy as np
import pytest
import torch

import needles as N
from oracle import cacheblend_oracle as O


def _np64(t):
    return t.to(torch.float64).numpy()


def _case(n, hq, hkv, d, family, seed):
    rng = np.random.default_rng(seed)
    k_sel = max(64, n // 100)
    sel = np.unique(np.concatenate([rng.choice(n, k_sel, replace=False), [n - 1]]))
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(len(sel), hq, d, generator=gen).to(torch.bfloat16)
    k = torch.randn(n, hkv, d, generator=gen).to(torch.bfloat16)
    v = torch.randn(n, hkv, d, generator=gen).to(torch.bfloat16)
    needle = np.zeros(0, np.int64)
    if family == "needle":
        needle = N.needle_rows(sel, np.array([0, n]), np.array([0, len(sel)]))
        # q holds one row per selected row here: sharpen those, plant in k / v
        q, k, v = N.plant_in_cache(q, k, v, needle, seed)
    else:
        q = N.peak_queries(q)
    return _np64(q), _np64(k), _np64(v), sel, needle


def _attend(q, rows, sel, k, v, hq, hkv, d, end=None, start=None):
    end = sel[rows] if end is None else end
    start = np.zeros(len(rows), np.int64) if start is None else start
    return O.attention_rows(q[rows], np.arange(len(rows)), end, start, k, v, hq, hkv,
                            1.0 / math.sqrt(d))


@pytest.mark.parametrize("family", ["needle", "peaked"])
@pytest.mark.parametrize("n", [32768, 131072])
def test_bar_rejects_a_lost_key_chunk(n, family):
    hq, hkv, d = 8, 2, 128
    q, k, v, sel, needle = _case(n, hq, hkv, d, family, seed=n + len(family))
    rows = np.arange(len(sel) - 4, len(sel))          # the last rows see every chunk
    ref = _attend(q, rows, sel, k, v, hq, hkv, d)
    # what a correct bf16 kernel can store passes
    rounded = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    assert N.attention_close(rounded, ref)
    assert np.abs(ref).max() > 0.2                     # the outputs are O(1)
    chunk = n // 8
    for c in (0, 3, 7):
        lo, hi = c * chunk, (c + 1) * chunk
        kd, vd, end, start = N.drop_keys(k, v, sel[rows], np.zeros(len(rows), np.int64), lo, hi)
        if c == 7:
            # the last chunk holds the rows themselves: keep it, drop the one before
            lo, hi = 6 * chunk, 7 * chunk
            kd, vd, end, start = N.drop_keys(k, v, sel[rows], np.zeros(len(rows), np.int64), lo, hi)
        got = _attend(q, rows, sel, kd, vd, hq, hkv, d, end, start)
        err = N.attention_error(got, ref)
        assert not N.attention_close(got, ref), f"chunk [{lo}, {hi}) lost: max err {err}"


@pytest.mark.parametrize("n", [32768, 131072])
def test_bar_rejects_a_lost_needle_tile_or_diagonal(n):
    hq, hkv, d = 8, 2, 128
    q, k, v, sel, needle = _case(n, hq, hkv, d, "needle", seed=7 * n)
    assert len(needle) >= N.NEEDLES_PER_REQUEST
    last = np.arange(len(sel) - 2, len(sel))
    ref = _attend(q, last, sel, k, v, hq, hkv, d)
    # the 64-key tile of a needle in the middle of the row
    mid = needle[len(needle) // 2]
    lo = mid // 64 * 64
    kd, vd, end, start = N.drop_keys(k, v, sel[last], np.zeros(len(last), np.int64), lo, lo + 64)
    got = _attend(q, last, sel, kd, vd, hq, hkv, d, end, start)
    assert not N.attention_close(got, ref), f"tile of needle {mid}: max err {N.attention_error(got, ref)}"
    # the diagonal: a needle row that is also a query row loses its own key
    row = int(np.searchsorted(sel, needle[-2]))
    assert sel[row] == needle[-2]
    one = np.array([row])
    ref1 = _attend(q, one, sel, k, v, hq, hkv, d)
    got1 = _attend(q, one, sel, k, v, hq, hkv, d, end=sel[one] - 1)
    assert not N.attention_close(got1, ref1), f"diagonal: max err {N.attention_error(got1, ref1)}"


def test_needle_rows_cover_every_chunk():
    """Every chunk of every split the planner may choose (2 to 8 chunks of a
    row, 64-key multiples) holds a needle, in each request of a ragged batch,
    but for a trailing remainder shorter than a 16th of the row."""
    rng = np.random.default_rng(0)
    lens = [4111, 13478, 3671, 6262, 6703, 7355, 5621, 19899]
    tok_off = np.concatenate([[0], np.cumsum(lens)])
    sels = [np.sort(rng.choice(n, (25 * n + 99) // 100, replace=False)) + tok_off[r]
            for r, n in enumerate(lens)]
    sel_off = np.concatenate([[0], np.cumsum([len(s) for s in sels])])
    needle = N.needle_rows(np.concatenate(sels), tok_off, sel_off)
    for r, n in enumerate(lens):
        mine = needle[(needle >= tok_off[r]) & (needle < tok_off[r + 1])] - tok_off[r]
        assert len(mine) >= 8
        for chunks in range(2, 9):
            kc = (-(-n // chunks) + 63) // 64 * 64
            for c in range(-(-n // kc)):
                lo, hi = c * kc, min(n, (c + 1) * kc)
                if hi - lo < n / 16:
                    continue
                assert np.any((mine >= lo) & (mine < hi)), (r, chunks, c)
