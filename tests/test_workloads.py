"""Generator tests (CPU): determinism, planted structure, and the selection gap.

The gap and the planted selection are checked with the CPU oracle's own
deviation and top-k, on the exact stored values.
"""
import numpy as np
import pytest
import torch

from oracle import cacheblend_oracle as O
from selective_recompute_amd import workloads as W


def _np64(t):
    return t.to(torch.float64).cpu().numpy()


def test_presets_shapes():
    tiny, layer7b = W.make_workload("tiny"), W.make_workload("mistral7b-layer")
    assert tiny.n_tokens == 128 and tiny.head_dim == 16 and tiny.dtype == "f32"
    assert layer7b.n_tokens == 2048 and (layer7b.n_q_heads, layer7b.n_kv_heads) == (32, 8)
    gf6k, ctx32k, b70 = (W.make_workload(n) for n in ("7b-32layer-6k", "7b-32layer-32k", "70b-80layer-8req"))
    assert (gf6k.n_tokens, gf6k.n_layers) == (6144, 32)
    assert (ctx32k.n_tokens, ctx32k.n_layers) == (32768, 32)
    assert b70.n_requests == 8 and b70.n_layers == 80 and 57344 <= b70.n_tokens <= 73728
    for chunk_lens in b70.chunks:
        assert 2 <= len(chunk_lens) <= 16
        assert all(256 <= n <= 4096 for n in chunk_lens)
    # deterministic draw
    assert W.make_workload("70b-80layer-8req").chunks == b70.chunks


def test_delta_is_chunk_start():
    wl = W.make_workload("tiny")
    d = wl.delta()
    assert list(d[:64]) == [0] * 64 and list(d[64:]) == [64] * 64
    assert np.array_equal(wl.positions() - d, np.tile(np.arange(64), 2))   # chunk-local p_old


def test_generation_is_deterministic():
    wl = W.make_workload("tiny")
    a = W.layer_inputs(wl, W.PlantedSets(wl), 0)
    b = W.layer_inputs(wl, W.PlantedSets(wl), 0)
    for key in ("k_old", "v_old", "k_new_c", "v_new_c", "q_c", "cand_idx"):
        assert torch.equal(a[key], b[key])
    c = W.layer_inputs(wl, W.PlantedSets(wl), 0, draw=1)
    assert not torch.equal(a["k_old"], c["k_old"])


@pytest.mark.parametrize("name,layers", [("tiny", [0]), ("mistral7b-layer", [0]), ("7b-32layer-6k", [0, 1, 2, 5]),
                                         ("7b-32layer-32k", [0, 1]), ("70b-80layer-8req", [0, 1])])
@pytest.mark.parametrize("schedule", ["pool", "chain"])
def test_planted_selection_has_gap(name, layers, schedule):
    wl = W.make_workload(name)
    sets = W.PlantedSets(wl, schedule)
    for layer in layers:
        x = W.layer_inputs(wl, sets, layer)
        cand = x["cand_idx"].numpy().astype(np.int64)
        dev = O.deviation(_np64(x["v_new_c"]), _np64(x["v_old"]), cand)
        offs = x["h_cand_off"]
        for r in range(wl.n_requests):
            n = wl.request_lengths[r]
            _, k = O.layer_plan(layer + 1, n, wl.r1_pct, wl.r2_pct)
            d_r = dev[offs[r]:offs[r + 1]]
            _, glob = O.topk_select(d_r, cand[offs[r]:offs[r + 1]], k)
            planted = x["planted"][x["planted_off"][r]:x["planted_off"][r + 1]]
            assert np.array_equal(glob, planted)
            srt = np.sort(d_r)[::-1]
            if k < len(srt):
                assert (srt[k - 1] - srt[k]) / srt[k - 1] > 1e-3, (name, layer, r)


def test_persistence_and_pool():
    wl = W.make_workload("7b-32layer-6k")
    sets = W.PlantedSets(wl)
    l0, l1, l2 = sets.layer(0), sets.layer(1), sets.layer(2)
    assert l0.hot.sum() == 922 and len(l0.planted) == 1844
    assert np.array_equal(l1.cand_idx, l0.planted) and np.array_equal(l2.cand_idx, l0.planted)
    assert np.sum(l0.hot & l1.hot) == 738 and np.sum(l1.hot & l2.hot) == 738
    assert len(l1.planted) == 922 and len(l2.planted) == 922
    chain = W.PlantedSets(wl, "chain")
    assert np.array_equal(chain.layer(1).cand_idx, l0.planted)
    assert np.array_equal(chain.layer(2).cand_idx, chain.layer(1).planted)


@pytest.mark.parametrize("name,layer", [("tiny", 0), ("mistral7b-layer", 0), ("7b-32layer-6k", 1)])
@pytest.mark.parametrize("source", ["k", "kv"])
def test_tied_keys_carry_the_planted_gap(name, layer, source):
    """With tied keys and a cache already at the new positions, a key-based
    deviation selects the planted rows with the same tier gap."""
    wl = W.make_workload(name)
    sets = W.PlantedSets(wl)
    x = W.layer_inputs(wl, sets, layer, k_new="tied")
    base = W.layer_inputs(wl, sets, layer)
    for key in ("k_old", "v_old", "v_new_c", "q_c"):            # only K_new changes
        assert torch.equal(x[key], base[key])
    cand = x["cand_idx"].numpy().astype(np.int64)
    dev = O.kv_deviation(source, k_new_c=_np64(x["k_new_c"]), k_cached=_np64(x["k_old"]),
                         v_new_c=_np64(x["v_new_c"]), v_old=_np64(x["v_old"]), cand_idx=cand)
    offs = x["h_cand_off"]
    for r in range(wl.n_requests):
        _, k = O.layer_plan(layer + 1, wl.request_lengths[r], wl.r1_pct, wl.r2_pct)
        d_r = dev[offs[r]:offs[r + 1]]
        _, glob = O.topk_select(d_r, cand[offs[r]:offs[r + 1]], k)
        assert np.array_equal(glob, x["planted"][x["planted_off"][r]:x["planted_off"][r + 1]])
        srt = np.sort(d_r)[::-1]
        assert (srt[k - 1] - srt[k]) / srt[k - 1] > 1e-3


@pytest.mark.parametrize("schedule", ["pool", "chain"])
def test_candidates_and_selections_ascend_over_the_batch(schedule):
    """cb_blend_layer's rotate-or-replace pass needs the selection strictly
    ascending over the whole packed batch; it is, whenever each request's
    candidates ascend inside the request's rows: the oracle's top-k emits each
    request's selection in ascending order, and the requests' rows follow
    each other.  Checked on the ragged 8-request workload, layers 1-3."""
    wl = W.make_workload("70b-80layer-8req")
    sets = W.PlantedSets(wl, schedule)
    for layer in range(3):
        s = sets.layer(layer)
        assert np.all(np.diff(s.cand_idx) > 0)
        for r in range(wl.n_requests):
            c = s.cand_idx[s.cand_off[r]:s.cand_off[r + 1]]
            assert c.min() >= wl.tok_off[r] and c.max() < wl.tok_off[r + 1]
        rng = np.random.default_rng(layer)
        dev = rng.random(len(s.cand_idx))
        sel = []
        for r in range(wl.n_requests):
            c0, c1 = s.cand_off[r], s.cand_off[r + 1]
            k = O.layer_plan(layer + 1, wl.request_lengths[r], wl.r1_pct, wl.r2_pct)[1]
            sel.append(O.topk_select(dev[c0:c1], s.cand_idx[c0:c1], min(k, c1 - c0))[1])
        assert np.all(np.diff(np.concatenate(sel)) > 0)
        assert np.all(np.diff(s.planted) > 0)
