"""cb_check_indices: the device-side check of the index preconditions.

Valid inputs give 0 -- a hand-made ragged batch and a real layer's
candidates and selection (the 70B-shaped batch, layers 1 and 2, after
cb_blend_layer) -- and each planted violation sets exactly its own bit."""
import math

import numpy as np
import pytest
import torch

from selective_recompute_amd import binding as B
from selective_recompute_amd import pipeline as PL
from selective_recompute_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(x):
    return torch.tensor(x, dtype=torch.int32, device=DEV)


def _flags(rb, cand, sl, sg):
    out = B.check_indices(rb, cand, sl, sg)
    torch.cuda.synchronize()
    return int(out.item())


def test_each_violation_sets_its_bit():
    # two requests: tokens [0, 10) and [10, 25)
    rb = B.RaggedBatch([0, 10, 25], [0, 6, 13], [0, 2, 5], DEV)
    cand = [0, 2, 3, 5, 8, 9, 10, 11, 15, 16, 20, 21, 24]
    sl = [1, 4, 7, 9, 12]
    sg = [cand[i] for i in sl]
    assert _flags(rb, _i32(cand), _i32(sl), _i32(sg)) == 0
    # every pointer may be left out
    assert _flags(rb, None, None, None) == 0
    assert _flags(rb, _i32(cand), None, None) == 0
    cases = [
        ("cand outside its request", dict(cand={0: 11}), B.CB_CHECK_CAND_RANGE | B.CB_CHECK_CAND_ORDER),
        ("cand not ascending", dict(cand={2: 2}), B.CB_CHECK_CAND_ORDER),
        ("sel outside its request", dict(sg={2: 5}), B.CB_CHECK_SEL_RANGE | B.CB_CHECK_SEL_ORDER | B.CB_CHECK_LOCAL_MISMATCH),
        ("sel not ascending over the batch", dict(sg={1: 2}, sl={1: 1}), B.CB_CHECK_SEL_ORDER),
        ("sel_local outside its candidates", dict(sl={0: 6}), B.CB_CHECK_LOCAL_RANGE),
        ("sel_local and sel_global disagree", dict(sl={3: 8}), B.CB_CHECK_LOCAL_MISMATCH),
    ]
    for name, edits, want in cases:
        c, l, g = list(cand), list(sl), list(sg)
        for i, v in edits.get("cand", {}).items():
            c[i] = v
        for i, v in edits.get("sl", {}).items():
            l[i] = v
        for i, v in edits.get("sg", {}).items():
            g[i] = v
        got = _flags(rb, _i32(c), _i32(l), _i32(g))
        assert got == want, f"{name}: flags {got:#x}, expected {want:#x}"


@pytest.mark.parametrize("layer", [0, 1])
def test_a_real_layer_passes(layer):
    wl = W.make_workload("70b-80layer-8req")
    sets = W.PlantedSets(wl)
    counts = PL.GradualFilter(wl.request_lengths, wl.r1_pct, wl.r2_pct).counts(layer)
    x = {k: (v.to(DEV) if torch.is_tensor(v) else v)
         for k, v in W.layer_inputs(wl, sets, layer, device=DEV).items()}
    g = B.geom(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.torch_dtype)
    rb = B.RaggedBatch(x["h_tok_off"], x["h_cand_off"], PL.offsets(counts), DEV)
    dev = torch.empty(rb.n_cand, dtype=torch.float32, device=DEV)
    sl = torch.empty(rb.n_sel, dtype=torch.int32, device=DEV)
    sg = torch.empty(rb.n_sel, dtype=torch.int32, device=DEV)
    out = torch.empty((rb.n_sel, wl.n_q_heads, wl.head_dim), dtype=wl.torch_dtype, device=DEV)
    B.blend_layer(g, rb, k=x["k_old"], v=x["v_old"], k_new_c=x["k_new_c"],
                  v_new_c=x["v_new_c"], q_c=x["q_c"], delta=x["delta"], cand_idx=x["cand_idx"],
                  rope_theta=wl.rope_theta, rope_style=B.ROPE_HALF,
                  softmax_scale=1.0 / math.sqrt(wl.head_dim), dev=dev, sel_local=sl,
                  sel_global=sg, out=out)
    assert _flags(rb, x["cand_idx"], sl, sg) == 0
    assert np.array_equal(sg.cpu().numpy(), x["planted"])
