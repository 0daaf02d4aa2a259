"""cb_blend_layer inside a captured HIP graph: every replay, with the
program's own eager work and synchronisations between replays, must match the
eager call bit for bit (the library issues kernel launches only -- no memsets,
allocations or synchronisation -- so its per-layer sequence is capturable)."""
import numpy as np
import pytest
import torch

from selective_recompute_amd import binding as B
from selective_recompute_amd import pipeline as PL
from selective_recompute_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[graph-test] {msg}", flush=True)


@pytest.mark.parametrize("name,source,in_launch", [("mistral7b-layer", "v", False),
                                                   ("tiny", "v", False),
                                                   ("mistral7b-layer", "kv", False),
                                                   ("mistral7b-layer", "v", True),
                                                   ("70b-80layer-8req", "v", True)])
def test_blend_layer_graph_replays_match_eager(name, source, in_launch):
    """in_launch: the top-k inside the deviation launch, whose arrival counters
    every replay leaves at zero for the next (no memset in the graph)."""
    say(f"graph replay {name} deviation source {source} select in launch {in_launch}")
    wl = W.make_workload(name)
    sets = W.PlantedSets(wl)
    runner = PL.BlendRunner(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.torch_dtype,
                            wl.request_lengths, wl.r1_pct, wl.r2_pct, 1, wl.rope_theta,
                            dev_source=source, device=DEV, in_launch_select=in_launch)
    x = W.layer_inputs(wl, sets, 0, device=DEV)
    k0, v0 = x["k_old"].clone(), x["v_old"].clone()
    o = runner.outs[0]
    prep = B.PreparedLayer(runner.geom, runner.batches[0], k=x["k_old"], v=x["v_old"],
                           k_new_c=x["k_new_c"], v_new_c=x["v_new_c"], q_c=x["q_c"],
                           delta=x["delta"], cand_idx=runner.candidates(0),
                           rope_theta=wl.rope_theta, rope_style=B.ROPE_HALF,
                           softmax_scale=runner.scale, dev=o["dev"], sel_local=o["sel_local"],
                           sel_global=o["sel_global"], out=o["out"], workspace=runner.workspace,
                           dev_source=runner.dev_source, flags=runner.flags)
    outs = [o["dev"], o["sel_local"], o["sel_global"], o["out"], x["k_old"], x["v_old"]]
    stream = torch.cuda.Stream()

    def restore():
        x["k_old"].copy_(k0)
        x["v_old"].copy_(v0)
        for t in outs[:4]:
            t.fill_(-1 if t.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()

    restore()
    with torch.cuda.stream(stream):
        prep.launch(stream.cuda_stream)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    if source == "v":       # the inputs plant the deviation tiers in V
        assert np.array_equal(eager[2].cpu().numpy(), sets.layer(0).planted)

    restore()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        prep.launch(stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a, b), f"replay {rep} differs"
