"""The forward step enqueues GPU work only: no host synchronisation and no
host read of device data anywhere between routing and the combine, as the pages ask of the layout (xtuner PR #2056, review: a histogram
that forces a host-device sync is avoided; DeepSpeed PR #8847, section
"Change": worst-case sizing instead of a sync). Stream capture in global mode
(torch's default) rejects synchronising calls (stream or device
synchronisation, synchronous copies), so a step that captures is the check;
the graph must then replay to the eager step's output bit for bit, several times,
with eager work between the replays."""
from __future__ import annotations

import pytest
import torch

import workloads
from workloads import MoEConfig

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

CONFIGS = {
    "tiny": (workloads.get("tiny"), "balanced", 1),
    "ragged": (MoEConfig(name="ragged_graph", num_tokens=3000, hidden=384, num_experts=16,
                         top_k=4, inter=256, ep_size=4, local_rank=2, align=128,
                         dists=("mild",), shares=(2,)), "mild", 2),
    # above 4096 assignments the layout takes its three-launch form
    "tiled": (MoEConfig(name="tiled_graph", num_tokens=8192, hidden=512, num_experts=32,
                        top_k=4, inter=256, ep_size=1, local_rank=-1, align=128,
                        dists=("severe",)), "severe", -1),
}


@pytest.mark.parametrize("name", list(CONFIGS))
def test_forward_step_captures_and_replays_bit_exactly(name):
    cfg, dist, share = CONFIGS[name]
    print("CASE graph", name, dist, share, flush=True)
    dev = torch.device("cuda:0")
    x, logits = workloads.gen.routing_inputs(cfg, dist, 0, device=dev)
    w1, w3, w2 = workloads.gen.expert_weights(cfg, cfg.local_experts(share), 0, device=dev)
    layer = moe.MoELayer(cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter,
                         w1, w3, w2, cfg.ep_size, share, cfg.align)
    stages = layer.stages(x, logits)

    def step():
        for _, run in stages:
            run()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):  # raises if any call synchronises or reads back
        step()
    torch.cuda.synchronize()

    step()
    torch.cuda.synchronize()
    ref = layer.out.view(torch.int16).clone()
    assert ref.any()
    for rep in range(3):
        layer.out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        diff = int((layer.out.view(torch.int16) != ref).sum())
        assert diff == 0, (rep, diff)
        step()  # eager work between the replays
        torch.cuda.synchronize()
        assert bool((layer.out.view(torch.int16) == ref).all())
