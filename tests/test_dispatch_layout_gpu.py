"""GPU parity of moe_dispatch_layout (the per-rank deduplicated dispatch
layout) against oracle/layout.py::dispatch_layout: every output bit-exact.
Routing comes from the oracle on the workloads' seeded logits; ep ranges from
1 to 64 virtual ranks, including shapes whose token count is not a multiple
of the 256-token tile and expert ids outside [0, E), which are skipped."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import layout as olayout, route as oroute
from gpu_util import i32

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

CASES = [  # (workload, ep)
    ("tiny", 2), ("mixtral_8x7b", 8), ("qwen3_30b_a3b", 8), ("qwen3_30b_a3b", 64),
    ("deepseek_v3_ep8_share", 8), ("deepseek_v3_large", 8), ("deepseek_v3_large", 32),
    ("deepseek_v3_large", 64),  # 256 tiles over 8-thread rank groups: several load batches
]


def _check(idx, E, ep):
    print("CASE dispatch_layout", idx.shape, E, ep, flush=True)
    per_rank, per_expert, in_rank, pos = moe.ops.dispatch_layout(i32(idx), E, ep)
    torch.cuda.synchronize()
    want = olayout.dispatch_layout(idx, E, ep)
    np.testing.assert_array_equal(per_rank.cpu().numpy(), want["num_tokens_per_rank"])
    np.testing.assert_array_equal(per_expert.cpu().numpy(), want["num_tokens_per_expert"])
    np.testing.assert_array_equal(in_rank.cpu().numpy(), want["is_token_in_rank"])
    np.testing.assert_array_equal(pos.cpu().numpy(), want["token_rank_pos"])


@pytest.mark.parametrize("name,ep", CASES, ids=[f"{n}-ep{e}" for n, e in CASES])
def test_dispatch_layout(name, ep):
    cfg = workloads.get(name)
    dist = cfg.dists[-1]
    _, logits = workloads.gen.routing_inputs(cfg, dist, 0, device="cpu")
    idx = oroute.select(logits.numpy(), cfg.top_k)
    _check(idx, cfg.num_experts, ep)


@pytest.mark.parametrize("T", [1, 255, 257, 1000])
def test_dispatch_layout_ragged_and_bad_ids(T):
    rng = np.random.default_rng(T)
    E, k, ep = 48, 6, 12
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    bad = rng.random(idx.shape) < 0.03
    idx[bad] = rng.choice([-1, E, E + 7], size=int(bad.sum()))
    _check(idx, E, ep)


def test_dispatch_layout_no_tokens():
    per_rank, per_expert, _, _ = moe.ops.dispatch_layout(
        torch.zeros((0, 2), dtype=torch.int32, device="cuda"), 8, 4)
    torch.cuda.synchronize()
    assert not per_rank.cpu().numpy().any() and not per_expert.cpu().numpy().any()
