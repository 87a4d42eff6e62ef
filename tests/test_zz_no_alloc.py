"""moe_layout_noalloc, the layout for callers that cannot allocate: called
through the C ABI, its outputs equal moe_layout's bit for bit, on two calls
in a row (the second with a smaller input, so the static scratch array holds
the first call's contents when the second starts), then on a layout small
enough for the one-workgroup path (no scratch used) and a large one again."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import layout as olayout, route as oroute

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

KEYS = ("expert_counts", "send_counts", "split_matrix", "recv_counts", "output_splits",
        "offsets", "dst_row", "src_row")

# (tokens, experts, top_k, ep, local rank, align, routing)
SHAPES = [
    (8192, 256, 8, 8, 0, 128, "severe"),   # the DeepSeek-V3 EP=8 share: 65536 assignments
    (3000, 16, 4, 4, 2, 128, "mild"),      # smaller, ragged: 12000 assignments
    (1020, 32, 4, 4, 3, 32, "balanced"),   # 4080 assignments: the one-workgroup path
    (40000, 64, 4, 2, -1, 64, "mild"),     # 160000 assignments, all experts local
]


def _idx(T, E, k, ep, dist, seed):
    cfg = workloads.MoEConfig(name=f"noalloc_{T}_{E}", num_tokens=T, hidden=128,
                              num_experts=E, top_k=k, inter=128, ep_size=ep)
    _, logits = workloads.gen.routing_inputs(cfg, dist, seed, device="cpu")
    return oroute.select(logits.numpy(), k)


def test_noalloc_layout_equals_moe_layout_on_consecutive_calls():
    for i, (T, E, k, ep, lr, align, dist) in enumerate(SHAPES):
        print("CASE noalloc layout", T, E, k, ep, lr, align, dist, flush=True)
        idx = _idx(T, E, k, ep, dist, i)
        idx_d = torch.as_tensor(idx, dtype=torch.int32).cuda()
        want = moe.layout(idx_d, E, ep, lr, align)
        # outputs prefilled with garbage: everything must be written by the call
        got = moe.ops.alloc_layout(want.desc, idx_d.device, workspace=False)
        for key in KEYS:
            getattr(got, key).fill_(-7)
        moe.ops.layout_noalloc(idx_d, E, ep, lr, align, out=got)
        torch.cuda.synchronize()
        for key in KEYS:
            a, b = getattr(got, key).cpu().numpy(), getattr(want, key).cpu().numpy()
            assert (a == b).all(), (key, np.argwhere(a != b)[:5])
        # and the oracle agrees
        L = olayout.layout(idx, E, ep, lr, align, want.m_cap)
        for key in KEYS:
            assert (getattr(got, key).cpu().numpy() == L[key]).all(), key
