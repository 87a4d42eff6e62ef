"""One GPU's MoE layer as a fixed pipeline of the library's calls:

    moe_route -> moe_layout -> moe_grouped_gate_up_gather -> moe_grouped_down -> moe_combine

where the gate/up GEMM gathers its rows from the token rows itself (the
permute fused into its operand loads, so the expert-major copy of x is never
written), or, with ``gather=False``, the permute as its own stage:

    moe_route -> moe_layout -> moe_permute -> moe_grouped_gate_up
              -> moe_grouped_down -> moe_combine

All buffers are allocated once, at construction, for the worst case
(``m_cap`` local rows), so a forward pass launches kernels only: no
allocation, no host sync (the dispatch-without-waiting principle of DeepEP's
``num_worst_tokens`` in DeepEP issue #272 and the host-sync-free hot path of
xtuner PR #2056, section "Design").
"""
from __future__ import annotations

import torch

from . import ops


class MoELayer:
    def __init__(self, num_tokens: int, hidden: int, num_experts: int, top_k: int, inter: int,
                 w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, ep_size: int = 1,
                 local_rank: int = -1, align: int = 128, gather: bool = True):
        """w1, w3: [E_loc, H, I] and w2: [E_loc, I, H], bf16 on the GPU (math
        orientation); repacked once here into the GEMM's layout."""
        dev = w1.device
        self.T, self.H, self.E, self.k, self.I = num_tokens, hidden, num_experts, top_k, inter
        self.desc = ops.layout_desc(num_tokens, num_experts, top_k, ep_size, local_rank, align)
        self.ep_size, self.local_rank, self.align = ep_size, local_rank, align
        self.gather = gather
        self.L = ops.alloc_layout(self.desc, dev)
        self.m_cap = self.L.m_cap
        self.w1t = ops.pack_weights(w1)
        self.w3t = ops.pack_weights(w3)
        self.w2t = ops.pack_weights(w2)
        self.topk_idx = torch.empty((num_tokens, top_k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((num_tokens, top_k), dtype=torch.float32, device=dev)
        self.x_perm = torch.empty((self.m_cap, hidden), dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((self.m_cap, inter), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((self.m_cap, hidden), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((num_tokens, hidden), dtype=torch.bfloat16, device=dev)

    def stages(self, x: torch.Tensor, logits: torch.Tensor):
        """The layer as (name, thunk) pairs, in order, for timing each stage."""
        L = self.L
        front = [
            ("route", lambda: ops.route(logits, self.k, self.topk_idx, self.topk_w)),
            ("layout", lambda: ops.layout(self.topk_idx, self.E, self.ep_size, self.local_rank,
                                          self.align, out=L)),
        ]
        if self.gather:
            middle = [("gate_up", lambda: ops.grouped_gate_up_gather(
                x, L.src_row, self.k, L.offsets, L.local_counts, self.w1t, self.w3t,
                out=self.h))]
        else:
            middle = [
                ("permute", lambda: ops.permute(x, L.dst_row, L.src_row, L.offsets, self.m_cap,
                                                out=self.x_perm)),
                ("gate_up", lambda: ops.grouped_gate_up(self.x_perm, L.offsets, L.local_counts,
                                                        self.w1t, self.w3t, out=self.h)),
            ]
        back = [
            ("down", lambda: ops.grouped_down(self.h, L.offsets, L.local_counts, self.w2t,
                                              out=self.y)),
            ("combine", lambda: ops.combine(self.y, L.dst_row, self.topk_w, out=self.out)),
        ]
        return front + middle + back

    def forward(self, x: torch.Tensor, logits: torch.Tensor) -> torch.Tensor:
        for _, run in self.stages(x, logits):
            run()
        return self.out

    __call__ = forward
