"""The whole single-GPU MoE layer (oracle): route -> layout -> permute ->
experts -> combine, the order of the AutoEP runtime path (DeepSpeed AutoEP
commit text, section "Design": route, reorder by expert, dispatch, local
grouped expert compute, combine and restore the original order), with the
cross-GPU all-to-all steps absent because one GPU runs its own share.

The layer's output is the exact (fp64) weighted sum of fp64 expert outputs;
the bf16 rounding of expert outputs on the GPU and its FP32 combine are
covered by the layer tolerance. ``token_outputs`` gives the same result for a
few tokens at a time, straight
from the definition (the sum over a token's local slots of weight times its
expert's SwiGLU output), for sampling layers too large to run whole.
"""
from __future__ import annotations

import numpy as np

from . import bf16, combine, experts, layout, permute, route


def layer(x, logits, top_k: int, weights_of, num_experts: int, ep_size: int = 1,
          local_rank: int = -1, align: int = 128, m_cap: int | None = None) -> dict:
    """x [T, H] (bf16 values as float), logits [T, E] fp32; ``weights_of(e)``
    returns local expert e's (w1 [H, I], w3 [H, I], w2 [I, H])."""
    idx, w = route.route(logits, top_k)
    L = layout.layout(idx, num_experts, ep_size, local_rank, align, m_cap)
    xp = permute.permute(np.asarray(x, dtype=np.float64), L["src_row"], top_k)
    y = experts.grouped_swiglu(xp, L["offsets"], L["local_counts"], weights_of)
    out = combine.combine_exact(y, L["dst_row"], w)
    return {"topk_idx": idx, "topk_w": w, "layout": L, "x_perm": xp, "y": y,
            "out": out, "out_bf16": bf16.round_to_bf16(out)}


def token_outputs(tokens, x, topk_idx, topk_w, weights_of, first_local: int,
                  num_local: int) -> np.ndarray:
    """out[t] (fp64, unrounded) for the listed tokens: slots whose expert is
    local contribute topk_w[t, s] * SwiGLU_e(x[t]), added in slot order."""
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = np.asarray(topk_idx, dtype=np.int64)[tokens]
    w = np.asarray(topk_w, dtype=np.float64)[tokens]
    xs = np.asarray(x, dtype=np.float64)[tokens]
    n, k = idx.shape
    ys = np.zeros((n, k, xs.shape[1]), dtype=np.float64)
    for e in np.unique(idx):
        if not (first_local <= e < first_local + num_local):
            continue
        i, s = np.nonzero(idx == e)
        ys[i, s] = experts.swiglu(xs[i], *weights_of(int(e) - first_local))
    out = np.zeros_like(xs)
    for s in range(k):
        local = (idx[:, s] >= first_local) & (idx[:, s] < first_local + num_local)
        out[local] += w[local, s][:, None] * ys[local, s]
    return out
