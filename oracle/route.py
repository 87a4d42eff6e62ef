"""Token-choice top-k routing (oracle).

The AutoEP runtime routes with a token-choice top-k router (DeepSpeed AutoEP
commit text, section "Attribution": ep_router.py, from TorchTitan's
TokenChoiceTopKRouter; section "Design", runtime step 2 "route tokens with
the EP router"). Each token picks distinct experts (DeepSpeed PR #8847,
section "Benchmark": random routing with distinct experts per token), and the
routing weights stay in the router dtype, FP32 (same page, section "Change").

The pages print no router formula; the workloads define it as softmax over
all E experts, keep the top k, renormalise the k weights. Readings where the
pages are silent: the selection is taken on the fp32 logits themselves
(softmax is strictly increasing, so the same experts win), ordered by
descending logit with ties going to the lower expert id; the output slots
are in that order.
"""
from __future__ import annotations

import numpy as np


def select(logits, top_k: int) -> np.ndarray:
    """topk_idx [T, k] int32: per token, the k experts with the largest fp32
    logit, descending, ties to the lower expert id.

    A stable sort of the negated logits keeps equal logits in ascending
    expert order; -0.0 and +0.0 compare equal and so tie as well."""
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :top_k]).astype(np.int32)


def weights(logits, topk_idx) -> np.ndarray:
    """topk_w [T, k] float64: softmax over all E experts (fp64), the selected
    probabilities, renormalised to sum to one."""
    l64 = np.asarray(logits, dtype=np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, np.asarray(topk_idx, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(logits, top_k: int):
    """(topk_idx [T, k] int32, topk_w [T, k] float64)."""
    idx = select(logits, top_k)
    return idx, weights(logits, idx)
