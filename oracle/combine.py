"""Fused weighted-sum combine (oracle): un-permute the expert output rows and
sum ``routing weight x row`` over each token's top-k slots.

Passages followed (DeepSpeed PR #8847 "AutoEP: support
combine_impl=fused_weighted_sum with AutoEP+AutoTP folding"):

* section "Change": rows are addressed by one flat index
  ``token * top_k + slot``; the routing weights stay in the router dtype
  (FP32) laid out as ``[tokens, top_k]``; if some (token, slot) is not
  covered, a RuntimeError is raised instead of reading an unset row;
* section "Problem": the fused kernel accumulates in FP32, where the default
  folded restore multiplies and adds in the activation dtype with one
  ``index_add_`` per top-k slot;
* section "Benchmark": the fused output's error against an FP64 reference is
  the rounding of the bf16 output itself.

So the oracle sums in fp64, in slot order, and rounds once to bf16. A slot
whose row lives on another GPU share has ``dst_row = -1`` and contributes
nothing; a token with no local slot gives a zero row. ``restore_default``
is the activation-dtype restore of section "Problem", kept for the error
contrast of section "Benchmark".
"""
from __future__ import annotations

import numpy as np

from . import bf16


def combine(y, dst_row, topk_w, validate_coverage: bool = False) -> np.ndarray:
    """out [T, H] float64 (unrounded): sum over slots s with dst_row[t, s] >= 0
    of topk_w[t, s] * y[dst_row[t, s]], added in slot order."""
    y = np.asarray(y, dtype=np.float64)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = dst.shape
    if validate_coverage and (dst < 0).any():
        t, s = np.argwhere(dst < 0)[0]
        raise RuntimeError(f"(token {t}, slot {s}) is not covered by any expert row")
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        out[m] += w[m, s][:, None] * y[r[m]]
    return out


def combine_bf16(y, dst_row, topk_w, validate_coverage: bool = False) -> np.ndarray:
    """The fused restore's output: fp64 sum, one round-to-nearest-even to bf16
    (returned as float64 values)."""
    return bf16.round_to_bf16(combine(y, dst_row, topk_w, validate_coverage))


def restore_default(y, dst_row, topk_w) -> np.ndarray:
    """Default folded restore in bf16: the weight is cast to bf16, each
    product is rounded to bf16 and each per-slot addition is rounded to bf16."""
    y = np.asarray(y, dtype=np.float64)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = bf16.round_to_bf16(np.asarray(topk_w, dtype=np.float64))
    T, k = dst.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        prod = bf16.round_to_bf16(w[m, s][:, None] * y[r[m]])
        out[m] = bf16.round_to_bf16(out[m] + prod)
    return out
