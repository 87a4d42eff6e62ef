"""Backward of the routing, permute and fused combine steps (oracle).

Passages followed:

* DeepEP issue #272 (answer of Jul 2, 2025): the backward of the dispatch
  (here the permute, its single-GPU part) is a combine of the row gradients,
  and the backward of the combine is a dispatch of the output gradient.
* DeepSpeed PR #8847, section "Tests": the fused restore back-propagates a
  row gradient and a score gradient; section "Benchmark": one forward and
  backward, errors against an FP64 reference, and the score (router)
  gradient computed in FP32 by the fused path (relative L2 error about
  8.4e-8), where the default path goes through bf16 weights.

The forward being differentiated is the plain definition each forward
oracle states:

    combine:  out[t]  = sum_s w[t, s] * y[dst_row[t, s]]        (local slots)
    permute:  x_perm[dst_row[t, s]] = x[t]
    route:    w[t, :] = softmax over the k selected logits of token t

so the gradients are, for a loss with gradient G = dL/d out:

    combine:  grad_y[dst_row[t, s]] = w[t, s] * G[t]
              grad_w[t, s]          = <G[t], y[dst_row[t, s]]>   (0 if not local)
    permute:  grad_x[t]             = sum_s grad_x_perm[dst_row[t, s]]
    route:    grad_logit[t, e_j]    = w_j * (g_j - sum_i w_i * g_i)
              for the selected e_j with g = grad_w[t, :]; 0 for the others.

Readings where the pages are silent (the precision the fused kernel keeps
for the gradients it returns): the row gradient is the fp32 product
``w * G`` rounded once to bf16, the row dtype; the score gradient is an FP32
sum whose order the pages do not fix, so the oracle gives it exactly (fp64,
the reference of the pages' error figure) and tests hold the GPU to the
bound any fp32 summation order satisfies; the permute gradient is summed in
fp32 in slot order and rounded once to bf16, like the combine with unit
weights; the routing gradient is formed in fp64 here and compared within an
fp32 bound. A slot whose row lives on another GPU share (``dst_row = -1``)
has score gradient 0 on this share, and its row is not touched.
"""
from __future__ import annotations

import numpy as np

from . import bf16


def combine_backward_rows(grad_out, dst_row, topk_w, y_rows: int) -> tuple[np.ndarray, np.ndarray]:
    """(grad_y [y_rows, H] float64 holding bf16 values, written [y_rows] bool).

    Row dst_row[t, s] receives bf16(fp32(w[t, s]) * G[t]) with the product
    taken in fp32; rows no local slot points at are not written (False)."""
    g32 = np.asarray(grad_out).astype(np.float32)
    dst = np.asarray(dst_row, dtype=np.int64)
    w32 = np.asarray(topk_w).astype(np.float32)
    T, k = dst.shape
    out = np.zeros((y_rows, g32.shape[1]), dtype=np.float64)
    written = np.zeros(y_rows, dtype=bool)
    for t in range(T):
        for s in range(k):
            r = dst[t, s]
            if r < 0:
                continue
            prod = (w32[t, s] * g32[t]).astype(np.float32)  # fp32 product
            out[r] = bf16.round_to_bf16(prod.astype(np.float64))
            written[r] = True
    return out, written


def combine_backward_scores(grad_out, y, dst_row) -> np.ndarray:
    """grad_w [T, k] float64: <G[t], y[dst_row[t, s]]> summed exactly (fp64
    products of the bf16 values are exact, the fp64 sum is the reference);
    0 where the slot is not local."""
    g = np.asarray(grad_out, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    dst = np.asarray(dst_row, dtype=np.int64)
    T, k = dst.shape
    gw = np.zeros((T, k), dtype=np.float64)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        gw[m, s] = np.einsum("th,th->t", g[m], y[r[m]])
    return gw


def score_bound(grad_out, y, dst_row) -> np.ndarray:
    """[T, k] float64: the largest error any fp32 summation order of the H
    exact products can make, (H - 1) * 2^-24 * sum_h |G[t, h] * y[r, h]|.
    (bf16 x bf16 products are exact in fp32: 8 + 8 significant bits.)"""
    g = np.abs(np.asarray(grad_out, dtype=np.float64))
    y = np.abs(np.asarray(y, dtype=np.float64))
    dst = np.asarray(dst_row, dtype=np.int64)
    T, k = dst.shape
    H = g.shape[1]
    b = np.zeros((T, k), dtype=np.float64)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        b[m, s] = (H - 1) * 2.0 ** -24 * np.einsum("th,th->t", g[m], y[r[m]])
    return b


def pairwise_fp32_sum(v: np.ndarray) -> np.float32:
    """Sum of a 1-D float32 array by recursive halving, every addition in
    fp32: one concrete fp32 reduction order, used to show the size of an
    fp32 score-gradient error."""
    v = np.asarray(v, dtype=np.float32)
    while v.shape[0] > 1:
        if v.shape[0] % 2:
            v = np.concatenate([v, np.zeros(1, dtype=np.float32)])
        v = (v[0::2] + v[1::2]).astype(np.float32)
    return v[0] if v.shape[0] else np.float32(0.0)


def permute_backward(grad_x_perm, dst_row) -> np.ndarray:
    """grad_x [T, H] float32 before rounding: for each token, the fp32 sum in
    slot order of the gradient rows of its local slots (0 if none)."""
    gp = np.asarray(grad_x_perm).astype(np.float32)
    dst = np.asarray(dst_row, dtype=np.int64)
    T, k = dst.shape
    out = np.zeros((T, gp.shape[1]), dtype=np.float32)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        out[m] = out[m] + gp[r[m]]
    return out


def permute_backward_bf16(grad_x_perm, dst_row) -> np.ndarray:
    """The permute gradient as returned: the fp32 slot-order sum rounded once
    to bf16, as float64 values."""
    return bf16.round_to_bf16(permute_backward(grad_x_perm, dst_row).astype(np.float64))


def route_backward(topk_idx, topk_w, grad_w, num_experts: int) -> np.ndarray:
    """grad_logits [T, E] float64: the softmax-over-selected gradient
    w_j * (g_j - sum_i w_i g_i) at the selected experts, zero elsewhere."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    g = np.asarray(grad_w, dtype=np.float64)
    T, k = idx.shape
    out = np.zeros((T, num_experts), dtype=np.float64)
    dot = (w * g).sum(axis=1, keepdims=True)
    np.put_along_axis(out, idx, w * (g - dot), axis=1)
    return out
