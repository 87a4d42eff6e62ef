"""Expert-major permute (oracle): gather each token's row into every local row
that one of its (token, slot) assignments occupies.

Follows the reorder step of the AutoEP flow (DeepSpeed AutoEP commit text,
section "Design", runtime step 3 "reorder tokens by expert assignment") and
the dispatch of DeepEP issue #272 (x with topk_idx/topk_weights in, rows
grouped per expert out). Row r holds token ``src_row[r] // top_k``.
A pure gather: works on any dtype, including uint16 bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np


def permute(x, src_row, top_k: int, rows=None) -> np.ndarray:
    """x_perm [len(rows), H]; rows default to all of ``src_row``. Padding
    rows (src_row < 0) come back as zeros; the kernel leaves them unwritten,
    so only rows with src_row >= 0 are compared."""
    x = np.asarray(x)
    src = np.asarray(src_row, dtype=np.int64)
    rows = np.arange(src.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], x.shape[1]), dtype=x.dtype)
    s = src[rows]
    valid = s >= 0
    out[valid] = x[s[valid] // top_k]
    return out


def permute_weighted(x, dst_row, topk_w, rows: int) -> tuple[np.ndarray, np.ndarray]:
    """x_perm with the routing score applied before the experts (AutoEP's
    score_apply="pre", DeepSpeed PR #8847, section "Change", the fused restore
    refuses it; the experts then see ``w * x`` and the combine sums with unit
    weights). Row dst_row[t, s] = bf16(fp32(w[t, s]) * x[t]), one rounding.
    Returns (float64 values [rows, H], written [rows] bool)."""
    from . import bf16
    x32 = np.asarray(x).astype(np.float32)
    dst = np.asarray(dst_row, dtype=np.int64)
    w32 = np.asarray(topk_w).astype(np.float32)
    T, k = dst.shape
    out = np.zeros((rows, x32.shape[1]), dtype=np.float64)
    written = np.zeros(rows, dtype=bool)
    for t in range(T):
        for s in range(k):
            r = dst[t, s]
            if r >= 0:
                out[r] = bf16.round_to_bf16((w32[t, s] * x32[t]).astype(np.float64))
                written[r] = True
    return out, written
