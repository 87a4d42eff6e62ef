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
