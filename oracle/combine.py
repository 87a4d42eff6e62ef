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

The pages fix the precision of this step, so ``combine`` is the FP32 sum:
each product ``w * y`` is an fp32 multiplication, each partial sum an fp32
addition, slots added in order 0..k-1 starting from zero, and the result is
rounded once to bf16 (reading: "accumulates in FP32" taken literally, IEEE
fp32 operations, no fused multiply-add). A slot whose row lives on another
GPU share has ``dst_row = -1`` and contributes nothing; a token with no local
slot gives a zero row. ``combine_exact`` is the same sum in fp64, the
reference the pages measure the error against, and ``combine_error_bound``
bounds the FP32 restore's distance from it a priori; ``restore_default`` is the
activation-dtype restore of section "Problem", kept for the error contrast
of section "Benchmark".
"""
from __future__ import annotations

import numpy as np

from . import bf16


def _coverage(dst, validate_coverage):
    if validate_coverage and (dst < 0).any():
        t, s = np.argwhere(dst < 0)[0]
        raise RuntimeError(f"(token {t}, slot {s}) is not covered by any expert row")


def combine(y, dst_row, topk_w, validate_coverage: bool = False) -> np.ndarray:
    """out [T, H] float32 (before the bf16 rounding): slots s with
    dst_row[t, s] >= 0 contribute topk_w[t, s] * y[dst_row[t, s]], the weight
    taken as fp32, product and running sum each rounded to fp32, slot order."""
    y32 = np.asarray(y).astype(np.float32)
    dst = np.asarray(dst_row, dtype=np.int64)
    w32 = np.asarray(topk_w).astype(np.float32)
    _coverage(dst, validate_coverage)
    T, k = dst.shape
    out = np.zeros((T, y32.shape[1]), dtype=np.float32)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        prod = w32[m, s][:, None] * y32[r[m]]  # fp32 products
        out[m] = out[m] + prod  # fp32 sums
    return out


def combine_bf16(y, dst_row, topk_w, validate_coverage: bool = False) -> np.ndarray:
    """The fused restore's output: the FP32 sum rounded once to bf16 (nearest
    even), returned as float64 values."""
    return bf16.round_to_bf16(combine(y, dst_row, topk_w, validate_coverage).astype(np.float64))


def combine_exact(y, dst_row, topk_w, validate_coverage: bool = False) -> np.ndarray:
    """The same weighted sum in fp64 (unrounded), the reference of the error
    figures."""
    y = np.asarray(y, dtype=np.float64)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    _coverage(dst, validate_coverage)
    T, k = dst.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        out[m] += w[m, s][:, None] * y[r[m]]
    return out


def combine_error_bound(y, dst_row, topk_w) -> np.ndarray:
    """A-priori bound [T, H] on |fused restore - exact sum|, fp64.

    The fused restore (section "Problem": FP32 accumulation; section
    "Benchmark": the error left against FP64 is the bf16 output rounding)
    forms n fp32 products and adds them in fp32, n being the token's local
    slots, then rounds once to bf16. Each product and each addition is one
    correctly rounded fp32 operation (unit roundoff u = 2^-24), so by the
    standard error analysis of a recursively summed dot product
    |fp32 sum - exact| <= gamma_n * sum_s |w_s y_s|, gamma_n = n u / (1 - n u),
    plus at most one fp32 subnormal spacing (2^-149) per product for
    underflow. The bf16 rounding adds at most half a bf16 unit of the fp32
    value, which lies within |exact| + that bound; half a unit at a value in
    [2^e, 2^(e+1)) is 2^(e-8), never below the subnormal half-spacing 2^-134.
    """
    y = np.asarray(y, dtype=np.float64)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(topk_w).astype(np.float32).astype(np.float64)
    T, k = dst.shape
    mag = np.zeros((T, y.shape[1]), dtype=np.float64)
    exact = np.zeros_like(mag)
    n = np.zeros(T, dtype=np.int64)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        p = w[m, s][:, None] * y[r[m]]
        exact[m] += p
        mag[m] += np.abs(p)
        n += m
    u = 2.0 ** -24
    gamma = (n * u / (1.0 - n * u))[:, None]
    fp32_err = gamma * mag + n[:, None] * 2.0 ** -149
    top = np.abs(exact) + fp32_err
    _, e = np.frexp(top)  # top = f * 2^e, 0.5 <= f < 1: top in [2^(e-1), 2^e)
    half_unit = np.ldexp(1.0, np.maximum(e.astype(np.int64) - 9, -134))
    return fp32_err + np.where(top > 0, half_unit, 0.0)


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


def combine_rows(y, dst_row, topk_w=None, shared=None, row_dtype: str = "bf16") -> np.ndarray:
    """The fused restore for other row dtypes and the variants the pages name,
    as float64 values of the returned rows.

    * Row dtype (DeepSpeed PR #8847, section "Tests": the fused restore runs on
      fp32 and on bf16 rows; section "Problem" and the fp16 note of the end-to-
      end test: in fp16 the default restore rounds each product and addition).
      Reading: the same FP32 slot-order sum as ``combine``, rounded once to the
      row dtype -- bf16 or fp16 nearest even, none for fp32 rows.
    * ``topk_w=None``: unit weights, the plain sum of a token's local rows
      (the routing score was applied before the experts, AutoEP's
      score_apply="pre" (same page, section "Change"), or the permute's
      backward).
    * ``shared``: rows [T, H] of a shared expert merged into the output (the
      last step of the AutoEP runtime, DeepSpeed AutoEP commit text, section
      "Design": merge shared experts if the model has them). Reading: added
      in fp32 after the routed sum, before the one rounding."""
    y32 = np.asarray(y).astype(np.float32)
    dst = np.asarray(dst_row, dtype=np.int64)
    T, k = dst.shape
    w32 = (np.ones((T, k), dtype=np.float32) if topk_w is None
           else np.asarray(topk_w).astype(np.float32))
    out = np.zeros((T, y32.shape[1]), dtype=np.float32)
    for s in range(k):
        r = dst[:, s]
        m = r >= 0
        out[m] = out[m] + w32[m, s][:, None] * y32[r[m]]
    if shared is not None:
        out = out + np.asarray(shared).astype(np.float32)
    if row_dtype == "fp32":
        return out.astype(np.float64)
    if row_dtype == "fp16":
        return out.astype(np.float16).astype(np.float64)
    if row_dtype == "bf16":
        return bf16.round_to_bf16(out.astype(np.float64))
    raise ValueError(f"unknown row dtype {row_dtype!r}")
