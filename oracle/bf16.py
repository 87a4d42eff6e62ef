"""bfloat16 encoding for the oracle: decode stored bits exactly, round fp64
values to the nearest bf16 (ties to even) in one step.

bf16 is the activation and expert-weight dtype of the grouped-GEMM path
(DeepSpeed PR #8847 "AutoEP: support combine_impl=fused_weighted_sum ...",
section "Tests": torch._grouped_mm takes bf16 only) and the row dtype of the
fused restore's benchmark (same page, section "Benchmark": bf16 rows, FP32
routing weights). A bf16 number has 1 sign bit, fp32's 8 exponent bits and
7 stored significand bits (8 significant bits).
"""
from __future__ import annotations

import numpy as np

# largest finite bf16: (2 - 2**-7) * 2**127
BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))


def decode(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each fp64 input, ties to even, as float64.

    With x = m * 2**e (0.5 <= |m| < 1), the bf16 spacing at x is 2**(e-8),
    floored at the subnormal spacing 2**-133. Scaling by the spacing, rounding
    to the nearest integer (numpy's rint breaks ties to even) and scaling back
    is one correctly rounded step, with no intermediate fp32 rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)


def encode(x) -> np.ndarray:
    """fp64 values -> uint16 bits of their bf16 rounding (ties to even)."""
    r = round_to_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
