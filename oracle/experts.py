"""Local expert compute (oracle): one SwiGLU MLP per local expert over its
contiguous group of rows.

The AutoEP runtime runs local grouped expert compute over the rows grouped
per expert (DeepSpeed AutoEP commit text, section "Attribution":
ep_experts.py from TorchTitan's GroupedExperts / grouped-GEMM execution;
section "Design", runtime step 5), with expert weights ``w1, w2, w3`` in a
grouped layout (section "Adding new model support": expert_w1/w2/w3).

Reading (pages silent on the MLP): Mixtral/LLaMA naming, W1 = gate [H, I],
W3 = up [H, I], W2 = down [I, H]; ``h = silu(x W1) * (x W3)`` with
``silu(a) = a * sigmoid(a) = a / (1 + exp(-a))``; ``y = h W2``. All in
fp64 on the bf16 input values; h is not rounded.
"""
from __future__ import annotations

import numpy as np


def silu(a):
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu(x, w1, w3, w2) -> np.ndarray:
    """y [m, H] for rows x [m, H] of one expert (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(w1, dtype=np.float64)
    u = x @ np.asarray(w3, dtype=np.float64)
    return (silu(g) * u) @ np.asarray(w2, dtype=np.float64)


def grouped_swiglu(x_perm, offsets, counts, weights_of) -> np.ndarray:
    """y for every local row: rows ``[offsets[e], offsets[e] + counts[e])``
    go through expert e, whose matrices ``weights_of(e)`` returns as
    (w1, w3, w2). Padding rows stay zero."""
    x_perm = np.asarray(x_perm, dtype=np.float64)
    y = np.zeros_like(x_perm)  # the down projection maps back to width H
    for e, c in enumerate(counts):
        c = int(c)
        if c == 0:
            continue
        a = int(offsets[e])
        y[a:a + c] = swiglu(x_perm[a:a + c], *weights_of(e))
    return y


def swiglu_backward(x, w1, w3, w2, dy):
    """Gradients of ``y = (silu(x W1) * (x W3)) W2`` for one expert, fp64 from
    the definition (nothing rounded in between). Training runs this backward
    through the grouped-GEMM path and returns the expert gradients in BF16
    (xtuner PR #2056 "Integrate MoonEP dispatcher ...", section "Summary");
    the formulas are the plain calculus of the forward above:

        g = x W1, u = x W3, h = silu(g) * u
        dh = dy W2^T
        dg = dh * u * silu'(g),  silu'(g) = s (1 + g (1 - s)),  s = sigmoid(g)
        du = dh * silu(g)
        dx = dg W1^T + du W3^T
        dW1 = x^T dg,  dW3 = x^T du,  dW2 = h^T dy

    Returns (dx [m, H], dw1 [H, I], dw3 [H, I], dw2 [I, H])."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w3 = np.asarray(w3, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    g = x @ w1
    u = x @ w3
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    h = g * s * u
    dh = dy @ w2.T
    dg = dh * u * (s * (1.0 + g * (1.0 - s)))
    du = dh * g * s
    dx = dg @ w1.T + du @ w3.T
    return dx, x.T @ dg, x.T @ du, h.T @ dy


def grouped_swiglu_backward_data(x_perm, dy, offsets, counts, weights_of) -> np.ndarray:
    """dx_perm for every local row (the data gradient of ``grouped_swiglu``);
    padding rows stay zero."""
    x_perm = np.asarray(x_perm, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    dx = np.zeros_like(x_perm)
    for e, c in enumerate(counts):
        c = int(c)
        if c == 0:
            continue
        a = int(offsets[e])
        dx[a:a + c] = swiglu_backward(x_perm[a:a + c], *weights_of(e), dy[a:a + c])[0]
    return dx
