"""Seeded synthetic inputs for the MoE-layer workloads.

Value recipe (the same for every configuration):

* activations ``x ~ N(0, 1)``, drawn in fp32 and rounded to bf16;
* router projection ``Wr ~ N(0, 1/H)`` (variance 1/H), fp32;
* router logits ``x_bf16 @ Wr + b`` in fp32, where ``b`` is the per-expert
  routing bias of the distribution (below);
* expert matrices, math orientation: gate ``W1[e]`` and up ``W3[e]`` are
  ``[H, I]`` with entries ``N(0, 1/H)``, down ``W2[e]`` is ``[I, H]`` with
  entries ``N(0, 1/I)``; drawn in fp32, rounded to bf16.

Routing distributions (bias added to the logits):

* ``balanced``: no bias;
* ``mild``: one ``N(0, 0.5)`` draw per expert (variance 0.5);
* ``severe``: +3 on 16 hot experts, the first 16 of a seeded permutation;
* ``zipf``: ``-1.2 * ln(1 + pi(e))`` for a seeded permutation ``pi``, so the
  softmax prior of an expert falls off as its rank to the power -1.2.

Every tensor has its own seed, derived from (configuration, tensor name,
distribution, expert index, base seed), so one expert's weights do not
depend on how many experts are generated next to it. Large tensors are drawn
on the device that asks for them with ``torch.Generator``; the same call on
another device gives other (equally distributed) values, so a test always
hands one generated tensor to both implementations.

This module only draws random numbers and forms the logits; it contains none
of the routing, layout, permute, expert or combine arithmetic.
"""
from __future__ import annotations

import hashlib
import math

import torch

from .configs import MoEConfig

HOT_EXPERTS = 16
SEVERE_BIAS = 3.0
MILD_VAR = 0.5
ZIPF_S = 1.2


def seed_of(*parts) -> int:
    """Stable 63-bit seed from any printable parts."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def _randn(shape, std, device, *parts) -> torch.Tensor:
    g = _gen(device, *parts)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def routing_bias(cfg: MoEConfig, dist: str, seed: int = 0) -> torch.Tensor:
    """Per-expert logit bias [E] (fp32, CPU) of a routing distribution."""
    E = cfg.num_experts
    if dist == "balanced":
        return torch.zeros(E, dtype=torch.float32)
    g = _gen("cpu", cfg.name, "bias", dist, seed)
    if dist == "mild":
        return torch.randn(E, generator=g, dtype=torch.float32) * math.sqrt(MILD_VAR)
    perm = torch.randperm(E, generator=g)
    if dist == "severe":
        b = torch.zeros(E, dtype=torch.float32)
        b[perm[:HOT_EXPERTS]] = SEVERE_BIAS
        return b
    if dist == "zipf":
        rank = torch.empty(E, dtype=torch.float64)
        rank[perm] = torch.arange(E, dtype=torch.float64)
        return (-ZIPF_S * torch.log1p(rank)).to(torch.float32)
    raise ValueError(f"unknown routing distribution {dist!r}")


def routing_inputs(cfg: MoEConfig, dist: str, seed: int = 0, device="cpu"):
    """Returns ``x`` [T, H] bf16 and ``logits`` [T, E] fp32 on ``device``."""
    T, H, E = cfg.num_tokens, cfg.hidden, cfg.num_experts
    x = _randn((T, H), 1.0, device, cfg.name, "x", seed).to(torch.bfloat16)
    wr = _randn((H, E), 1.0 / math.sqrt(H), device, cfg.name, "wr", seed)
    logits = x.float() @ wr
    logits += routing_bias(cfg, dist, seed).to(device)
    return x, logits.contiguous()


def expert_weights(cfg: MoEConfig, experts, seed: int = 0, device="cpu"):
    """Math-orientation expert matrices for the listed global expert ids:
    ``w1, w3`` [n, H, I] and ``w2`` [n, I, H], bf16 on ``device``."""
    H, I = cfg.hidden, cfg.inter
    experts = list(experts)
    n = len(experts)
    w1 = torch.empty((n, H, I), dtype=torch.bfloat16, device=device)
    w3 = torch.empty((n, H, I), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((n, I, H), dtype=torch.bfloat16, device=device)
    for j, e in enumerate(experts):
        w1[j] = _randn((H, I), 1.0 / math.sqrt(H), device, cfg.name, "w1", e, seed)
        w3[j] = _randn((H, I), 1.0 / math.sqrt(H), device, cfg.name, "w3", e, seed)
        w2[j] = _randn((I, H), 1.0 / math.sqrt(I), device, cfg.name, "w2", e, seed)
    return w1, w3, w2


def expert_outputs(cfg: MoEConfig, rows: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Stand-in expert outputs ``y`` [rows, H] bf16, N(0, 1), for exercising the
    combine on its own."""
    return _randn((rows, cfg.hidden), 1.0, device, cfg.name, "y", seed).to(torch.bfloat16)


def output_gradient(cfg: MoEConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    """Stand-in gradient of the layer output ``G`` [T, H] bf16, N(0, 1), for
    the backward steps."""
    return _randn((cfg.num_tokens, cfg.hidden), 1.0, device, cfg.name, "grad_out",
                  seed).to(torch.bfloat16)


def score_gradient(cfg: MoEConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    """Stand-in gradient of the routing weights [T, k] fp32, N(0, 1)."""
    return _randn((cfg.num_tokens, cfg.top_k), 1.0, device, cfg.name, "grad_w", seed)


def random_rows(cfg: MoEConfig, rows: int, dtype: torch.dtype, seed: int = 0,
                device="cpu") -> torch.Tensor:
    """Rows [rows, H] of N(0, 1) values in ``dtype`` (fp32 rows keep all 24
    bits), for exercising the row movers on their own."""
    return _randn((rows, cfg.hidden), 1.0, device, cfg.name, "rows", str(dtype), seed).to(dtype)
