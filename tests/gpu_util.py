"""Helpers of the GPU parity tests: tensor conversion, seeded inputs on the
device, and the oracle run on the same inputs. Inputs come from
``workloads.gen``; expected values come from ``oracle`` only."""
from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import bf16 as obf16

DEV = "cuda"


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> exact float64 values (host)."""
    return obf16.decode(bits(t))


def from_bits(a: np.ndarray, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def i32(a, device=DEV) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def rel_max(got, want) -> float:
    """max |got - want| / max |want| (the full-layer criterion)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.abs(want).max()
    return float(np.abs(got - want).max() / (den if den > 0 else 1.0))


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between two bit arrays
    (sign-magnitude mapped onto a monotone integer line; +0 and -0 coincide)."""
    def line(b):
        b = b.astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(line(a_bits) - line(b_bits))


class Case:
    """One workload instance on the GPU, with the math-orientation expert
    weights of the local experts and their oracle views."""

    def __init__(self, cfg, dist="balanced", local_rank=None, seed=0, weights=True):
        self.cfg = cfg
        self.dist = dist
        self.local_rank = cfg.local_rank if local_rank is None else local_rank
        self.x, self.logits = workloads.gen.routing_inputs(cfg, dist, seed, device=DEV)
        self.experts = list(cfg.local_experts(self.local_rank))
        self.first = self.experts[0]
        self.num_local = len(self.experts)
        self.w1 = self.w3 = self.w2 = None
        if weights:
            self.w1, self.w3, self.w2 = workloads.gen.expert_weights(cfg, self.experts, seed,
                                                                     device=DEV)
        self._wcache = {}

    def weights_of(self, e_local: int):
        """Oracle view (float64 host arrays) of local expert e's matrices."""
        if e_local not in self._wcache:
            if len(self._wcache) > 8:
                self._wcache.clear()
            self._wcache[e_local] = (f64(self.w1[e_local]), f64(self.w3[e_local]),
                                     f64(self.w2[e_local]))
        return self._wcache[e_local]

    def logits_np(self):
        return self.logits.cpu().numpy()

    def x_np(self):
        return f64(self.x)
