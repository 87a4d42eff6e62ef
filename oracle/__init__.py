"""CPU oracle of the single-GPU MoE-layer path: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation (fp64 wherever the
method does floating point) of what the HIP library computes:

  route    -> ``oracle.route``     token-choice top-k routing
  layout   -> ``oracle.layout``    histogram, split plan, padded offsets, stable permutation
  permute  -> ``oracle.permute``   expert-major row gather
  experts  -> ``oracle.experts``   per-expert SwiGLU MLP
  combine  -> ``oracle.combine``   weighted un-permute, fp32 slot-order sums, one bf16 rounding
  layer    -> ``oracle.layer``     the composition, and per-token outputs for sampling
  backward -> ``oracle.backward``  gradients of route, permute and combine

It shares no code with the HIP path and imports nothing from it. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it;
the product path never does.

Pinned by ``tests/test_oracle_*.py`` against a hand-computed worked example
(``tests/golden/``), closed forms, brute force on tiny inputs and the
invariants the pages state. Parity unpinned: nothing (every function has at
least one pin that does not re-run its own formula).
"""
from . import backward, bf16, checks, combine, experts, layer, layout, permute, route  # noqa: F401
