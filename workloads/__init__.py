"""Synthetic MoE-layer workloads: shapes (``configs``) and seeded inputs (``gen``).

Shared by the tests, the benchmark and the smoke check; imported by neither
the oracle nor the HIP library."""
from .configs import CONFIGS, CONFIG_ORDER, MoEConfig, get  # noqa: F401
from . import gen  # noqa: F401
