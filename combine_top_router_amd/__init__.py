"""combine_top_router_amd: the single-GPU MoE-layer hot path on AMD MI355X.

    route -> layout -> permute -> grouped SwiGLU experts -> fused weighted combine

Every stage is a hand-written HIP kernel for gfx950 in ``libmoe.so`` behind the
C ABI of ``include/moe.h``; this package is its PyTorch binding (``ops``) and
a preallocated one-GPU layer pipeline (``layer.MoELayer``). Build the library
with ``python -m combine_top_router_amd.build``.
"""
from ._lib import LIB_PATH, MoEError, lib  # noqa: F401
from .ops import (  # noqa: F401
    Layout, alloc_layout, combine, grouped_down, grouped_gate_up, grouped_gate_up_gather,
    grouped_swiglu, layout,
    layout_desc, layout_m_cap, layout_workspace_bytes, pack_weights, permute, route,
    validate_layout,
)
from .layer import MoELayer  # noqa: F401
