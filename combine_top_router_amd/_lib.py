"""ctypes view of libmoe.so (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_HIP",
          4: "MOE_ERR_COVERAGE", 5: "MOE_ERR_EXPERT_ID", 6: "MOE_ERR_LAYOUT"}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        name = STATUS.get(status, f"status {status}")
        super().__init__(f"{fn} returned {name}" + (f": {detail}" if detail else ""))


class LayoutDesc(C.Structure):
    _fields_ = [("num_tokens", C.c_int64), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("ep_size", C.c_int32), ("local_rank", C.c_int32), ("align", C.c_int32)]


_P = C.c_void_p
_I32, _I64, _SZ = C.c_int32, C.c_int64, C.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [_I32]),
    "moe_abi_version": (_I32, []),
    "moe_route": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_layout_m_cap": (_I64, [C.POINTER(LayoutDesc)]),
    "moe_layout_workspace_bytes": (_SZ, [C.POINTER(LayoutDesc)]),
    "moe_layout": (_I32, [C.POINTER(LayoutDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _P,
                          _SZ, _P]),
    "moe_layout_noalloc": (_I32, [C.POINTER(LayoutDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _I64, _P]),
    "moe_dispatch_layout_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32]),
    "moe_dispatch_layout": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _I32, _I64, _P, _P]),
    "moe_permute_weighted": (_I32, [_P, _I64, _I32, _I32, _P, _P, _I64, _P, _P]),
    "moe_combine_rows": (_I32, [_P, _I32, _I64, _P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_pack_weights": (_I32, [_P, _I64, _I32, _I32, _P, _P]),
    "moe_grouped_gate_up": (_I32, [_P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P, _P]),
    "moe_grouped_gate_up_gather": (_I32, [_P, _I64, _I32, _P, _P, _P, _I32, _I64, _I32, _I32,
                                          _P, _P, _P, _P]),
    "moe_grouped_down": (_I32, [_P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P]),
    "moe_grouped_swiglu": (_I32, [_P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_gate_up_save": (_I32, [_P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_grouped_down_backward": (_I32, [_P, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P]),
    "moe_grouped_gate_up_backward": (_I32, [_P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P, _P]),
    "moe_grouped_gate_up_wgrad": (_I32, [_P, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P]),
    "moe_grouped_down_wgrad": (_I32, [_P, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P]),
    "moe_combine": (_I32, [_P, _I64, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_combine_backward": (_I32, [_P, _P, _I64, _P, _P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_permute_backward": (_I32, [_P, _I64, _P, _I64, _I32, _I32, _P, _P]),
    "moe_route_backward": (_I32, [_P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_validate_layout": (_I32, [C.POINTER(LayoutDesc), _P, _P, _P, _P, _I64, _P, C.c_char_p,
                                   _SZ]),
}


def load(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m combine_top_router_amd.build` "
            "(hipcc, gfx950). There is no CPU or fallback path.")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def check(fn: str, status: int, detail: str = "") -> None:
    if status != MOE_OK:
        raise MoEError(fn, status, detail)
