"""The C ABI library loads and exports every entry point include/moe.h
declares; host-side argument checks reject bad calls before any launch.
Runs without a GPU: none of these calls reaches a kernel."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "combine_top_router_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def declared():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:const char\*|int32_t|int64_t|size_t)\s+(moe_\w+)\(", text, re.M)


def test_header_declares_the_five_stage_calls():
    names = set(declared())
    for n in ("moe_route", "moe_layout", "moe_permute", "moe_grouped_swiglu", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = C.CDLL(LIB)
    names = declared()
    assert len(names) == len(set(names)) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_the_header():
    from combine_top_router_amd import _lib
    assert set(_lib.SIGNATURES) == set(declared())


@pytest.fixture(scope="module")
def lib():
    from combine_top_router_amd import _lib
    return _lib.load()


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(4) == b"MOE_ERR_COVERAGE"
    assert lib.moe_status_string(99) == b"MOE_ERR_UNKNOWN"
    assert lib.moe_abi_version() == 2


def _desc(T, E, k, ep=1, lr=-1, align=128):
    from combine_top_router_amd._lib import LayoutDesc
    return LayoutDesc(T, E, k, ep, lr, align)


def test_m_cap_matches_the_worst_case_bound(lib):
    from oracle.layout import m_cap_bound
    for T, E, k, ep, lr, a in [(64, 8, 2, 2, -1, 128), (64, 8, 2, 2, 1, 128),
                               (8192, 256, 8, 8, 0, 128), (65536, 256, 8, 1, -1, 128),
                               (10, 4, 4, 1, -1, 1)]:
        assert lib.moe_layout_m_cap(C.byref(_desc(T, E, k, ep, lr, a))) == \
            m_cap_bound(T, E, k, ep, lr, a)
        assert lib.moe_layout_workspace_bytes(C.byref(_desc(T, E, k, ep, lr, a))) > 0


@pytest.mark.parametrize("bad", [
    dict(T=-1), dict(E=0), dict(E=1025), dict(k=0), dict(k=17), dict(T=10, ep=4),
    dict(E=10, ep=4), dict(lr=2, ep=2), dict(lr=-2), dict(align=3), dict(align=2048),
])
def test_bad_descriptors_are_rejected(lib, bad):
    p = dict(T=64, E=8, k=2, ep=1, lr=-1, align=128)
    p.update(bad)
    d = _desc(p["T"], p["E"], p["k"], p["ep"], p["lr"], p["align"])
    assert lib.moe_layout_m_cap(C.byref(d)) == -1
    assert lib.moe_layout_workspace_bytes(C.byref(d)) == 0
    fake = C.c_void_p(1 << 20)
    st = lib.moe_layout(C.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                        1 << 20, fake, 1 << 30, None)
    assert st == 1


def test_argument_checks_return_before_launch(lib):
    fake = C.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks
    odd = C.c_void_p((1 << 20) + 4)
    assert lib.moe_route(fake, 16, 8, 0, fake, fake, None) == 1          # k = 0
    assert lib.moe_route(fake, 16, 8, 9, fake, fake, None) == 1          # k > E
    assert lib.moe_route(None, 16, 8, 2, fake, fake, None) == 1          # null logits
    assert lib.moe_route(None, 0, 8, 2, None, None, None) == 0           # T = 0: no-op
    d = _desc(64, 8, 2)
    ws = lib.moe_layout_workspace_bytes(C.byref(d))
    m_cap = lib.moe_layout_m_cap(C.byref(d))
    args = [fake] * 9
    assert lib.moe_layout(C.byref(d), *args, m_cap - 1, fake, ws, None) == 1   # m_cap too small
    assert lib.moe_layout(C.byref(d), *args, m_cap, fake, ws - 1, None) == 1   # workspace small
    assert lib.moe_layout(C.byref(d), *args, m_cap, odd, ws, None) == 1        # misaligned ws
    assert lib.moe_permute(fake, 4, 12, 2, fake, fake, fake, 2, 8, fake, None) == 1  # H % 8
    assert lib.moe_permute(odd, 4, 16, 2, fake, fake, fake, 2, 8, fake, None) == 1   # misaligned x
    assert lib.moe_permute(fake, 4, 16, 2, fake, None, fake, 2, 8, fake, None) == 1  # no src_row
    assert lib.moe_permute(fake, 4, 16, 2, fake, fake, fake, 0, 8, fake, None) == 1  # E_loc = 0
    assert lib.moe_permute(None, 0, 16, 2, None, None, None, 2, 0, None, None) == 0  # m_cap 0
    assert lib.moe_combine(fake, 8, fake, fake, 4, 16, 0, fake, None) == 1      # k = 0
    assert lib.moe_combine(fake, 8, fake, fake, 4, 16, 2, odd, None) == 1       # misaligned out
    # GEMM shapes the kernels do not implement
    assert lib.moe_grouped_gate_up(fake, fake, fake, 4, 1024, 100 * 8, 256, fake, fake, fake,
                                   None) == 2
    assert lib.moe_grouped_down(fake, fake, fake, 4, 1024, 256, 136, fake, fake, None) == 2
    assert lib.moe_grouped_gate_up(fake, fake, fake, 0, 1024, 128, 256, fake, fake, fake,
                                   None) == 1
    assert lib.moe_pack_weights(fake, 2, 4, 4, fake, None) == 1                 # in place
    assert lib.moe_pack_weights(fake, 2, 64, 128, odd, None) == 2               # K % 128
    assert lib.moe_pack_weights(fake, 2, 128, 192, odd, None) == 2              # N % 128


def test_noalloc_layout_rejects_work_past_its_static_scratch(lib):
    # layout tiles grow with the assignment count (about 128 of them), so the
    # per-tile histograms fit the 4 MiB static array up to 2^30 assignments:
    # 2^20 tokens, top-16 of 1024 experts fits
    d = _desc(1 << 20, 1024, 16, 1, -1, 1)
    assert lib.moe_layout_workspace_bytes(C.byref(d)) <= 4 << 20
    # past 2^27 the tiles stop growing: ~2^31 assignments over 1024 experts
    # need 2048 tiles of histograms, 8 MiB, and are refused on the host, before
    # any device call
    T, E, k = (1 << 27) - 16, 1024, 16
    d = _desc(T, E, k, 1, -1, 1)
    assert lib.moe_layout_workspace_bytes(C.byref(d)) > 4 << 20
    m_cap = lib.moe_layout_m_cap(C.byref(d))
    fake = C.c_void_p(1 << 20)
    st = lib.moe_layout_noalloc(C.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                m_cap, None)
    assert st == 7 and lib.moe_status_string(st) == b"MOE_ERR_TOO_LARGE"
    # the checks moe_layout makes come first
    assert lib.moe_layout_noalloc(C.byref(d), fake, fake, fake, fake, fake, fake, fake, fake,
                                  fake, m_cap - 1, None) == 1
    assert lib.moe_layout_noalloc(C.byref(_desc(64, 8, 2)), fake, fake, fake, fake, fake, fake,
                                  None, fake, fake, 2000, None) == 1


def test_gate_up_gather_argument_checks_launch_nothing(lib):
    fake = C.c_void_p(1 << 20)
    odd = C.c_void_p((1 << 20) + 8)  # not 16-byte aligned
    args = lambda x, T, k, src, H: (x, T, k, src, fake, fake, 4, 1024, H, 256, fake, fake,  # noqa: E731
                                    fake, None)
    # shapes the kernels do not implement: H not a multiple of 128; token rows
    # past 32-bit byte offsets ((T + 1) * H * 2 >= 2^32)
    assert lib.moe_grouped_gate_up_gather(*args(fake, 64, 2, fake, 100 * 8)) == 2
    assert lib.moe_grouped_gate_up_gather(*args(fake, 1 << 20, 2, fake, 2048)) == 2
    # bad arguments: misaligned x, top_k out of range, missing src_row, negative T
    assert lib.moe_grouped_gate_up_gather(*args(odd, 64, 2, fake, 256)) == 1
    assert lib.moe_grouped_gate_up_gather(*args(fake, 64, 0, fake, 256)) == 1
    assert lib.moe_grouped_gate_up_gather(*args(fake, 64, 17, fake, 256)) == 1
    assert lib.moe_grouped_gate_up_gather(*args(fake, 64, 2, None, 256)) == 1
    assert lib.moe_grouped_gate_up_gather(*args(fake, -1, 2, fake, 256)) == 1
