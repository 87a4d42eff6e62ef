"""Thin PyTorch binding of libmoe: argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of
the path runs in the library's HIP kernels. Each function checks that its
tensors live on the GPU with the dtype and layout the C ABI expects, hands
raw pointers to the library, and raises ``MoEError`` on a non-OK status.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from ._lib import LayoutDesc, MoEError, check, lib


def _stream(dev: torch.device):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _empty(shape, dtype, dev):
    return torch.empty(shape, dtype=dtype, device=dev)


# ---------------------------------------------------------------- route

def route(logits: torch.Tensor, top_k: int, topk_idx=None, topk_w=None):
    """(topk_idx [T, k] int32, topk_w [T, k] float32) from logits [T, E] fp32."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    topk_idx = _empty((T, top_k), torch.int32, dev) if topk_idx is None else topk_idx
    topk_w = _empty((T, top_k), torch.float32, dev) if topk_w is None else topk_w
    _need(topk_idx, "topk_idx", torch.int32, (T, top_k))
    _need(topk_w, "topk_w", torch.float32, (T, top_k))
    check("moe_route", lib().moe_route(_ptr(logits), T, E, top_k, _ptr(topk_idx), _ptr(topk_w),
                                       _stream(dev)))
    return topk_idx, topk_w


# ---------------------------------------------------------------- layout

def layout_desc(num_tokens, num_experts, top_k, ep_size=1, local_rank=-1, align=128) -> LayoutDesc:
    return LayoutDesc(num_tokens, num_experts, top_k, ep_size, local_rank, align)


def layout_m_cap(desc: LayoutDesc) -> int:
    m = lib().moe_layout_m_cap(C.byref(desc))
    if m < 0:
        raise MoEError("moe_layout_m_cap", 1, "invalid layout descriptor")
    return int(m)


def layout_workspace_bytes(desc: LayoutDesc) -> int:
    return int(lib().moe_layout_workspace_bytes(C.byref(desc)))


@dataclass
class Layout:
    desc: LayoutDesc
    m_cap: int
    first_local: int
    num_local: int
    expert_counts: torch.Tensor  # [E]
    send_counts: torch.Tensor    # [ep, E]
    split_matrix: torch.Tensor   # [ep, ep]
    recv_counts: torch.Tensor    # [ep, E_loc]
    output_splits: torch.Tensor  # [ep]
    offsets: torch.Tensor        # [E_loc + 1]
    dst_row: torch.Tensor        # [T, k]
    src_row: torch.Tensor        # [m_cap]
    workspace: torch.Tensor      # bytes

    @property
    def local_counts(self) -> torch.Tensor:
        return self.expert_counts[self.first_local:self.first_local + self.num_local]


def alloc_layout(desc: LayoutDesc, device, m_cap=None, workspace: bool = True) -> Layout:
    T, E, k, ep = desc.num_tokens, desc.num_experts, desc.top_k, desc.ep_size
    first = 0 if desc.local_rank < 0 else desc.local_rank * (E // ep)
    el = E if desc.local_rank < 0 else E // ep
    m_cap = layout_m_cap(desc) if m_cap is None else m_cap
    i32 = torch.int32
    return Layout(desc, m_cap, first, el,
                  _empty((E,), i32, device), _empty((ep, E), i32, device),
                  _empty((ep, ep), i32, device), _empty((ep, el), i32, device),
                  _empty((ep,), i32, device), _empty((el + 1,), i32, device),
                  _empty((T, k), i32, device), _empty((m_cap,), i32, device),
                  _empty((max(layout_workspace_bytes(desc) if workspace else 0, 16),),
                         torch.uint8, device))


def layout(topk_idx: torch.Tensor, num_experts: int, ep_size: int = 1, local_rank: int = -1,
           align: int = 128, out: Layout | None = None) -> Layout:
    """Histogram, split plan, padded offsets and stable permutation (no host sync)."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    desc = layout_desc(T, num_experts, k, ep_size, local_rank, align)
    L = alloc_layout(desc, topk_idx.device) if out is None else out
    check("moe_layout", lib().moe_layout(
        C.byref(desc), _ptr(topk_idx), _ptr(L.expert_counts), _ptr(L.send_counts),
        _ptr(L.split_matrix), _ptr(L.recv_counts), _ptr(L.output_splits), _ptr(L.offsets),
        _ptr(L.dst_row), _ptr(L.src_row), L.m_cap, _ptr(L.workspace), L.workspace.numel(),
        _stream(topk_idx.device)))
    return L


def layout_noalloc(topk_idx: torch.Tensor, num_experts: int, ep_size: int = 1,
                   local_rank: int = -1, align: int = 128, out: Layout | None = None) -> Layout:
    """As ``layout``, through moe_layout_noalloc: the library's static scratch
    array serves as the workspace, so the call allocates nothing (``out``,
    when given, holds every output; its workspace is not used)."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    desc = layout_desc(T, num_experts, k, ep_size, local_rank, align)
    L = alloc_layout(desc, topk_idx.device, workspace=False) if out is None else out
    check("moe_layout_noalloc", lib().moe_layout_noalloc(
        C.byref(desc), _ptr(topk_idx), _ptr(L.expert_counts), _ptr(L.send_counts),
        _ptr(L.split_matrix), _ptr(L.recv_counts), _ptr(L.output_splits), _ptr(L.offsets),
        _ptr(L.dst_row), _ptr(L.src_row), L.m_cap, _stream(topk_idx.device)))
    return L


def validate_layout(topk_idx: torch.Tensor, L: Layout) -> None:
    """Debug check (synchronises): raises MoEError naming the first violation."""
    buf = C.create_string_buffer(256)
    st = lib().moe_validate_layout(C.byref(L.desc), _ptr(topk_idx), _ptr(L.offsets),
                                   _ptr(L.dst_row), _ptr(L.src_row), L.m_cap,
                                   _stream(topk_idx.device), buf, 256)
    check("moe_validate_layout", st, buf.value.decode())


# ---------------------------------------------------------------- permute

def permute(x: torch.Tensor, dst_row: torch.Tensor, src_row: torch.Tensor,
            offsets: torch.Tensor, m_cap: int, out=None) -> torch.Tensor:
    """x_perm [m_cap, H] bf16: row dst_row[t, s] holds x[t]; padding rows of the
    expert groups (src_row < 0 below offsets[E_loc]) zero; rows from
    offsets[E_loc] on untouched."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    _need(dst_row, "dst_row", torch.int32)
    _need(src_row, "src_row", torch.int32, (m_cap,))
    _need(offsets, "offsets", torch.int32)
    k = dst_row.shape[1]
    e_loc = offsets.numel() - 1
    out = _empty((m_cap, H), torch.bfloat16, x.device) if out is None else out
    _need(out, "x_perm", torch.bfloat16, (m_cap, H))
    check("moe_permute", lib().moe_permute(_ptr(x), T, H, k, _ptr(dst_row), _ptr(src_row),
                                           _ptr(offsets), e_loc, m_cap, _ptr(out),
                                           _stream(x.device)))
    return out


# ---------------------------------------------------------------- experts

def pack_weights(w: torch.Tensor, out=None) -> torch.Tensor:
    """Math-orientation [n, K, N] bf16 matrices -> the packed layout the forward
    grouped GEMMs read (moe_pack_weights): output-major, N rows in blocks of 256
    (128 if N % 256), each block stored as K/64 contiguous [block][64] slices.
    Returned with shape [n, N, K]; only its element order differs from the
    plain transpose."""
    _need(w, "w", torch.bfloat16)
    n, R, Cc = w.shape
    out = _empty((n, Cc, R), torch.bfloat16, w.device) if out is None else out
    _need(out, "wt", torch.bfloat16, (n, Cc, R))
    check("moe_pack_weights", lib().moe_pack_weights(_ptr(w), n, R, Cc, _ptr(out),
                                                     _stream(w.device)))
    return out


def _gemm_common(a, offsets, counts):
    _need(a, "activations", torch.bfloat16)
    _need(offsets, "offsets", torch.int32)
    if counts.dtype != torch.int32 or counts.device.type != "cuda" or not counts.is_contiguous():
        raise TypeError("counts must be a contiguous int32 GPU tensor")
    return offsets.numel() - 1


def grouped_gate_up(x_perm, offsets, counts, w1t, w3t, out=None):
    """h = silu(x W1) * (x W3) per local expert group; w1t/w3t are W1/W3 [E_loc, H, I]
    after pack_weights (shape [E_loc, I, H])."""
    e_loc = _gemm_common(x_perm, offsets, counts)
    m_cap, H = x_perm.shape
    I = w1t.shape[1]
    _need(w1t, "w1t", torch.bfloat16, (e_loc, I, H))
    _need(w3t, "w3t", torch.bfloat16, (e_loc, I, H))
    out = _empty((m_cap, I), torch.bfloat16, x_perm.device) if out is None else out
    _need(out, "h", torch.bfloat16, (m_cap, I))
    check("moe_grouped_gate_up", lib().moe_grouped_gate_up(
        _ptr(x_perm), _ptr(offsets), _ptr(counts), e_loc, m_cap, H, I, _ptr(w1t), _ptr(w3t),
        _ptr(out), _stream(x_perm.device)))
    return out


def grouped_gate_up_gather(x, src_row, top_k, offsets, counts, w1t, w3t, out=None):
    """h as grouped_gate_up, its rows read straight from the token rows x [T, H]:
    grouped row r is x[src_row[r] // top_k] (the permute fused into the GEMM's
    loads); h has src_row's length."""
    e_loc = _gemm_common(x, offsets, counts)
    _need(src_row, "src_row", torch.int32)
    T, H = x.shape
    m_cap = src_row.numel()
    I = w1t.shape[1]
    _need(w1t, "w1t", torch.bfloat16, (e_loc, I, H))
    _need(w3t, "w3t", torch.bfloat16, (e_loc, I, H))
    out = _empty((m_cap, I), torch.bfloat16, x.device) if out is None else out
    _need(out, "h", torch.bfloat16, (m_cap, I))
    check("moe_grouped_gate_up_gather", lib().moe_grouped_gate_up_gather(
        _ptr(x), T, top_k, _ptr(src_row), _ptr(offsets), _ptr(counts), e_loc, m_cap, H, I,
        _ptr(w1t), _ptr(w3t), _ptr(out), _stream(x.device)))
    return out


def grouped_down(h, offsets, counts, w2t, out=None):
    """y = h W2 per local expert group; w2t is W2 [E_loc, I, H] after pack_weights
    (shape [E_loc, H, I])."""
    e_loc = _gemm_common(h, offsets, counts)
    m_cap, I = h.shape
    H = w2t.shape[1]
    _need(w2t, "w2t", torch.bfloat16, (e_loc, H, I))
    out = _empty((m_cap, H), torch.bfloat16, h.device) if out is None else out
    _need(out, "y", torch.bfloat16, (m_cap, H))
    check("moe_grouped_down", lib().moe_grouped_down(
        _ptr(h), _ptr(offsets), _ptr(counts), e_loc, m_cap, I, H, _ptr(w2t), _ptr(out),
        _stream(h.device)))
    return out


def grouped_swiglu(x_perm, offsets, counts, w1t, w3t, w2t, h=None, out=None):
    """y = (silu(x W1) * (x W3)) W2 per local expert group, through workspace h."""
    e_loc = _gemm_common(x_perm, offsets, counts)
    m_cap, H = x_perm.shape
    I = w1t.shape[1]
    _need(w1t, "w1t", torch.bfloat16, (e_loc, I, H))
    _need(w3t, "w3t", torch.bfloat16, (e_loc, I, H))
    _need(w2t, "w2t", torch.bfloat16, (e_loc, H, I))
    h = _empty((m_cap, I), torch.bfloat16, x_perm.device) if h is None else h
    out = _empty((m_cap, H), torch.bfloat16, x_perm.device) if out is None else out
    _need(h, "h", torch.bfloat16, (m_cap, I))
    _need(out, "y", torch.bfloat16, (m_cap, H))
    check("moe_grouped_swiglu", lib().moe_grouped_swiglu(
        _ptr(x_perm), _ptr(offsets), _ptr(counts), e_loc, m_cap, H, I, _ptr(w1t), _ptr(w3t),
        _ptr(w2t), _ptr(h), _ptr(out), _stream(x_perm.device)))
    return out


# ---------------------------------------------------------------- combine

def combine(y: torch.Tensor, dst_row: torch.Tensor, topk_w: torch.Tensor, out=None):
    """out [T, H] bf16 = sum_s topk_w[t, s] * y[dst_row[t, s]] (fp32 accumulate)."""
    _need(y, "y", torch.bfloat16)
    _need(dst_row, "dst_row", torch.int32)
    T, k = dst_row.shape
    _need(topk_w, "topk_w", torch.float32, (T, k))
    H = y.shape[1]
    out = _empty((T, H), torch.bfloat16, y.device) if out is None else out
    _need(out, "out", torch.bfloat16, (T, H))
    check("moe_combine", lib().moe_combine(_ptr(y), y.shape[0], _ptr(dst_row), _ptr(topk_w), T,
                                           H, k, _ptr(out), _stream(y.device)))
    return out


# ---------------------------------------------------------------- backward

def combine_backward(grad_out: torch.Tensor, y: torch.Tensor, dst_row: torch.Tensor,
                     topk_w: torch.Tensor, grad_y=None, grad_w=None):
    """(grad_y [y_rows, H] bf16, grad_w [T, k] fp32): the row gradient
    bf16(w * G) written to each local row, the score gradient <G[t], y[r]>
    (0 for slots on other shares). Rows no slot points at are left as given."""
    _need(grad_out, "grad_out", torch.bfloat16)
    _need(y, "y", torch.bfloat16)
    _need(dst_row, "dst_row", torch.int32)
    T, k = dst_row.shape
    H = grad_out.shape[1]
    _need(topk_w, "topk_w", torch.float32, (T, k))
    _need(grad_out, "grad_out", torch.bfloat16, (T, H))
    _need(y, "y", torch.bfloat16, (y.shape[0], H))
    grad_y = _empty(tuple(y.shape), torch.bfloat16, y.device) if grad_y is None else grad_y
    grad_w = _empty((T, k), torch.float32, y.device) if grad_w is None else grad_w
    _need(grad_y, "grad_y", torch.bfloat16, tuple(y.shape))
    _need(grad_w, "grad_w", torch.float32, (T, k))
    check("moe_combine_backward", lib().moe_combine_backward(
        _ptr(grad_out), _ptr(y), y.shape[0], _ptr(dst_row), _ptr(topk_w), T, H, k,
        _ptr(grad_y), _ptr(grad_w), _stream(y.device)))
    return grad_y, grad_w


def permute_backward(grad_x_perm: torch.Tensor, dst_row: torch.Tensor, out=None):
    """grad_x [T, H] bf16: per token, the fp32 slot-order sum of its local row
    gradients, rounded once (zero row without a local slot)."""
    _need(grad_x_perm, "grad_x_perm", torch.bfloat16)
    _need(dst_row, "dst_row", torch.int32)
    T, k = dst_row.shape
    H = grad_x_perm.shape[1]
    out = _empty((T, H), torch.bfloat16, grad_x_perm.device) if out is None else out
    _need(out, "grad_x", torch.bfloat16, (T, H))
    check("moe_permute_backward", lib().moe_permute_backward(
        _ptr(grad_x_perm), grad_x_perm.shape[0], _ptr(dst_row), T, H, k, _ptr(out),
        _stream(out.device)))
    return out


def route_backward(topk_idx: torch.Tensor, topk_w: torch.Tensor, grad_w: torch.Tensor,
                   num_experts: int, out=None):
    """grad_logits [T, E] fp32: w_j (g_j - sum_i w_i g_i) at the selected
    experts, zero elsewhere."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    _need(topk_w, "topk_w", torch.float32, (T, k))
    _need(grad_w, "grad_w", torch.float32, (T, k))
    out = _empty((T, num_experts), torch.float32, topk_idx.device) if out is None else out
    _need(out, "grad_logits", torch.float32, (T, num_experts))
    check("moe_route_backward", lib().moe_route_backward(
        _ptr(topk_idx), _ptr(topk_w), _ptr(grad_w), T, num_experts, k, _ptr(out),
        _stream(out.device)))
    return out


def grouped_gate_up_save(x_perm, offsets, counts, w1t, w3t, h=None, gu=None):
    """(h, gu): h as grouped_gate_up, and gu [m_cap, 2I] = [x W1 | x W3] in bf16
    for the backward."""
    e_loc = _gemm_common(x_perm, offsets, counts)
    m_cap, H = x_perm.shape
    I = w1t.shape[1]
    _need(w1t, "w1t", torch.bfloat16, (e_loc, I, H))
    _need(w3t, "w3t", torch.bfloat16, (e_loc, I, H))
    h = _empty((m_cap, I), torch.bfloat16, x_perm.device) if h is None else h
    gu = _empty((m_cap, 2 * I), torch.bfloat16, x_perm.device) if gu is None else gu
    _need(h, "h", torch.bfloat16, (m_cap, I))
    _need(gu, "gu", torch.bfloat16, (m_cap, 2 * I))
    check("moe_grouped_gate_up_save", lib().moe_grouped_gate_up_save(
        _ptr(x_perm), _ptr(offsets), _ptr(counts), e_loc, m_cap, H, I, _ptr(w1t), _ptr(w3t),
        _ptr(h), _ptr(gu), _stream(x_perm.device)))
    return h, gu


def grouped_down_backward(dy, gu, offsets, counts, w2, dgu=None):
    """dgu [m_cap, 2I] = [dh u silu'(g) | dh silu(g)] with dh = dy W2^T; w2 is
    the math-orientation [E_loc, I, H]."""
    e_loc = _gemm_common(dy, offsets, counts)
    m_cap, H = dy.shape
    I = w2.shape[1]
    _need(w2, "w2", torch.bfloat16, (e_loc, I, H))
    _need(gu, "gu", torch.bfloat16, (m_cap, 2 * I))
    dgu = _empty((m_cap, 2 * I), torch.bfloat16, dy.device) if dgu is None else dgu
    _need(dgu, "dgu", torch.bfloat16, (m_cap, 2 * I))
    check("moe_grouped_down_backward", lib().moe_grouped_down_backward(
        _ptr(dy), _ptr(gu), _ptr(offsets), _ptr(counts), e_loc, m_cap, I, H, _ptr(w2), _ptr(dgu),
        _stream(dy.device)))
    return dgu


def grouped_gate_up_backward(dgu, offsets, counts, w1, w3, dx=None):
    """dx_perm [m_cap, H] = dg W1^T + du W3^T; w1, w3 are the math-orientation
    [E_loc, H, I]."""
    e_loc = _gemm_common(dgu, offsets, counts)
    m_cap, I2 = dgu.shape
    I = I2 // 2
    H = w1.shape[1]
    _need(w1, "w1", torch.bfloat16, (e_loc, H, I))
    _need(w3, "w3", torch.bfloat16, (e_loc, H, I))
    dx = _empty((m_cap, H), torch.bfloat16, dgu.device) if dx is None else dx
    _need(dx, "dx_perm", torch.bfloat16, (m_cap, H))
    check("moe_grouped_gate_up_backward", lib().moe_grouped_gate_up_backward(
        _ptr(dgu), _ptr(offsets), _ptr(counts), e_loc, m_cap, H, I, _ptr(w1), _ptr(w3), _ptr(dx),
        _stream(dgu.device)))
    return dx


def grouped_gate_up_wgrad(x_perm, dgu, offsets, counts, dw1=None, dw3=None):
    """(dW1, dW3) [E_loc, H, I] bf16: x_perm_e^T dg_e and x_perm_e^T du_e."""
    e_loc = _gemm_common(x_perm, offsets, counts)
    m_cap, H = x_perm.shape
    I = dgu.shape[1] // 2
    _need(dgu, "dgu", torch.bfloat16, (m_cap, 2 * I))
    dw1 = _empty((e_loc, H, I), torch.bfloat16, x_perm.device) if dw1 is None else dw1
    dw3 = _empty((e_loc, H, I), torch.bfloat16, x_perm.device) if dw3 is None else dw3
    _need(dw1, "dw1", torch.bfloat16, (e_loc, H, I))
    _need(dw3, "dw3", torch.bfloat16, (e_loc, H, I))
    check("moe_grouped_gate_up_wgrad", lib().moe_grouped_gate_up_wgrad(
        _ptr(x_perm), _ptr(dgu), _ptr(offsets), _ptr(counts), e_loc, m_cap, H, I, _ptr(dw1),
        _ptr(dw3), _stream(x_perm.device)))
    return dw1, dw3


def grouped_down_wgrad(h, dy, offsets, counts, dw2=None):
    """dW2 [E_loc, I, H] bf16: h_e^T dy_e."""
    e_loc = _gemm_common(h, offsets, counts)
    m_cap, I = h.shape
    H = dy.shape[1]
    _need(dy, "dy", torch.bfloat16, (m_cap, H))
    dw2 = _empty((e_loc, I, H), torch.bfloat16, h.device) if dw2 is None else dw2
    _need(dw2, "dw2", torch.bfloat16, (e_loc, I, H))
    check("moe_grouped_down_wgrad", lib().moe_grouped_down_wgrad(
        _ptr(h), _ptr(dy), _ptr(offsets), _ptr(counts), e_loc, m_cap, I, H, _ptr(dw2),
        _stream(h.device)))
    return dw2


# ---------------------------------------------------------------- dedup layout

def dispatch_layout(topk_idx: torch.Tensor, num_experts: int, ep_size: int):
    """DeepEP-style per-rank layout: (num_tokens_per_rank [ep], num_tokens_per_expert [E],
    is_token_in_rank [T, ep] uint8, token_rank_pos [T, ep] int32)."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    dev = topk_idx.device
    ws_bytes = int(lib().moe_dispatch_layout_workspace_bytes(T, num_experts, k, ep_size))
    if ws_bytes == 0 and T > 0:
        raise MoEError("moe_dispatch_layout_workspace_bytes", 1, "invalid sizes")
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    per_rank = _empty((ep_size,), torch.int32, dev)
    per_expert = _empty((num_experts,), torch.int32, dev)
    in_rank = _empty((T, ep_size), torch.uint8, dev)
    pos = _empty((T, ep_size), torch.int32, dev)
    check("moe_dispatch_layout", lib().moe_dispatch_layout(
        _ptr(topk_idx), T, num_experts, k, ep_size, _ptr(per_rank), _ptr(per_expert),
        _ptr(in_rank), _ptr(pos), _ptr(ws), ws.numel(), _stream(dev)))
    return per_rank, per_expert, in_rank, pos


# ---------------------------------------------------------------- variants

_ROWS = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}


def permute_weighted(x: torch.Tensor, dst_row: torch.Tensor, topk_w: torch.Tensor, m_cap: int,
                     out=None) -> torch.Tensor:
    """x_perm with the routing score applied before the experts:
    row dst_row[t, s] = bf16(w[t, s] * x[t])."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    _need(dst_row, "dst_row", torch.int32)
    k = dst_row.shape[1]
    _need(topk_w, "topk_w", torch.float32, (T, k))
    out = _empty((m_cap, H), torch.bfloat16, x.device) if out is None else out
    _need(out, "x_perm", torch.bfloat16, (m_cap, H))
    check("moe_permute_weighted", lib().moe_permute_weighted(
        _ptr(x), T, H, k, _ptr(dst_row), _ptr(topk_w), m_cap, _ptr(out), _stream(x.device)))
    return out


def combine_rows(y: torch.Tensor, dst_row: torch.Tensor, topk_w=None, shared=None, out=None):
    """The fused restore on bf16 / fp16 / fp32 rows: fp32 slot-order sum of
    w * y (w = 1 without weights), plus the shared expert's rows if given,
    rounded once to the row dtype."""
    if y.dtype not in _ROWS:
        raise TypeError(f"y must be bf16, fp16 or fp32 (got {y.dtype})")
    _need(y, "y", y.dtype)
    _need(dst_row, "dst_row", torch.int32)
    T, k = dst_row.shape
    H = y.shape[1]
    if topk_w is not None:
        _need(topk_w, "topk_w", torch.float32, (T, k))
    if shared is not None:
        _need(shared, "shared", y.dtype, (T, H))
    out = _empty((T, H), y.dtype, y.device) if out is None else out
    _need(out, "out", y.dtype, (T, H))
    check("moe_combine_rows", lib().moe_combine_rows(
        _ptr(y), _ROWS[y.dtype], y.shape[0], _ptr(dst_row),
        _ptr(topk_w) if topk_w is not None else None,
        _ptr(shared) if shared is not None else None, T, H, k, _ptr(out), _stream(y.device)))
    return out
