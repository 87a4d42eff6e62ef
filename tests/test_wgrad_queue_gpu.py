"""Under skewed row counts the weight-gradient calls hand out tiles from a
per-stream device queue (after its first tile, a workgroup claims the next
unclaimed one). Which workgroup computes a tile then changes from launch to
launch, but each tile is still one workgroup's fixed-order sum, so every
launch must give the same bits. Checked here, on row counts skewed enough to
take the queue (the busiest workgroup of the fixed order would have over
twice the mean work) and more tiles than workgroups, for
consecutive calls on one stream (the queue left at zero by the last
workgroup), two streams at once (two queues), graph replays between eager
calls, and a stream past the library's queues (the static tile walk).
Agreement with the fp64 calculus is in test_backward_gpu.py."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import DEV, i32

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

H, I, ALIGN = 1024, 768, 128
# Zipf-like rows over 32 experts, including empty experts and a one-row one:
# dW1/dW3 make 24 tiles per expert (768), dW2 12 (384), past 256 workgroups
COUNTS = [1900, 1100, 700, 520, 400, 333, 260, 200, 170, 129, 128, 100, 90, 77, 64, 63,
          50, 41, 33, 30, 25, 20, 17, 12, 9, 5, 3, 1, 0, 0, 2, 7]
QUEUE_SLOTS = 64  # queues per GPU in the library; later streams walk statically


def _inputs():
    counts = np.asarray(COUNTS, np.int64)
    padded = (counts + ALIGN - 1) // ALIGN * ALIGN
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    m_cap = int(offsets[-1])
    g = torch.Generator(device=DEV).manual_seed(2024)
    x = torch.randn((m_cap, H), generator=g, device=DEV).to(torch.bfloat16)
    dgu = torch.randn((m_cap, 2 * I), generator=g, device=DEV).to(torch.bfloat16)
    h = torch.randn((m_cap, I), generator=g, device=DEV).to(torch.bfloat16)
    dy = torch.randn((m_cap, H), generator=g, device=DEV).to(torch.bfloat16)
    return x, dgu, h, dy, i32(offsets), i32(counts)


def _run(x, dgu, h, dy, off, cnt, outs=None):
    e = len(COUNTS)
    if outs is None:
        outs = [torch.empty((e, H, I), dtype=torch.bfloat16, device=DEV),
                torch.empty((e, H, I), dtype=torch.bfloat16, device=DEV),
                torch.empty((e, I, H), dtype=torch.bfloat16, device=DEV)]
    moe.ops.grouped_gate_up_wgrad(x, dgu, off, cnt, dw1=outs[0], dw3=outs[1])
    moe.ops.grouped_down_wgrad(h, dy, off, cnt, dw2=outs[2])
    return outs


def _same(a, b, what):
    for k, (p, q) in enumerate(zip(a, b)):  # bit patterns, compared on the device
        assert torch.equal(p.view(torch.int16), q.view(torch.int16)), f"{what}: output {k} differs"


def test_wgrad_same_bits_on_every_launch():
    torch.cuda.set_device(0)
    args = _inputs()
    ref = [t.clone() for t in _run(*args)]
    torch.cuda.synchronize()
    # consecutive calls on one stream reuse its queue
    for rep in range(3):
        _same(_run(*args), ref, f"call {rep + 2} on one stream")
    # empty experts come back as zero gradients
    for e in np.flatnonzero(np.asarray(COUNTS) == 0):
        assert not ref[0][e].any() and not ref[1][e].any() and not ref[2][e].any()

    # two side streams at once: each has a queue of its own
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        o1 = _run(*args)
    with torch.cuda.stream(s2):
        o2 = _run(*args)
    torch.cuda.synchronize()
    _same(o1, ref, "stream 1")
    _same(o2, ref, "stream 2")


def test_wgrad_graph_replays_between_eager_calls():
    torch.cuda.set_device(0)
    args = _inputs()
    ref = [t.clone() for t in _run(*args)]
    outs = [torch.empty_like(t) for t in ref]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream's queue lookup
        _run(*args, outs=outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _run(*args, outs=outs)
    for rep in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _same(outs, ref, f"replay {rep}")
        _same(_run(*args), ref, f"eager call after replay {rep}")
        torch.cuda.synchronize()


def _hip():
    import ctypes
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return lib


def test_wgrad_static_walk_past_the_queues():
    import ctypes
    torch.cuda.set_device(0)
    args = _inputs()
    ref = [t.clone() for t in _run(*args)]
    torch.cuda.synchronize()
    # more distinct streams than the library has queues (torch's own streams
    # come from a pool of 32, so these are made directly, at the default
    # priority): the later ones walk their tiles statically
    hip = _hip()
    handles = []
    try:
        for _ in range(QUEUE_SLOTS + 2):
            h = ctypes.c_void_p()
            assert hip.hipStreamCreate(ctypes.byref(h)) == 0
            handles.append(h.value)
        outs = [torch.empty_like(t) for t in ref]
        for k, h in enumerate(handles):
            for t in outs:
                t.zero_()
            s = torch.cuda.ExternalStream(h)
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                _run(*args, outs=outs)
            torch.cuda.current_stream().wait_stream(s)
            _same(outs, ref, f"stream {k}")
    finally:
        torch.cuda.synchronize()
        for h in handles:
            hip.hipStreamDestroy(h)
