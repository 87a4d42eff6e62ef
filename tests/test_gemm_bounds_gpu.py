"""Grouped GEMMs given device counts that run past the row buffers.

Every grouped-GEMM call takes m_cap, the number of rows of its row buffers,
and clamps each expert's rows to [offsets[e], m_cap): a stale layout or the
wrong slice of expert_counts must not move a read or a write past the
buffers. The buffers here are twice m_cap long (views of their first m_cap
rows are passed), so the rows at and past m_cap are memory the call must not
touch but can reach without leaving the allocation; they hold a sentinel that
must survive. The rows inside [offsets[e], m_cap) come out as for an expert of
that many rows (oracle: fp64 SwiGLU and its calculus, max|gpu - oracle| /
max|oracle| <= 1e-2)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import bf16 as obf16, experts as oexperts
from gpu_util import DEV, bits, f64, from_bits, i32, rel_max

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

SENTINEL = 0x7FC1
H, I, M_CAP = 256, 256, 384
# expert 0: 100 rows at 0; expert 1: 1000 rows claimed at 128, clamped to the
# 256 rows [128, 384); expert 2: a negative offset, clamped to no rows
OFFSETS = [0, 128, -64, 384]
COUNTS = [100, 1000, 50]
ROWS = [(0, 100), (128, 256)]  # (first row, rows) each expert really has


def _sentinel(rows, cols):
    return torch.full((rows, cols), SENTINEL, dtype=torch.int32, device=DEV).to(
        torch.int16).view(torch.bfloat16)


def _weights(rng, e):
    w1 = obf16.round_to_bf16(rng.standard_normal((e, H, I)) / np.sqrt(H))
    w3 = obf16.round_to_bf16(rng.standard_normal((e, H, I)) / np.sqrt(H))
    w2 = obf16.round_to_bf16(rng.standard_normal((e, I, H)) / np.sqrt(I))
    return w1, w3, w2


def test_forward_rows_past_m_cap_untouched():
    print("CASE gemm bounds forward", flush=True)
    rng = np.random.default_rng(31)
    w1, w3, w2 = _weights(rng, 3)
    x = obf16.round_to_bf16(rng.standard_normal((2 * M_CAP, H)))
    xd = from_bits(obf16.encode(x))
    off, cnt = i32(OFFSETS), i32(COUNTS)
    w1t, w3t, w2t = (moe.pack_weights(from_bits(obf16.encode(w))) for w in (w1, w3, w2))
    h, y = _sentinel(2 * M_CAP, I), _sentinel(2 * M_CAP, H)
    moe.grouped_swiglu(xd[:M_CAP], off, cnt, w1t, w3t, w2t, h=h[:M_CAP], out=y[:M_CAP])
    torch.cuda.synchronize()
    assert (bits(h[M_CAP:]) == SENTINEL).all() and (bits(y[M_CAP:]) == SENTINEL).all()
    for e, (a, c) in enumerate(ROWS):
        want = oexperts.swiglu(x[a:a + c], w1[e], w3[e], w2[e])
        assert rel_max(f64(y[a:a + c]), want) <= 1e-2, e
    # rows of no expert (100..127) are not written either
    assert (bits(y[100:128]) == SENTINEL).all()


def test_backward_rows_past_m_cap_untouched():
    print("CASE gemm bounds backward", flush=True)
    rng = np.random.default_rng(32)
    w1, w3, w2 = _weights(rng, 3)
    x = obf16.round_to_bf16(rng.standard_normal((2 * M_CAP, H)))
    dy = obf16.round_to_bf16(rng.standard_normal((2 * M_CAP, H)))
    xd, dyd = from_bits(obf16.encode(x)), from_bits(obf16.encode(dy))
    w1d, w3d, w2d = (from_bits(obf16.encode(w)) for w in (w1, w3, w2))
    off, cnt = i32(OFFSETS), i32(COUNTS)
    gu, dgu = _sentinel(2 * M_CAP, 2 * I), _sentinel(2 * M_CAP, 2 * I)
    dx = _sentinel(2 * M_CAP, H)
    h = _sentinel(2 * M_CAP, I)
    ops = moe.ops
    ops.grouped_gate_up_save(xd[:M_CAP], off, cnt, ops.pack_weights(w1d), ops.pack_weights(w3d),
                             h=h[:M_CAP], gu=gu[:M_CAP])
    ops.grouped_down_backward(dyd[:M_CAP], gu[:M_CAP], off, cnt, w2d, dgu=dgu[:M_CAP])
    ops.grouped_gate_up_backward(dgu[:M_CAP], off, cnt, w1d, w3d, dx=dx[:M_CAP])
    dw1, dw3 = ops.grouped_gate_up_wgrad(xd[:M_CAP], dgu[:M_CAP], off, cnt)
    dw2 = ops.grouped_down_wgrad(h[:M_CAP], dyd[:M_CAP], off, cnt)
    torch.cuda.synchronize()
    for t in (gu, dgu, dx, h):
        assert (bits(t[M_CAP:]) == SENTINEL).all()
    for e, (a, c) in enumerate(ROWS):
        want, wd1, wd3, wd2 = oexperts.swiglu_backward(x[a:a + c], w1[e], w3[e], w2[e],
                                                       dy[a:a + c])
        assert rel_max(f64(dx[a:a + c]), want) <= 1e-2, e
        for gpu, ref in ((dw1[e], wd1), (dw3[e], wd3), (dw2[e], wd2)):
            assert rel_max(f64(gpu), ref) <= 1e-2, e
    # the expert clamped to no rows gets zero weight gradients
    for gpu in (dw1[2], dw3[2], dw2[2]):
        assert not bits(gpu).any()
