"""GPU parity of the backward calls (moe_combine_backward, moe_permute_backward,
moe_route_backward, and the expert calls moe_grouped_gate_up_save,
moe_grouped_down_backward, moe_grouped_gate_up_backward) against
oracle/backward.py and oracle/experts.py on the same seeded inputs.

Routing and layout come from the oracle (inputs never come from the HIP path);
expert outputs and gradients from ``workloads.gen``. Bars:
- row gradient (bf16 of the fp32 product) and permute gradient (fp32
  slot-order sum, one rounding): bit-exact; rows no slot points at keep what
  they held;
- score gradient: every entry within the error any fp32 summation order can
  make, (H-1) 2^-24 sum|G y|, exact zeros on slots of other shares, and over
  a whole workload a relative L2 error vs fp64 of the FP32 class the pages
  report (8.4e-8 at hidden 6144; held to <= 5e-7);
- routing gradient: within an fp32 bound of the fp64 formula, exact zeros on
  unselected experts;
- expert backward: the saved pre-activations, dg/du, dx_perm and the weight
  gradients dW1, dW3, dW2 within max|gpu - oracle| / max|oracle| <= 1e-2 of
  the fp64 calculus per expert group (the layer's bar: bf16 inputs, bf16 g/u/dg/du/dx roundings); the
  saving forward's h bit-equal to the plain forward's; rows outside the
  expert groups untouched.
Small shapes are checked in full; the DeepSeek-V3 share and the pages' restore
benchmark shape (8192 tokens, top-4 of 128 experts, hidden 6144) on all
scores and on sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from workloads import MoEConfig
from oracle import backward as ob, layout as olayout, route as oroute
from gpu_util import DEV, bits, f64, from_bits, i32

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

SHAPES = {
    "tiny": (workloads.get("tiny"), 1),
    "ragged": (MoEConfig(name="ragged_bwd", num_tokens=3000, hidden=384, num_experts=16, top_k=4,
                         inter=128, ep_size=4, local_rank=2, align=128), 2),
    "top1": (MoEConfig(name="top1_bwd", num_tokens=37, hidden=136, num_experts=4, top_k=1,
                       inter=128, align=16), -1),
    "wide": (MoEConfig(name="wide_bwd", num_tokens=256, hidden=128, num_experts=1024, top_k=16,
                       inter=128, align=128), -1),
    "odd_k": (MoEConfig(name="k3_bwd", num_tokens=501, hidden=264, num_experts=12, top_k=3,
                        inter=128, ep_size=3, local_rank=0, align=8), 0),
    "deepseek_share": (workloads.get("deepseek_v3_ep8_share"), 0),
    # the fused restore benchmark shape of the pages (8192 tokens per TP group,
    # top-4 of 128 experts, hidden 6144), all experts local
    "restore_k4": (MoEConfig(name="restore_k4", num_tokens=8192, hidden=6144, num_experts=128,
                             top_k=4, inter=128, align=1), -1),
}
FULL = {"tiny", "ragged", "top1", "wide", "odd_k"}
SENTINEL = 0x7FC1  # a NaN pattern no gradient row can produce here


def announce(*what):
    print("CASE", *what, flush=True)


def _inputs(name):
    cfg, share = SHAPES[name]
    _, logits = workloads.gen.routing_inputs(cfg, "balanced", 0, device="cpu")
    lg = logits.numpy()
    idx = oroute.select(lg, cfg.top_k)
    w = oroute.weights(lg, idx).astype(np.float32)
    L = olayout.layout(idx, cfg.num_experts, cfg.ep_size, share, cfg.align)
    rows = max(int(L["offsets"][-1]), 1)
    y = workloads.gen.expert_outputs(cfg, rows, 0, device="cpu")
    G = workloads.gen.output_gradient(cfg, 0, device="cpu")
    return cfg, share, idx, w, L, y, G


def _tokens(T, full, rng, n=384):
    return np.arange(T) if full else np.sort(rng.choice(T, size=min(n, T), replace=False))


@pytest.mark.parametrize("name", list(SHAPES))
def test_combine_backward(name):
    announce("combine_backward", name)
    cfg, share, idx, w, L, y, G = _inputs(name)
    dst = L["dst_row"]
    T, k = dst.shape
    rows = y.shape[0]
    gy = from_bits(np.full((rows, cfg.hidden), SENTINEL, dtype=np.uint16))
    gw = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    yd, Gd = y.to(DEV), G.to(DEV)
    moe.ops.combine_backward(Gd, yd, i32(dst), torch.from_numpy(w).to(DEV), gy, gw)
    torch.cuda.synchronize()

    y64, G64 = f64(y), f64(G)
    got_w = gw.cpu().numpy().astype(np.float64)
    exact = ob.combine_backward_scores(G64, y64, dst)
    bound = ob.score_bound(G64, y64, dst)
    local = dst >= 0
    assert (got_w[~local] == 0.0).all(), "slots of other shares must get a zero score gradient"
    err = np.abs(got_w - exact)
    assert (err <= bound + 1e-30).all(), float((err - bound).max())
    if local.any():
        rel = np.linalg.norm((got_w - exact)[local]) / np.linalg.norm(exact[local])
        assert rel <= 5e-7, rel

    rng = np.random.default_rng(7)
    toks = _tokens(T, name in FULL, rng)
    want, written = ob.combine_backward_rows(G64[toks], dst[toks], w[toks], rows)
    got = bits(gy)
    r_w = np.nonzero(written)[0]
    np.testing.assert_array_equal(got[r_w], bits(from_bits_host(want[r_w])))
    if name in FULL:
        untouched = np.ones(rows, dtype=bool)
        untouched[dst[dst >= 0]] = False
        assert (got[untouched] == SENTINEL).all(), "rows no slot points at must not be written"


def from_bits_host(vals: np.ndarray) -> torch.Tensor:
    """float64 values that are exact bf16 -> bf16 tensor on the host."""
    return torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("name", list(SHAPES))
def test_permute_backward(name):
    announce("permute_backward", name)
    cfg, share, idx, w, L, y, G = _inputs(name)
    dst = L["dst_row"]
    T = dst.shape[0]
    gp = y  # any bf16 rows serve as the gradient of x_perm
    gx = moe.ops.permute_backward(gp.to(DEV), i32(dst))
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    toks = _tokens(T, name in FULL, rng)
    want = ob.permute_backward_bf16(f64(gp), dst[toks])
    np.testing.assert_array_equal(bits(gx)[toks], bits(from_bits_host(want)))


@pytest.mark.parametrize("name", ["tiny", "top1", "wide", "odd_k", "deepseek_share"])
def test_route_backward(name):
    announce("route_backward", name)
    cfg, share, idx, w, L, y, G = _inputs(name)
    g = workloads.gen.score_gradient(cfg, 0).numpy()
    gl = moe.ops.route_backward(i32(idx), torch.from_numpy(w).to(DEV),
                                torch.from_numpy(g).to(DEV), cfg.num_experts)
    torch.cuda.synchronize()
    got = gl.cpu().numpy().astype(np.float64)
    want = ob.route_backward(idx, w.astype(np.float64), g.astype(np.float64), cfg.num_experts)
    sel = np.zeros_like(got, dtype=bool)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert (got[~sel] == 0.0).all()
    # fp32: the slot-order sum of k products (k+1 roundings) and one
    # subtraction and product (2 more), relative to the magnitudes involved
    w64, g64 = w.astype(np.float64), g.astype(np.float64)
    mag = np.abs(w64) * (np.abs(g64) + (cfg.top_k + 2) * (np.abs(w64 * g64)).sum(1, keepdims=True))
    bound = np.zeros_like(got)
    np.put_along_axis(bound, idx.astype(np.int64), 4 * 2.0 ** -24 * mag, axis=1)
    assert (np.abs(got - want) <= bound + 1e-37).all()


def test_backward_argument_checks_launch_nothing():
    lib = moe._lib.load()
    assert lib.moe_combine_backward(None, None, 0, None, None, 4, 7, 2, None, None, None) == 1
    assert lib.moe_permute_backward(None, 0, None, 4, 128, 17, None, None) == 1
    assert lib.moe_route_backward(None, None, None, 4, 8, 9, None, None) == 1
    # T * E past 2^32 entries is refused before any launch
    assert lib.moe_route_backward(None, None, None, 1 << 30, 16, 2, None, None) == 2


# ---------------------------------------------------------------- experts

from oracle import experts as oexperts  # noqa: E402

EXPERT_SHAPES = {
    # name: (config, local share, sample rows of at most this many experts)
    "tiny": (workloads.get("tiny"), 1, None),
    "small_h": (MoEConfig(name="small_h_bwd", num_tokens=600, hidden=384, num_experts=6,
                          top_k=2, inter=128, ep_size=2, local_rank=1, align=64), 1, None),
    "wide_i": (MoEConfig(name="wide_i_bwd", num_tokens=512, hidden=256, num_experts=4,
                         top_k=2, inter=640, align=32), -1, None),
    "deepseek_share": (workloads.get("deepseek_v3_ep8_share"), 0, 3),
    # ~1024 rows per expert: several 320-row m-tiles per expert on the 320x256
    # kinds (H and I multiples of 256), the last one short
    "tall": (MoEConfig(name="tall_bwd", num_tokens=2048, hidden=256, num_experts=4, top_k=2,
                       inter=256, align=128), -1, None),
    # the large DeepSeek-V3 layer (65536 tokens, all 256 experts local, severe
    # skew): inputs made on the device; the hottest expert (~20k rows, about
    # 60 row tiles walked in bands) and two others, checked on sampled rows
    # and sampled weight-gradient columns
    "deepseek_large": (workloads.get("deepseek_v3_large"), -1, 3),
    # 64 tokens, top-1 of 32 experts under severe skew: several experts get no
    # rows and must come back with zero weight gradients
    "empty_experts": (MoEConfig(name="empty_bwd", num_tokens=64, hidden=128, num_experts=32,
                                top_k=1, inter=128, align=16), -1, None),
    # row counts on the tile boundaries (given below, not routed): none, one,
    # the 64-row small-tile limit, one 320-row tile and one row past it, a
    # band of four row tiles plus one more; these counts are also the K
    # extents of the weight gradients
    "tile_edges": (MoEConfig(name="edges_bwd", num_tokens=3110, hidden=256, num_experts=11,
                             top_k=1, inter=256, align=128), -1, None),
}
EXPERT_COUNTS = {"tile_edges": [0, 1, 33, 63, 64, 65, 319, 320, 321, 641, 1283]}
EXPERT_DIST = {"empty_experts": "severe", "deepseek_large": "severe"}
ON_DEVICE = {"deepseek_large"}  # inputs too large to draw on the host
SAMPLE_ROWS = 4096  # groups larger than this are checked on sampled rows and columns
REL = 1e-2  # max|gpu - oracle| / max|oracle| per checked expert group


def _expert_inputs(name):
    cfg, share, sample = EXPERT_SHAPES[name]
    if name in EXPERT_COUNTS:
        counts = np.array(EXPERT_COUNTS[name])
        assert counts.size == cfg.num_experts and counts.sum() == cfg.num_tokens
        padded = (counts + cfg.align - 1) // cfg.align * cfg.align
        L = {"local_counts": counts, "offsets": np.concatenate([[0], np.cumsum(padded)])}
        m_cap = int(L["offsets"][-1]) + cfg.align  # a tail past the last group
    else:
        _, logits = workloads.gen.routing_inputs(cfg, EXPERT_DIST.get(name, "balanced"), 0,
                                                 device="cpu")
        idx = oroute.select(logits.numpy(), cfg.top_k)
        L = olayout.layout(idx, cfg.num_experts, cfg.ep_size, share, cfg.align)
        m_cap = cfg.m_cap(share)
    where = DEV if name in ON_DEVICE else "cpu"
    x_perm = workloads.gen.expert_outputs(cfg, m_cap, 1, device=where)  # stand-in rows
    dy = workloads.gen.expert_outputs(cfg, m_cap, 2, device=where)
    experts = list(cfg.local_experts(share))
    w1, w3, w2 = workloads.gen.expert_weights(cfg, experts, 0, device=where)
    return cfg, L, m_cap, x_perm, dy, (w1, w3, w2), sample


def _groups(L, sample):
    """Expert groups checked: all, or `sample` of them, the one with the most
    rows always among them."""
    counts = L["local_counts"]
    nz = [e for e in range(len(counts)) if counts[e] > 0]
    if sample is not None:
        rng = np.random.default_rng(5)
        top = int(np.argmax(counts))
        rest = [e for e in nz if e != top]
        nz = sorted([top] + rng.choice(rest, size=min(sample - 1, len(rest)),
                                       replace=False).tolist())
    return [(e, int(L["offsets"][e]), int(counts[e])) for e in nz]


def _sentinel_rows(rows, cols):
    return torch.full((rows, cols), SENTINEL, dtype=torch.int32, device=DEV).to(
        torch.int16).view(torch.bfloat16)


def _check_rows(r, c):
    """Rows of a group of c rows that are compared: all of them, or for a
    group past SAMPLE_ROWS one random row in every 80-row window plus the
    first and last, so that every row tile is sampled."""
    if c <= SAMPLE_ROWS:
        return np.arange(c)
    pick = {0, c - 1} | {int(r.integers(w0, min(w0 + 80, c))) for w0 in range(0, c, 80)}
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", list(EXPERT_SHAPES))
def test_expert_backward(name):
    announce("expert_backward", name)
    cfg, L, m_cap, x_perm, dy, (w1, w3, w2), sample = _expert_inputs(name)
    I = cfg.inter
    off_d, cnt_d = i32(L["offsets"]), i32(L["local_counts"])
    xd, dyd = x_perm.to(DEV), dy.to(DEV)
    w1d, w3d, w2d = w1.to(DEV), w3.to(DEV), w2.to(DEV)
    w1t, w3t = moe.ops.pack_weights(w1d), moe.ops.pack_weights(w3d)

    gu = _sentinel_rows(m_cap, 2 * I)
    dgu = _sentinel_rows(m_cap, 2 * I)
    dx = _sentinel_rows(m_cap, cfg.hidden)
    h, _ = moe.ops.grouped_gate_up_save(xd, off_d, cnt_d, w1t, w3t, gu=gu)
    h_plain = moe.ops.grouped_gate_up(xd, off_d, cnt_d, w1t, w3t)
    moe.ops.grouped_down_backward(dyd, gu, off_d, cnt_d, w2d, dgu=dgu)
    moe.ops.grouped_gate_up_backward(dgu, off_d, cnt_d, w1d, w3d, dx=dx)
    dw1, dw3 = moe.ops.grouped_gate_up_wgrad(xd, dgu, off_d, cnt_d)
    dw2 = moe.ops.grouped_down_wgrad(h, dyd, off_d, cnt_d)
    torch.cuda.synchronize()

    groups = _groups(L, sample)
    for _, a, c in groups:  # the saving forward computes h exactly as the plain one
        np.testing.assert_array_equal(bits(h[a:a + c]), bits(h_plain[a:a + c]))
    if sample is None:  # rows outside every expert group are never written
        rows = np.concatenate([np.arange(a, a + c) for _, a, c in groups])
        inside = np.zeros(m_cap, dtype=bool)
        inside[rows] = True
        gu_b, dgu_b, dx_b = bits(gu), bits(dgu), bits(dx)
        assert (gu_b[~inside] == SENTINEL).all() and (dgu_b[~inside] == SENTINEL).all()
        assert (dx_b[~inside] == SENTINEL).all()

    rng = np.random.default_rng(6)
    for e, a, c in groups:
        w1e, w3e, w2e = f64(w1[e]), f64(w3[e]), f64(w2[e])
        r = _check_rows(rng, c)
        rr = torch.as_tensor(a + r, device=DEV)
        xs, dys = f64(xd[rr]), f64(dyd[rr])
        gu_g, dgu_g = f64(gu[rr]), f64(dgu[rr])
        g = xs @ w1e
        u = xs @ w3e
        assert relmax(gu_g[:, :I], g) <= REL and relmax(gu_g[:, I:], u) <= REL
        s = 1.0 / (1.0 + np.exp(-g))
        dh = dys @ w2e.T
        assert relmax(dgu_g[:, :I], dh * u * (s * (1 + g * (1 - s)))) <= REL, e
        assert relmax(dgu_g[:, I:], dh * g * s) <= REL, e
        want, wd1, wd3, wd2 = oexperts.swiglu_backward(xs, w1e, w3e, w2e, dys)
        got = f64(dx[rr])
        assert relmax(got, want) <= REL, (e, relmax(got, want))
        if r.size < c:
            # weight gradients sum over every row of the group: check 64
            # sampled columns of the intermediate dimension in full. The
            # backward restricted to those columns of W1, W3 (and rows of W2)
            # gives exactly those columns of dW1, dW3 (and rows of dW2).
            cols = np.sort(rng.choice(I, 64, replace=False))
            xa, dya = f64(xd[a:a + c]), f64(dyd[a:a + c])
            _, wd1, wd3, wd2 = oexperts.swiglu_backward(xa, w1e[:, cols], w3e[:, cols],
                                                        w2e[cols, :], dya)
            ct = torch.as_tensor(cols, device=DEV)
            pairs = (("dW1", dw1[e][:, ct], wd1), ("dW3", dw3[e][:, ct], wd3),
                     ("dW2", dw2[e][ct, :], wd2))
        else:
            pairs = (("dW1", dw1[e], wd1), ("dW3", dw3[e], wd3), ("dW2", dw2[e], wd2))
        for name_, gpu, ref in pairs:
            rel = relmax(f64(gpu), ref)
            assert rel <= REL, (name_, e, rel)
    # experts without rows get exactly zero weight gradients
    if name == "empty_experts":
        assert (L["local_counts"] == 0).any()
    for e in np.nonzero(L["local_counts"] == 0)[0][:32]:
        for gpu in (dw1, dw3, dw2):
            assert not bits(gpu[int(e)]).any()


def obf16_decode(b):
    from oracle import bf16 as _b
    return _b.decode(b)


def relmax(got, want):
    den = np.abs(want).max()
    return float(np.abs(np.asarray(got, np.float64) - want).max() / (den if den > 0 else 1.0))
