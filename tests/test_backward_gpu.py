"""GPU parity of the backward calls (moe_combine_backward, moe_permute_backward,
moe_route_backward) against oracle/backward.py on the same seeded inputs.

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
  unselected experts.
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
