"""GPU parity: every stage of the HIP path, called through the C ABI (via the
ctypes binding), against the CPU oracle on the same seeded inputs.

Bars: bit-exact for topk_idx, counts, splits, offsets, dst_row, src_row and
permuted rows; routing weights within 1e-6; the combine within 1 bf16 ulp of
the oracle's FP32 combine given the same expert outputs (in fact bit-exact:
both sides do the same fp32 operations in the same order), and within the
a-priori error bound of an FP32 restore against the fp64 sum; expert outputs and
the whole layer within max|gpu - oracle| / max|oracle| <= 1e-2 of the fp64
oracle.

Small workloads are compared element by element in full; the large ones
(the Mixtral-, Qwen3-MoE- and DeepSeek-V3-shaped layers, in the same launch
configuration the benchmark times) on rows and tokens sampled with a fixed
seed, plus the integer outputs in full.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from workloads import MoEConfig
from oracle import bf16 as obf16, checks, combine as ocombine, experts as oexperts
from oracle import layer as olayer, layout as olayout, permute as opermute, route as oroute

from gpu_util import Case, bits, f64, from_bits, i32, rel_max, ulp_distance

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("combine_top_router_amd")

# extra shapes: ragged tails, several layout tiles per rank, edge cases
EXTRA = {
    "ragged": MoEConfig(name="ragged", num_tokens=3000, hidden=384, num_experts=16, top_k=4,
                        inter=256, ep_size=4, local_rank=2, align=128,
                        dists=("mild",), shares=(-1, 2)),
    "top1_odd": MoEConfig(name="top1_odd", num_tokens=37, hidden=128, num_experts=4, top_k=1,
                          inter=128, ep_size=1, local_rank=-1, align=16),
    "wide": MoEConfig(name="wide", num_tokens=256, hidden=128, num_experts=1024, top_k=16,
                      inter=128, ep_size=1, local_rank=-1, align=128, dists=("zipf",)),
    # just under the single-workgroup layout limit (4096 assignments), ragged
    "fused_edge": MoEConfig(name="fused_edge", num_tokens=1020, hidden=128, num_experts=32,
                            top_k=4, inter=128, ep_size=4, local_rank=3, align=32,
                            dists=("severe",), shares=(3,)),
    # 160000 assignments: several layout tiles per source rank
    "tiled": MoEConfig(name="tiled", num_tokens=40000, hidden=128, num_experts=64, top_k=4,
                       inter=128, ep_size=2, local_rank=1, align=64, dists=("mild",),
                       shares=(1,)),
}


def cfg_of(name):
    return EXTRA[name] if name in EXTRA else workloads.get(name)


FULL = {"tiny", "ragged", "top1_odd", "wide", "tiled", "fused_edge"}  # oracle runs these whole

CASES = [("tiny", "balanced", s) for s in (-1, 0, 1)]
CASES += [("ragged", "mild", -1), ("ragged", "mild", 2), ("top1_odd", "balanced", -1),
          ("wide", "zipf", -1), ("tiled", "mild", 1), ("tiled", "mild", -1),
          ("fused_edge", "severe", 3), ("fused_edge", "severe", -1)]
CASES += [("mixtral_8x7b", "balanced", -1), ("qwen3_30b_a3b", "zipf", -1)]
CASES += [("deepseek_v3_ep8_share", d, 0) for d in ("balanced", "mild", "severe")]
CASES += [("deepseek_v3_large", "severe", -1)]
IDS = [f"{c}-{d}-r{s}" for c, d, s in CASES]


def announce(*what):
    print("CASE", *what, flush=True)


_case_cache = {}


def get_case(name, dist, share, weights=True):
    key = (name, dist, share, weights)
    if key not in _case_cache:
        _case_cache.clear()
        torch.cuda.empty_cache()
        _case_cache[key] = Case(cfg_of(name), dist, share, weights=weights)
    return _case_cache[key]


_oracle_cache = {}


def oracle_routing(case):
    key = (case.cfg.name, case.dist, case.local_rank)
    if key not in _oracle_cache:
        _oracle_cache.clear()
        cfg = case.cfg
        idx, w = oroute.route(case.logits_np(), cfg.top_k)
        L = olayout.layout(idx, cfg.num_experts, cfg.ep_size, case.local_rank, cfg.align,
                           cfg.m_cap(case.local_rank))
        _oracle_cache[key] = (idx, w, L)
    return _oracle_cache[key]


# ---------------------------------------------------------------- route

@pytest.mark.parametrize("name,dist,share", CASES, ids=IDS)
def test_route(name, dist, share):
    announce("route", name, dist, share)
    case = get_case(name, dist, share, weights=False)
    idx, w = moe.route(case.logits, case.cfg.top_k)
    want_idx, want_w = oracle_routing(case)[:2]
    got_idx = idx.cpu().numpy()
    assert (got_idx == want_idx).all(), np.argwhere(got_idx != want_idx)[:5]
    assert np.abs(w.cpu().numpy() - want_w).max() <= 1e-6


def test_route_ties_and_signed_zero():
    announce("route ties")
    logits = np.array([[3, 1, 2, 0], [0, 0, 5, 5], [1, 4, 0, 4], [2, 0, 2, 0],
                       [-0.0, 0.0, -1, -1], [0.0, -0.0, -1, -1]], np.float32)
    idx, w = moe.route(torch.from_numpy(logits).cuda(), 2)
    want_idx, want_w = oroute.route(logits, 2)
    assert (idx.cpu().numpy() == want_idx).all()
    assert np.abs(w.cpu().numpy() - want_w).max() <= 1e-6


def test_route_equal_logits_and_k_equals_e():
    announce("route equal logits")
    logits = torch.full((5, 16), 0.5, device="cuda")
    idx, w = moe.route(logits, 16)
    assert (idx.cpu().numpy() == np.arange(16)).all()
    assert np.abs(w.cpu().numpy() - 1 / 16).max() <= 1e-7


# ---------------------------------------------------------------- layout

LAYOUT_KEYS = ("expert_counts", "send_counts", "split_matrix", "recv_counts", "output_splits",
               "offsets", "dst_row", "src_row")


@pytest.mark.parametrize("name,dist,share", CASES, ids=IDS)
def test_layout(name, dist, share):
    announce("layout", name, dist, share)
    case = get_case(name, dist, share, weights=False)
    cfg = case.cfg
    idx, _, want = oracle_routing(case)
    idx_d = i32(idx)
    L = moe.layout(idx_d, cfg.num_experts, cfg.ep_size, share, cfg.align)
    assert L.m_cap == want["m_cap"]
    for k in LAYOUT_KEYS:
        got = getattr(L, k).cpu().numpy()
        assert (got == want[k]).all(), (k, np.argwhere(got != want[k])[:5])
    moe.validate_layout(idx_d, L)


def test_layout_every_share_covers_each_slot_once():
    announce("layout coverage over shares")
    cfg = workloads.get("deepseek_v3_ep8_share")
    case = get_case(cfg.name, "severe", 0, weights=False)
    idx = moe.route(case.logits, cfg.top_k)[0]
    dsts = []
    for d in range(cfg.ep_size):
        L = moe.layout(idx, cfg.num_experts, cfg.ep_size, d, cfg.align)
        moe.validate_layout(idx, L)
        dsts.append(L.dst_row.cpu().numpy())
        assert (L.split_matrix[:, d] == L.output_splits).all()
    checks.check_coverage(dsts, cfg.num_tokens, cfg.top_k)


def test_layout_zero_tokens():
    announce("layout T=0")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    L = moe.layout(idx, 8, 1, -1, 128)
    assert (L.offsets.cpu() == 0).all() and (L.expert_counts.cpu() == 0).all()
    assert (L.src_row.cpu() == -1).all()


def test_layout_all_to_one_expert():
    announce("layout one hot expert")
    T, k, E = 5000, 1, 64
    idx = np.full((T, k), 7, np.int32)
    want = olayout.layout(idx, E, 1, -1, 128)
    L = moe.layout(i32(idx), E, 1, -1, 128)
    for key in LAYOUT_KEYS:
        assert (getattr(L, key).cpu().numpy() == want[key]).all(), key


@pytest.mark.parametrize("T,ep,share", [(1 << 19, 1, -1), (1 << 21, 8, 3)])
def test_layout_tiles_walked_in_several_passes(T, ep, share):
    """4 M and 16 M assignments (top-8 of 256 experts): tiles of 16384 and 65536
    assignments, each placed in several passes with every expert's next row
    carried from pass to pass. Distinct ids per token, skewed toward low
    experts (43 of the 256 get nothing)."""
    announce("layout multi-pass", T, ep, share)
    k, E = 8, 256
    rng = np.random.default_rng(7)
    first = (rng.pareto(1.5, T) * 20).astype(np.int64) % (3 * E // 4)
    idx = ((first[:, None] + np.arange(k)[None, :] * 3) % E).astype(np.int32)
    want = olayout.layout(idx, E, ep, share, 128)
    L = moe.layout(i32(idx), E, ep, share, 128)
    assert L.m_cap == want["m_cap"]
    for key in LAYOUT_KEYS:
        got = getattr(L, key).cpu().numpy()
        assert (got == want[key]).all(), (key, np.argwhere(got != want[key])[:5])


def test_validator_reports_bad_input():
    announce("validator")
    idx = np.array([[0, 1], [1, 2], [2, 3], [3, 0]], np.int32)
    L = moe.layout(i32(idx), 4, 1, -1, 4)
    moe.validate_layout(i32(idx), L)
    bad = idx.copy()
    bad[2, 1] = 9  # out of range: the layout skips it, the validator names it
    with pytest.raises(moe.MoEError, match="EXPERT_ID"):
        moe.validate_layout(i32(bad), moe.layout(i32(bad), 4, 1, -1, 4))
    dup = idx.copy()
    dup[1, 1] = 1  # a token repeating an expert
    with pytest.raises(moe.MoEError, match="EXPERT_ID"):
        moe.validate_layout(i32(dup), moe.layout(i32(dup), 4, 1, -1, 4))
    L.dst_row[3, 0] = -1  # drop one (token, slot): uncovered
    with pytest.raises(moe.MoEError, match="COVERAGE"):
        moe.validate_layout(i32(idx), L)


# ---------------------------------------------------------------- permute

def _sample_rows(L, rng, n=2048):
    rows = np.nonzero(L["src_row"] >= 0)[0]
    if rows.size > n:
        rows = np.sort(np.concatenate([rng.choice(rows, n - 2, replace=False),
                                       rows[[0, -1]]]))
    return rows


@pytest.mark.parametrize("name,dist,share", CASES, ids=IDS)
def test_permute(name, dist, share):
    announce("permute", name, dist, share)
    case = get_case(name, dist, share, weights=False)
    cfg = case.cfg
    idx, _, L = oracle_routing(case)
    sentinel = 0x7FC1  # a NaN pattern: padding rows must keep it
    xp = torch.full((L["m_cap"], cfg.hidden), 0, dtype=torch.int16, device="cuda")
    xp.fill_(sentinel)
    xp = xp.view(torch.bfloat16)
    moe.permute(case.x, i32(L["dst_row"]), i32(L["src_row"]), i32(L["offsets"]), L["m_cap"],
                out=xp)
    rng = np.random.default_rng(0)
    rows = _sample_rows(L, rng) if name not in FULL else np.nonzero(L["src_row"] >= 0)[0]
    want = opermute.permute(bits(case.x), L["src_row"], cfg.top_k, rows)
    got = bits(xp[torch.as_tensor(rows, device="cuda")])
    assert (got == want).all()
    # padding rows of the groups come back as zeros (the oracle's value), rows
    # past the last group keep what they held
    n_grp = int(L["offsets"][-1])
    pad = np.nonzero(L["src_row"][:n_grp] < 0)[0]
    if pad.size:
        pad = pad if name in FULL else pad[rng.choice(pad.size, min(pad.size, 4096), replace=False)]
        want_pad = opermute.permute(bits(case.x), L["src_row"], cfg.top_k, pad)
        assert (bits(xp[torch.as_tensor(pad, device="cuda")]) == want_pad).all()
        assert not want_pad.any()
    tail = np.arange(n_grp, min(L["m_cap"], n_grp + 512))
    if tail.size:
        assert (bits(xp[torch.as_tensor(tail, device="cuda")]) == sentinel).all()


def test_permute_padding_without_tokens():
    """No token rows to copy, only padding: groups given by hand (three
    experts, 5, 0 and 3 rows padded to 8) with src_row -1 on the padding rows
    and on two rows no token fills; those rows come back zero, the rest of
    x_perm keeps its sentinel."""
    announce("permute padding only")
    H, k, m_cap = 136, 2, 40
    offsets = np.array([0, 8, 8, 16], np.int32)
    src = np.full(m_cap, -1, np.int32)
    src[[0, 1, 2, 3, 4, 8, 9, 10]] = [0, 1, 2, 3, 4, 5, 6, 7]  # rows the tokens would fill
    sentinel = 0x7FC1
    xp = torch.full((m_cap, H), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    x = torch.zeros((1, H), dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros((0, k), dtype=torch.int32, device="cuda")
    moe.permute(x[:0], dst, i32(src), i32(offsets), m_cap, out=xp)
    got = bits(xp)
    pad = [r for r in range(offsets[-1]) if src[r] < 0]
    assert pad == [5, 6, 7, 11, 12, 13, 14, 15]
    assert (got[pad] == 0).all()
    keep = [r for r in range(m_cap) if r not in pad]
    assert (got[keep] == sentinel).all()


# ---------------------------------------------------------------- grouped SwiGLU

WINDOW = 80  # rows: every 160-row half of a row tile holds two whole windows


def _gemm_rows(L, rng, full, large):
    """Rows the expert check compares: all of them on small workloads; else
    one random row in every WINDOW-row window of each checked expert's rows,
    plus its first and last row, so every row tile of the grouped GEMMs (at
    most 320 rows, whatever the banding) is sampled in each half. The large
    DeepSeek-V3 layer checks its 16 hottest experts and 16 others."""
    counts = L["local_counts"]
    if full:
        return np.nonzero(L["src_row"] >= 0)[0]
    nz = np.nonzero(counts)[0]
    if large:
        hot = nz[np.argsort(-counts[nz], kind="stable")[:16]]
        rest = np.setdiff1d(nz, hot)
        nz = np.sort(np.concatenate([hot, rng.choice(rest, min(16, rest.size), replace=False)]))
    rows = []
    for e in nz:
        a, c = int(L["offsets"][e]), int(counts[e])
        pick = [0, c - 1] + [int(rng.integers(w0, min(w0 + WINDOW, c)))
                             for w0 in range(0, c, WINDOW)]
        rows += [a + v for v in pick]
    return np.array(sorted(set(rows)))


@pytest.mark.parametrize("name,dist,share", CASES, ids=IDS)
def test_grouped_swiglu(name, dist, share):
    announce("grouped_swiglu", name, dist, share)
    case = get_case(name, dist, share)
    cfg = case.cfg
    idx, _, L = oracle_routing(case)
    m_cap, H, I = L["m_cap"], cfg.hidden, cfg.inter
    src = torch.as_tensor(L["src_row"].astype(np.int64), device="cuda")
    valid = src >= 0
    # x_perm: the token rows at their oracle places, NaN everywhere else
    xp = torch.full((m_cap, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    xp[valid] = case.x[src[valid] // cfg.top_k]
    y = torch.full((m_cap, H), 0, dtype=torch.int16, device="cuda").fill_(0x7FC1)
    y = y.view(torch.bfloat16)
    h = torch.empty((m_cap, I), dtype=torch.bfloat16, device="cuda")
    w1t, w3t, w2t = (moe.pack_weights(w) for w in (case.w1, case.w3, case.w2))
    counts = i32(L["local_counts"])
    moe.grouped_swiglu(xp, i32(L["offsets"]), counts, w1t, w3t, w2t, h=h, out=y)

    rng = np.random.default_rng(1)
    rows = _gemm_rows(L, rng, name in FULL, name == "deepseek_v3_large")
    xrows = f64(xp[torch.as_tensor(rows, device="cuda")])
    seg = np.searchsorted(L["offsets"], rows, side="right") - 1
    want = np.zeros((rows.size, H))
    for e in np.unique(seg):
        m = seg == e
        want[m] = oexperts.swiglu(xrows[m], *case.weights_of(int(e)))
    got = f64(y[torch.as_tensor(rows, device="cuda")])
    assert np.isfinite(got).all()
    assert rel_max(got, want) <= 1e-2, rel_max(got, want)
    for e in np.unique(seg):  # and each expert group on its own
        m = seg == e
        assert rel_max(got[m], want[m]) <= 1e-2, (int(e), rel_max(got[m], want[m]))
    # padding rows of y are never written
    pad = np.nonzero(L["src_row"][:L["offsets"][-1]] < 0)[0][:512]
    if pad.size:
        assert (bits(y[torch.as_tensor(pad, device="cuda")]) == 0x7FC1).all()


def packed_reference(w: np.ndarray) -> np.ndarray:
    """The packed layout written out from its definition in include/moe.h:
    output-major [m, N, K], N rows in blocks of R (256 if N % 256 == 0, else
    128), each block as K/64 consecutive [R][64] slices."""
    m, K, N = w.shape
    R = 256 if N % 256 == 0 else 128
    out = np.empty(m * N * K, dtype=w.dtype)
    for n in range(N):
        for k0 in range(0, K, 64):
            base = (n // R) * K * R + (k0 // 64) * R * 64 + (n % R) * 64
            for mm in range(m):
                out[mm * N * K + base: mm * N * K + base + 64] = w[mm, k0:k0 + 64, n]
    return out


@pytest.mark.parametrize("shape", [(3, 384, 256), (2, 256, 384), (1, 128, 128)])
def test_pack_weights_layout(shape):
    announce(f"pack {shape}")
    w = torch.randn(shape, device="cuda").to(torch.bfloat16)
    wt = moe.pack_weights(w)
    assert tuple(wt.shape) == (shape[0], shape[2], shape[1])
    assert (bits(wt).reshape(-1) == packed_reference(bits(w))).all()


def test_swiglu_orientation_closed_form():
    # W1 = permutation, W3 = W2 = identity: y[:, j] = silu(x[:, pi(j)]) * x[:, j]
    announce("swiglu orientation")
    n, rows = 128, 200
    rng = np.random.default_rng(3)
    pi = rng.permutation(n)
    P = np.zeros((n, n))
    P[pi, np.arange(n)] = 1.0
    eye = np.eye(n)
    to_d = lambda a: from_bits(obf16.encode(a))[None]  # noqa: E731
    x = obf16.round_to_bf16(rng.standard_normal((rows, n)))
    offsets, counts = i32([0, 256]), i32([rows])
    y = moe.grouped_swiglu(from_bits(obf16.encode(np.vstack([x, np.zeros((56, n))]))), offsets,
                           counts, moe.pack_weights(to_d(P)), moe.pack_weights(to_d(eye)),
                           moe.pack_weights(to_d(eye)))
    want = oexperts.swiglu(x, P, eye, eye)
    assert rel_max(f64(y[:rows]), want) <= 1e-2


# Row counts on every tile boundary of the grouped GEMMs: none, one, the
# 32-row block edges, the 64-row small-tile limit, one 320-row tile and one
# row past it, two and four tiles and one row past them (a band of four row
# tiles plus a tail band). H = 512 takes the 320 x 256 tiles for both
# products; H = 384 gives down an output width that is not a multiple of 256,
# which takes the 256 x 128 tiles.
EDGE_COUNTS = [0, 1, 31, 32, 33, 63, 64, 65, 96, 255, 256, 257, 319, 320, 321, 640, 641,
               1280, 1283, 0]


@pytest.mark.parametrize("H,I", [(512, 256), (384, 128)])
def test_grouped_swiglu_tile_edges(H, I):
    announce(f"grouped_swiglu tile edges H={H} I={I}")
    rng = np.random.default_rng(H + I)
    counts = np.array(EDGE_COUNTS)
    E = counts.size
    padded = (counts + 127) // 128 * 128
    offsets = np.concatenate([[0], np.cumsum(padded)])
    m_cap = int(offsets[-1]) + 128  # a tail past the last group
    w1 = obf16.round_to_bf16(rng.standard_normal((E, H, I)) / np.sqrt(H))
    w3 = obf16.round_to_bf16(rng.standard_normal((E, H, I)) / np.sqrt(H))
    w2 = obf16.round_to_bf16(rng.standard_normal((E, I, H)) / np.sqrt(I))
    x = np.full((m_cap, H), np.nan)
    for e in range(E):
        a = offsets[e]
        x[a:a + counts[e]] = obf16.round_to_bf16(rng.standard_normal((counts[e], H)))
    dev = lambda a: from_bits(obf16.encode(a))  # noqa: E731
    h = torch.zeros((m_cap, I), dtype=torch.int16, device="cuda").fill_(0x7FC1)
    y = torch.zeros((m_cap, H), dtype=torch.int16, device="cuda").fill_(0x7FC1)
    h, y = h.view(torch.bfloat16), y.view(torch.bfloat16)
    moe.grouped_swiglu(dev(x), i32(offsets), i32(counts), moe.pack_weights(dev(w1)),
                       moe.pack_weights(dev(w3)), moe.pack_weights(dev(w2)), h=h, out=y)
    got = f64(y)
    for e in range(E):
        a, c = int(offsets[e]), int(counts[e])
        if c:
            want = oexperts.swiglu(x[a:a + c], w1[e], w3[e], w2[e])
            assert np.isfinite(got[a:a + c]).all(), (e, c)
            assert rel_max(got[a:a + c], want) <= 1e-2, (e, c, rel_max(got[a:a + c], want))
        # rows past the group (padding, and the tail after the last group) are never written
        end = int(offsets[e + 1]) if e + 1 < E else m_cap
        assert (bits(y[a + c:end]) == 0x7FC1).all(), (e, c)
        assert (bits(h[a + c:end]) == 0x7FC1).all(), (e, c)


# ---------------------------------------------------------------- combine

def _combine_tokens(cfg, rng, full):
    return np.arange(cfg.num_tokens) if full else np.sort(
        rng.choice(cfg.num_tokens, min(cfg.num_tokens, 1024), replace=False))


@pytest.mark.parametrize("name,dist,share", CASES, ids=IDS)
def test_combine(name, dist, share):
    announce("combine", name, dist, share)
    case = get_case(name, dist, share, weights=False)
    cfg = case.cfg
    idx, w, L = oracle_routing(case)
    y = workloads.gen.expert_outputs(cfg, L["m_cap"], seed=5, device="cuda")
    w32 = w.astype(np.float32)
    out = moe.combine(y, i32(L["dst_row"]), torch.from_numpy(w32).cuda())
    rng = np.random.default_rng(2)
    toks = _combine_tokens(cfg, rng, name in FULL)
    dst = L["dst_row"][toks]
    rows = np.unique(dst[dst >= 0])
    ysub = f64(y[torch.as_tensor(rows, device="cuda")])
    remap = np.full(L["m_cap"], -1)
    remap[rows] = np.arange(rows.size)
    dsub = np.where(dst >= 0, remap[dst], -1)
    want = obf16.encode(ocombine.combine(ysub, dsub, w32[toks]))
    got = bits(out[torch.as_tensor(toks, device="cuda")])
    d = ulp_distance(got, want)
    assert d.max() <= 1, (d.max(), np.argwhere(d > 1)[:5])
    # both sides perform the same fp32 operations in the same order
    assert d.max() == 0, (int((d > 0).sum()), np.argwhere(d > 0)[:5])
    # and against the fp64 sum: within the a-priori bound of an FP32
    # slot-order restore plus half a bf16 unit of the result
    err = np.abs(obf16.decode(got) - ocombine.combine_exact(ysub, dsub, w32[toks]))
    bound = ocombine.combine_error_bound(ysub, dsub, w32[toks])
    assert (err <= bound).all(), np.argwhere(err > bound)[:5]
    # tokens without a local slot come back as zero rows
    none_local = (dst < 0).all(axis=1)
    assert (got[none_local] & 0x7FFF == 0).all()


def test_combine_invariant_under_row_shuffle():
    announce("combine shuffle")
    cfg = workloads.get("qwen3_30b_a3b")
    case = get_case(cfg.name, "zipf", -1, weights=False)
    idx, w, L = oracle_routing(case)
    y = workloads.gen.expert_outputs(cfg, L["m_cap"], seed=6, device="cuda")
    wt = torch.from_numpy(w.astype(np.float32)).cuda()
    a = moe.combine(y, i32(L["dst_row"]), wt)
    perm = torch.randperm(L["m_cap"], generator=torch.Generator().manual_seed(0)).cuda()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel(), device="cuda")
    dst = torch.as_tensor(L["dst_row"].astype(np.int64), device="cuda")
    dst2 = torch.where(dst >= 0, inv[dst.clamp(min=0)], dst).to(torch.int32)
    b = moe.combine(y[perm].contiguous(), dst2, wt)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_combine_only_large():
    # the combine on its own at the large DeepSeek-V3 shape: expert outputs
    # [T*8, H] in expert order with no padding (alignment 1), severe skew
    announce("combine-only large")
    cfg = workloads.get("deepseek_v3_large")
    case = get_case(cfg.name, "severe", -1, weights=False)
    idx, w = oroute.route(case.logits_np(), cfg.top_k)
    L = olayout.layout(idx, cfg.num_experts, 1, -1, 1)
    n = cfg.num_tokens * cfg.top_k
    y = workloads.gen.expert_outputs(cfg, n, seed=7, device="cuda")
    w32 = w.astype(np.float32)
    out = moe.combine(y, i32(L["dst_row"]), torch.from_numpy(w32).cuda())
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(cfg.num_tokens, 512, replace=False))
    dst = L["dst_row"][toks]
    rows = np.unique(dst)
    remap = np.full(n, -1)
    remap[rows] = np.arange(rows.size)
    ysub = f64(y[torch.as_tensor(rows, device="cuda")])
    want = obf16.encode(ocombine.combine(ysub, remap[dst], w32[toks]))
    got = bits(out[torch.as_tensor(toks, device="cuda")])
    assert ulp_distance(got, want).max() == 0
    err = np.abs(obf16.decode(got) - ocombine.combine_exact(ysub, remap[dst], w32[toks]))
    assert (err <= ocombine.combine_error_bound(ysub, remap[dst], w32[toks])).all()


# ---------------------------------------------------------------- whole layer

def _layer_tokens(case, idx, rng, full):
    """All tokens of small workloads; else 64 tokens (16 on the large
    DeepSeek-V3 layer), taken so that the local experts with the most rows
    (every hot expert under skew) are each reached by one of them, then random
    tokens with a local slot."""
    cfg = case.cfg
    if full:
        return np.arange(cfg.num_tokens)
    n = 16 if cfg.name == "deepseek_v3_large" else 64
    local = (idx >= case.first) & (idx < case.first + case.num_local)
    counts = np.bincount(idx[local] - case.first, minlength=case.num_local)
    chosen = []
    for e in np.argsort(-counts, kind="stable")[:n]:
        if counts[e] == 0 or len(chosen) == n:
            break
        cand = np.setdiff1d(np.nonzero((idx == case.first + e).any(axis=1))[0], chosen)
        if cand.size:
            chosen.append(int(rng.choice(cand)))
    rest = np.setdiff1d(np.nonzero(local.any(axis=1))[0], chosen)
    chosen += rng.choice(rest, min(n - len(chosen), rest.size), replace=False).tolist()
    return np.sort(np.array(chosen, dtype=np.int64))


@pytest.mark.parametrize("name,dist,share", CASES, ids=IDS)
def test_layer(name, dist, share):
    announce("layer", name, dist, share)
    case = get_case(name, dist, share)
    cfg = case.cfg
    layer = moe.MoELayer(cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter,
                         case.w1, case.w3, case.w2, cfg.ep_size, share, cfg.align)
    out = layer(case.x, case.logits).clone()
    idx, w, L = oracle_routing(case)
    # integer outputs of the GPU pipeline: bit-exact
    assert (layer.topk_idx.cpu().numpy() == idx).all()
    for k in LAYOUT_KEYS:
        assert (getattr(layer.L, k).cpu().numpy() == L[k]).all(), k
    rng = np.random.default_rng(3)
    toks = _layer_tokens(case, idx, rng, name in FULL)
    want = olayer.token_outputs(toks, case.x_np(), idx, w, case.weights_of, case.first,
                                case.num_local)
    got = f64(out[torch.as_tensor(toks, device="cuda")])
    assert np.isfinite(got).all()
    assert rel_max(got, want) <= 1e-2, rel_max(got, want)
    # running the layer again gives the same bits (no dependence on scheduling)
    again = layer(case.x, case.logits)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    del layer


# ---------------------------------------------------------------- permute fused into gate/up

GATHER_CASES = [("tiny", "balanced", 1), ("ragged", "mild", 2), ("top1_odd", "balanced", -1),
                ("tiled", "mild", 1), ("fused_edge", "severe", 3),
                ("mixtral_8x7b", "balanced", -1), ("qwen3_30b_a3b", "zipf", -1),
                ("deepseek_v3_ep8_share", "severe", 0), ("deepseek_v3_large", "severe", -1)]


@pytest.mark.parametrize("name,dist,share", GATHER_CASES,
                         ids=[f"{c}-{d}-r{s}" for c, d, s in GATHER_CASES])
def test_gate_up_gather_equals_permute_then_gate_up(name, dist, share):
    # the gathering gate/up reads the same operand values in the same row
    # order as the permute followed by the plain gate/up: h bit for bit, and
    # rows outside the expert groups untouched
    announce("gate_up gather", name, dist, share)
    case = get_case(name, dist, share)
    cfg = case.cfg
    idx, _, L = oracle_routing(case)
    m_cap = L["m_cap"]
    src = i32(L["src_row"])
    off, cnt = i32(L["offsets"]), i32(L["local_counts"])
    w1t, w3t = moe.pack_weights(case.w1), moe.pack_weights(case.w3)
    xp = moe.permute(case.x, i32(L["dst_row"]), src, off, m_cap)
    want = moe.grouped_gate_up(xp, off, cnt, w1t, w3t)
    got = torch.full((m_cap, cfg.inter), 0, dtype=torch.int16, device="cuda").fill_(0x7FC1)
    got = got.view(torch.bfloat16)
    moe.grouped_gate_up_gather(case.x, src, cfg.top_k, off, cnt, w1t, w3t, out=got)
    valid = torch.as_tensor(L["src_row"] >= 0, device="cuda")
    assert torch.equal(got[valid].view(torch.int16), want[valid].view(torch.int16))
    pad = torch.nonzero(~valid).flatten()[:4096]
    assert (bits(got[pad]) == 0x7FC1).all()


def test_layer_gather_equals_layer_with_permute():
    announce("layer gather vs permute")
    cfg = EXTRA["ragged"]
    case = get_case("ragged", "mild", 2)
    outs = []
    for gather in (True, False):
        layer = moe.MoELayer(cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter,
                             case.w1, case.w3, case.w2, cfg.ep_size, 2, cfg.align, gather=gather)
        outs.append(layer(case.x, case.logits).clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
