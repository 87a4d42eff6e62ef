"""Pins of the oracle's routing, layout and permute: a hand-computed example,
closed forms, brute force on tiny inputs and the invariants the pages state."""
import math

import numpy as np
import pytest

import workloads
from oracle import checks, layout as olayout, permute as opermute, route as oroute


# ---------------------------------------------------------------- worked example

def test_route_worked_example(worked_example):
    g = worked_example
    idx, w = oroute.route(np.array(g["logits"], np.float32), g["top_k"])
    assert idx.tolist() == g["topk_idx"]
    np.testing.assert_allclose(w, g["topk_w"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("share", ["-1", "0", "1"])
def test_layout_worked_example(worked_example, share):
    g = worked_example
    L = olayout.layout(np.array(g["topk_idx"]), g["num_experts"], g["ep_size"],
                       int(share), g["align"])
    want = g["shares"][share]
    assert L["send_counts"].tolist() == g["send_counts"]
    assert L["expert_counts"].tolist() == g["expert_counts"]
    assert L["split_matrix"].tolist() == g["split_matrix"]
    for key in ("recv_counts", "output_splits", "offsets", "dst_row"):
        assert L[key].tolist() == want[key], key
    n = len(want["src_row"])
    assert L["src_row"][:n].tolist() == want["src_row"]
    assert (L["src_row"][n:] == -1).all()


def test_permute_worked_example(worked_example):
    g = worked_example
    L = olayout.layout(np.array(g["topk_idx"]), 4, 2, -1, 2)
    x = np.array([[10], [11], [12], [13]], dtype=np.int64)
    xp = opermute.permute(x, L["src_row"], 2)
    # src_row [0,6,4,-1,1,2,7,-1,3,5] -> tokens [0,3,2,pad,0,1,3,pad,1,2]
    assert xp[:10, 0].tolist() == [10, 13, 12, 0, 10, 11, 13, 0, 11, 12]


# ---------------------------------------------------------------- route pins

def _brute_select(row, k):
    return [e for _, e in sorted((-float(v), e) for e, v in enumerate(row))][:k]


def test_route_select_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for E, k in [(4, 1), (8, 2), (8, 8), (16, 5), (64, 8)]:
        logits = rng.integers(-3, 4, size=(50, E)).astype(np.float32)  # many ties
        idx = oroute.select(logits, k)
        for t in range(50):
            assert idx[t].tolist() == _brute_select(logits[t], k)


def test_route_signed_zero_ties_to_lower_id():
    logits = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    assert oroute.select(logits, 2).tolist() == [[0, 1], [0, 1]]


def test_route_closed_forms():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((100, 16)).astype(np.float32)
    # k = 1: the weight is exactly one
    _, w1 = oroute.route(logits, 1)
    assert (w1 == 1.0).all()
    # k = 2: w0 = sigmoid(l0 - l1)
    idx, w2 = oroute.route(logits, 2)
    l = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), 1)
    sig = 1.0 / (1.0 + np.exp(-(l[:, 0] - l[:, 1])))
    np.testing.assert_allclose(w2[:, 0], sig, rtol=1e-14)
    # equal logits: the lowest k ids, each weighing 1/k
    eq = np.full((3, 16), 0.25, np.float32)
    idx, w = oroute.route(eq, 5)
    assert (idx == np.arange(5)).all()
    np.testing.assert_allclose(w, 0.2, rtol=1e-15)


def test_route_weights_equal_softmax_over_selection():
    # softmax over E then renormalise == softmax over the k selected logits
    rng = np.random.default_rng(3)
    logits = (3 * rng.standard_normal((64, 32))).astype(np.float32)
    idx, w = oroute.route(logits, 6)
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), 1)
    ref = np.array([[math.exp(v - r.max()) for v in r] for r in sel])
    ref /= ref.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-13)


# ---------------------------------------------------------------- layout pins

def _brute_layout(idx, E, ep, local_rank, align):
    """Pure-Python layout by nested loops (the definition, unvectorised)."""
    T, k = len(idx), len(idx[0])
    chunk = T // ep
    send = [[0] * E for _ in range(ep)]
    for t in range(T):
        for s in range(k):
            send[t // chunk][idx[t][s]] += 1
    first, el = (0, E) if local_rank < 0 else (local_rank * (E // ep), E // ep)
    offsets, src, dst = [0], [], [[-1] * k for _ in range(T)]
    for e in range(first, first + el):
        members = [(t, s) for t in range(T) for s in range(k) if idx[t][s] == e]
        for t, s in members:
            dst[t][s] = len(src)
            src.append(t * k + s)
        while len(src) % align:
            src.append(-1)
        offsets.append(len(src))
    recv = [[send[s][e] for e in range(first, first + el)] for s in range(ep)]
    split = [[sum(send[s][d * (E // ep):(d + 1) * (E // ep)]) for d in range(ep)]
             for s in range(ep)]
    return send, recv, split, offsets, src, dst


def test_layout_brute_force_small():
    rng = np.random.default_rng(4)
    for T, E, k, ep, align in [(8, 4, 2, 2, 2), (12, 6, 3, 3, 4), (16, 8, 8, 4, 1),
                               (32, 16, 4, 2, 8), (6, 3, 1, 3, 2)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        for lr in [-1] + list(range(ep)):
            send, recv, split, offsets, src, dst = _brute_layout(idx.tolist(), E, ep, lr, align)
            L = olayout.layout(idx, E, ep, lr, align)
            assert L["send_counts"].tolist() == send
            assert L["recv_counts"].tolist() == recv
            assert L["split_matrix"].tolist() == split
            assert L["offsets"].tolist() == offsets
            assert L["dst_row"].tolist() == dst
            assert L["src_row"][:len(src)].tolist() == src
            assert (L["src_row"][len(src):] == -1).all()
            checks.check_layout(idx, L, E, ep, lr, align)


def test_layout_zero_count_expert_takes_no_rows():
    idx = np.array([[0, 2], [2, 0]])
    L = olayout.layout(idx, 4, 1, -1, 128)
    assert L["offsets"].tolist() == [0, 128, 128, 256, 256]


def test_layout_rejects_small_m_cap():
    idx = np.array([[0, 1], [1, 0]])
    with pytest.raises(ValueError):
        olayout.layout(idx, 2, 1, -1, 4, m_cap=7)


def test_coverage_exactly_once_over_shares():
    rng = np.random.default_rng(5)
    T, E, k, ep = 32, 8, 3, 4
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    dsts = [olayout.layout(idx, E, ep, d, 4)["dst_row"] for d in range(ep)]
    checks.check_coverage(dsts, T, k)
    # split matrices of the shares are consistent: column d == output_splits of d
    full = olayout.layout(idx, E, ep, 0, 4)["split_matrix"]
    for d in range(ep):
        assert (full[:, d] == olayout.layout(idx, E, ep, d, 4)["output_splits"]).all()
    dropped = [d.copy() for d in dsts]
    dropped[1][dropped[1] >= 0] = -1
    with pytest.raises(RuntimeError):
        checks.check_coverage(dropped, T, k)
    with pytest.raises(RuntimeError):
        checks.check_coverage(dsts + [dsts[0]], T, k)


def test_check_layout_catches_planted_mistakes():
    rng = np.random.default_rng(6)
    idx = np.stack([rng.permutation(8)[:2] for _ in range(16)])
    L = olayout.layout(idx, 8, 2, 0, 4)
    bad = dict(L, src_row=L["src_row"].copy())
    o = L["offsets"]
    seg = bad["src_row"][o[0]:o[0] + L["local_counts"][0]]
    if len(seg) >= 2:
        seg[[0, 1]] = seg[[1, 0]]  # break stability
        with pytest.raises(AssertionError):
            checks.check_layout(idx, bad, 8, 2, 0, 4)
    bad2 = dict(L, output_splits=L["output_splits"] + 1)
    with pytest.raises(AssertionError):
        checks.check_layout(idx, bad2, 8, 2, 0, 4)



def _consistent(L, src):
    # a layout whose dst_row is the inverse of the given src_row, so that only
    # the property a test breaks is wrong
    dst = np.full(L["dst_row"].size, -1, dtype=np.int64)
    rows = np.nonzero(src >= 0)[0]
    dst[src[rows]] = rows
    return dict(L, src_row=src.astype(np.int32),
                dst_row=dst.reshape(L["dst_row"].shape).astype(np.int32))


def test_check_layout_catches_each_planted_mistake_alone():
    rng = np.random.default_rng(16)
    idx = np.stack([rng.permutation(8)[:2] for _ in range(64)])
    L = olayout.layout(idx, 8, 2, 0, 4)
    checks.check_layout(idx, L, 8, 2, 0, 4)
    o, c = L["offsets"].astype(np.int64), L["local_counts"].astype(np.int64)
    e = int(np.nonzero((c >= 2) & (c % 4 != 0))[0][0])  # an expert with padding
    a = o[e]
    src = L["src_row"].astype(np.int64).copy()
    src[[a, a + 1]] = src[[a + 1, a]]  # two rows of one expert swapped
    with pytest.raises(AssertionError, match="unstable"):
        checks.check_layout(idx, _consistent(L, src), 8, 2, 0, 4)
    src = L["src_row"].astype(np.int64).copy()
    src[a + c[e]], src[a + c[e] - 1] = src[a + c[e] - 1], -1  # last row moved into padding
    with pytest.raises(AssertionError, match="padding misplaced"):
        checks.check_layout(idx, _consistent(L, src), 8, 2, 0, 4)
    src = L["src_row"].astype(np.int64).copy()
    tail = int(o[-1])
    if tail < src.size:
        src[tail] = src[a]  # a tail row claims an assignment too
        with pytest.raises(AssertionError):
            checks.check_layout(idx, dict(L, src_row=src.astype(np.int32)), 8, 2, 0, 4)


def test_check_route_catches_each_planted_mistake_alone():
    rng = np.random.default_rng(17)
    logits = rng.standard_normal((32, 16)).astype(np.float32)
    idx, w = oroute.route(logits, 4)
    checks.check_route(logits, idx, w)
    swapped = idx.copy()
    swapped[3, [0, 1]] = swapped[3, [1, 0]]
    w_sw = w.copy()
    w_sw[3, [0, 1]] = w_sw[3, [1, 0]]
    with pytest.raises(AssertionError, match="descending logit order"):
        checks.check_route(logits, swapped, w_sw)
    fifth = np.argsort(-logits[5], kind="stable")[4]  # the best expert not selected
    worse = idx.copy()
    worse[5, 3] = fifth
    with pytest.raises(AssertionError, match="unselected logit beats"):
        checks.check_route(logits, worse, w)


# ---------------------------------------------------------------- workloads

@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_invariants_on_every_workload(name):
    cfg = workloads.get(name)
    for dist in cfg.dists:
        _, logits = workloads.gen.routing_inputs(cfg, dist, seed=0)
        idx, w = oroute.route(logits.numpy(), cfg.top_k)
        checks.check_route(logits.numpy(), idx, w)
        dsts = []
        for lr in ([-1] + list(range(cfg.ep_size)) if cfg.ep_size > 1 else [-1]):
            L = olayout.layout(idx, cfg.num_experts, cfg.ep_size, lr, cfg.align)
            checks.check_layout(idx, L, cfg.num_experts, cfg.ep_size, lr, cfg.align)
            if lr >= 0:
                dsts.append(L["dst_row"])
            assert L["offsets"][-1] <= cfg.m_cap(lr)
        if dsts:
            checks.check_coverage(dsts, cfg.num_tokens, cfg.top_k)


def test_skew_distributions_skew():
    cfg = workloads.get("deepseek_v3_ep8_share")
    counts = {}
    for dist in cfg.dists:
        _, logits = workloads.gen.routing_inputs(cfg, dist, seed=0)
        idx, _ = oroute.route(logits.numpy(), cfg.top_k)
        counts[dist] = np.bincount(idx.reshape(-1), minlength=256)
    spread = {d: c.max() / c.mean() for d, c in counts.items()}
    assert spread["balanced"] < spread["mild"] < spread["severe"]
    hot = workloads.gen.routing_bias(cfg, "severe").numpy() > 0
    assert counts["severe"][hot].min() > counts["severe"][~hot].max()


# ---------------------------------------------------------------- dedup layout

def _brute_dispatch_layout(idx, E, ep):
    el = E // ep
    T, k = len(idx), len(idx[0])
    in_rank = [[0] * ep for _ in range(T)]
    for t in range(T):
        for s in range(k):
            e = idx[t][s]
            if 0 <= e < E:
                in_rank[t][e // el] = 1
    pos = [[-1] * ep for _ in range(T)]
    count = [0] * ep
    for t in range(T):
        for r in range(ep):
            if in_rank[t][r]:
                pos[t][r] = count[r]
                count[r] += 1
    per_expert = [0] * E
    for row in idx:
        for e in row:
            if 0 <= e < E:
                per_expert[e] += 1
    return in_rank, count, per_expert, pos


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_dispatch_layout_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    E, ep, k = 12, 4, 3
    T = 40
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = E + 3  # a few out-of-range ids are skipped
    got = olayout.dispatch_layout(idx, E, ep)
    in_rank, count, per_expert, pos = _brute_dispatch_layout(idx.tolist(), E, ep)
    np.testing.assert_array_equal(got["is_token_in_rank"], np.array(in_rank, dtype=np.uint8))
    np.testing.assert_array_equal(got["num_tokens_per_rank"], count)
    np.testing.assert_array_equal(got["num_tokens_per_expert"], per_expert)
    np.testing.assert_array_equal(got["token_rank_pos"], pos)


def test_dispatch_layout_worked_example(worked_example):
    # the golden 4-token example: experts 0-1 on rank 0, 2-3 on rank 1
    g = worked_example
    idx = np.array(g["topk_idx"], dtype=np.int32)  # [[0,2],[2,3],[1,3],[0,2]]
    got = olayout.dispatch_layout(idx, 4, 2)
    # t0 -> ranks 0 and 1; t1 -> rank 1 only (two slots there, sent once); t2 -> both; t3 -> both
    np.testing.assert_array_equal(got["is_token_in_rank"], [[1, 1], [0, 1], [1, 1], [1, 1]])
    np.testing.assert_array_equal(got["num_tokens_per_rank"], [3, 4])
    np.testing.assert_array_equal(got["token_rank_pos"], [[0, 0], [-1, 1], [1, 2], [2, 3]])
    np.testing.assert_array_equal(got["num_tokens_per_expert"], g["expert_counts"])
    # a token never counts more than once per rank, and at most min(k, ep) times overall
    assert got["is_token_in_rank"].sum(axis=1).max() <= 2
