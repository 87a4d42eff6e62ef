"""Pins of the oracle's floating-point steps: bf16 rounding, the SwiGLU
expert, the weighted combine and the composed layer."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, checks, combine as ocombine, experts as oexperts
from oracle import layer as olayer, layout as olayout, permute as opermute, route as oroute


# ---------------------------------------------------------------- bf16

def test_bf16_ties_to_even_and_single_rounding():
    cases = {
        1.0 + 2 ** -8: 1.0,  # halfway, 1.0 is even
        1.0 + 3 * 2 ** -8: 1.0 + 2 ** -6,  # halfway, rounds up to even
        1.0 + 2 ** -8 + 2 ** -20: 1.0 + 2 ** -7,  # above halfway
        # above halfway only by 2^-30: rounding through fp32 first would lose
        # the 2^-30 and land on the tie (-> 1.0); one rounding gives 1 + 2^-7
        1.0 + 2 ** -8 + 2 ** -30: 1.0 + 2 ** -7,
        -2.0757656856: -2.078125,
        0.0: 0.0,
        3.4e38: math.inf,  # rounds past the largest finite bf16, (2 - 2^-7) * 2^127
    }
    for x, want in cases.items():
        assert bf16.round_to_bf16(x) == want, x


def test_bf16_matches_torch_on_fp32_values():
    # for inputs that are fp32 numbers, one rounding to bf16 is what torch's
    # fp32 -> bf16 conversion does
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf16.encode(x.astype(np.float64)) == want).all()
    assert (bf16.decode(want) == bf16.round_to_bf16(x.astype(np.float64))).all()



def test_bf16_ends_of_the_range():
    # Worked by hand from the bf16 format (8 significant bits, fp32's
    # exponent range, round to nearest, ties to even):
    #   the largest finite value (2 - 2^-7) * 2^127 stays finite;
    #   the midpoint between it and 2^128 ties to the even neighbour, 2^128,
    #   which overflows to infinity, and anything just below stays finite;
    #   the smallest subnormal 2^-133 stays; 2^-134 is the midpoint between 0
    #   and 2^-133 and goes to 0 (even); 3 * 2^-134 is the midpoint between
    #   2^-133 and 2^-132 and goes to 2^-132 (even); zeros keep their sign.
    mx = bf16.BF16_MAX
    mid = 2.0 ** 128 - 2.0 ** 119
    x = np.array([mx, -mx, mid, -mid, np.nextafter(np.float32(mid), np.float32(0)),
                  np.finfo(np.float32).max, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134,
                  -0.0, 0.0], dtype=np.float32).astype(np.float64)
    want = np.array([mx, -mx, np.inf, -np.inf, mx, np.inf, 2.0 ** -133, 0.0, 2.0 ** -132,
                     -0.0, 0.0])
    got = bf16.round_to_bf16(x)
    assert (got == want).all() and (np.signbit(got) == np.signbit(want)).all()
    tb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    assert (bf16.encode(x) == tb.numpy().view(np.uint16)).all()


# ---------------------------------------------------------------- experts

def test_swiglu_hand_example(swiglu_2x2):
    g = swiglu_2x2
    y = oexperts.swiglu(np.array(g["x"]), np.array(g["w1"]), np.array(g["w3"]), np.array(g["w2"]))
    np.testing.assert_allclose(y, g["y"], rtol=1e-12)


def test_swiglu_brute_force_loops():
    rng = np.random.default_rng(8)
    m, H, I = 3, 5, 4
    x, w1, w3, w2 = (rng.standard_normal(s) for s in [(m, H), (H, I), (H, I), (I, H)])
    y = oexperts.swiglu(x, w1, w3, w2)
    for r in range(m):
        h = []
        for i in range(I):
            g = sum(x[r, j] * w1[j, i] for j in range(H))
            u = sum(x[r, j] * w3[j, i] for j in range(H))
            h.append(g / (1 + math.exp(-g)) * u)
        for c in range(H):
            assert abs(y[r, c] - sum(h[i] * w2[i, c] for i in range(I))) < 1e-12


def test_swiglu_orientation_closed_form():
    # W1 = permutation P, W3 = W2 = identity: y[:, j] = silu(x[:, pi(j)]) * x[:, j]
    rng = np.random.default_rng(9)
    n = 6
    pi = rng.permutation(n)
    P = np.zeros((n, n))
    P[pi, np.arange(n)] = 1.0  # (x P)[:, j] = x[:, pi[j]]
    x = rng.standard_normal((4, n))
    y = oexperts.swiglu(x, P, np.eye(n), np.eye(n))
    want = x[:, pi] / (1 + np.exp(-x[:, pi])) * x
    np.testing.assert_allclose(y, want, rtol=1e-14)
    assert np.all(oexperts.swiglu(x, np.zeros((n, n)), np.zeros((n, n)), np.eye(n)) == 0)


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("share", ["-1", "1"])
def test_combine_worked_example(worked_example, share):
    g = worked_example
    want = g["shares"][share]
    dst = np.array(want["dst_row"])
    y = np.arange(1, 11, dtype=np.float64)[:, None]
    out = ocombine.combine_bf16(y, dst, np.array(g["topk_w"]))
    assert out[:, 0].tolist() == want["combine_y_r_plus_1"]


def test_combine_is_the_fp32_slot_order_sum():
    # products and partial sums are fp32 operations, not fused, not fp64:
    # slot 0 gives -1; slot 1's product (1 + 2^-23) * (1 + 2^-7) is exactly
    # 1 + 2^-7 + 2^-23 + 2^-30, rounded in fp32 to 1 + 2^-7 + 2^-23; the sum
    # is then 2^-7 + 2^-23 (an FMA would keep the 2^-30, fp64 too)
    w = np.array([[1.0, 1.0 + 2.0 ** -23]])
    y = np.array([[-1.0], [1.0 + 2.0 ** -7]])
    dst = np.array([[0, 1]])
    out = ocombine.combine(y, dst, w)
    assert out.dtype == np.float32 and out[0, 0] == np.float32(2.0 ** -7 + 2.0 ** -23)
    assert ocombine.combine_exact(y, dst, w)[0, 0] == 2.0 ** -7 + 2.0 ** -23 + 2.0 ** -30
    # a rounded product that changes the bf16 result: fp32 gives 2^-23 where
    # the exact sum is 2^-23 * (1 + 2^-7), itself a bf16 number
    w = np.array([[1.0 + 2.0 ** -23, 1.0]])
    y = np.array([[1.0 + 2.0 ** -7], [-(1.0 + 2.0 ** -7)]])
    assert ocombine.combine_bf16(y, dst, w)[0, 0] == 2.0 ** -23
    assert bf16.round_to_bf16(ocombine.combine_exact(y, dst, w))[0, 0] == 2.0 ** -23 * (1 + 2.0 ** -7)


def test_combine_missing_assignment_raises():
    dst = np.array([[0, 1], [2, -1]])
    with pytest.raises(RuntimeError):
        ocombine.combine(np.ones((3, 4)), dst, np.full((2, 2), 0.5), validate_coverage=True)


def test_combine_top1_is_exact_unpermute():
    rng = np.random.default_rng(10)
    T, E, H = 40, 8, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oroute.route(logits, 1)
    L = olayout.layout(idx, E, 1, -1, 4)
    y = bf16.round_to_bf16(rng.standard_normal((L["m_cap"], H)))
    out = ocombine.combine_bf16(y, L["dst_row"], w)
    assert (out == y[L["dst_row"][:, 0]]).all()


def test_combine_identity_experts_returns_x():
    # y = x_perm (identity experts), all slots local: sum_k w x = x, exact in bf16
    cfg = workloads.get("tiny")
    x, logits = workloads.gen.routing_inputs(cfg, "balanced")
    xb = bf16.decode(x.view(torch.int16).numpy().view(np.uint16))
    idx, w = oroute.route(logits.numpy(), cfg.top_k)
    L = olayout.layout(idx, cfg.num_experts, cfg.ep_size, -1, cfg.align)
    xp = opermute.permute(xb, L["src_row"], cfg.top_k)
    assert (ocombine.combine_bf16(xp, L["dst_row"], w, validate_coverage=True) == xb).all()


def test_combine_invariant_under_row_shuffle():
    rng = np.random.default_rng(11)
    T, k, H, R = 64, 4, 32, 300
    dst = np.stack([rng.permutation(R)[:k] for _ in range(T)])
    w = rng.random((T, k))
    y = bf16.round_to_bf16(rng.standard_normal((R, H)))
    perm = rng.permutation(R)  # new row of old row r is inv[r]
    inv = np.argsort(perm)
    y2 = y[perm]
    a = ocombine.combine_bf16(y, dst, w)
    b = ocombine.combine_bf16(y2, inv[dst], w)
    assert (a == b).all()


@pytest.mark.parametrize("k,E,default_err", [(4, 128, 3.58e-3), (8, 256, 4.36e-3)])
def test_combine_error_matches_the_pages_benchmark(k, E, default_err):
    # Against an fp64 reference, the fused restore's relative L2 error is the
    # rounding of the bf16 output, 1.66e-3, while the bf16 default restore,
    # which rounds the weight, every product and every per-slot sum, lands at
    # 3.58e-3 (top-4) and 4.36e-3 (top-8) (DeepSpeed PR #8847, section
    # Benchmark). Gaussian rows, softmax top-k weights of Gaussian logits;
    # the pages' routing weights are not given, hence the 15 % band.
    rng = np.random.default_rng(12)
    T, H = 4096, 256
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oroute.route(logits, k)
    L = olayout.layout(idx, E, 1, -1, 1)
    y = bf16.round_to_bf16(rng.standard_normal((L["m_cap"], H)))
    exact = ocombine.combine_exact(y, L["dst_row"], w)
    fused = ocombine.combine_bf16(y, L["dst_row"], w)
    default = ocombine.restore_default(y, L["dst_row"], w)
    rel = lambda a: np.linalg.norm(a - exact) / np.linalg.norm(exact)  # noqa: E731
    assert abs(rel(fused) / 1.66e-3 - 1) < 0.05
    assert abs(rel(default) / default_err - 1) < 0.15



def test_restore_default_rounds_the_weight_before_the_product():
    # The default restore works in the activation dtype (DeepSpeed PR #8847,
    # section "Problem"), so the routing weight is itself a bf16 number before
    # it multiplies the row. Worked by hand: w = 1 + 2^-8 + 2^-10 lies above
    # the midpoint 1 + 2^-8, so bf16(w) = 1 + 2^-7; times 3 that is
    # 3.0234375, the midpoint between 3.015625 and 3.03125, which ties to
    # the even 3.03125. Rounding only the product, 3w = 3.0146484375, would
    # give 3.015625.
    w = np.array([[1 + 2.0 ** -8 + 2.0 ** -10]], dtype=np.float32)
    out = ocombine.restore_default(np.array([[3.0]]), np.array([[0]]), w)
    assert out[0, 0] == 3.03125


# ---------------------------------------------------------------- layer

@pytest.mark.parametrize("share", [-1, 0, 1])
def test_layer_equals_per_token_definition(share):
    cfg = workloads.get("tiny")
    x, logits = workloads.gen.routing_inputs(cfg, "balanced")
    xb = bf16.decode(x.view(torch.int16).numpy().view(np.uint16))
    experts = list(cfg.local_experts(share))
    w1, w3, w2 = workloads.gen.expert_weights(cfg, experts)
    dec = lambda t: bf16.decode(t.view(torch.int16).numpy().view(np.uint16))  # noqa: E731
    W = [(dec(w1[j]), dec(w3[j]), dec(w2[j])) for j in range(len(experts))]
    res = olayer.layer(xb, logits.numpy(), cfg.top_k, lambda e: W[e], cfg.num_experts,
                       cfg.ep_size, share, cfg.align)
    tok = olayer.token_outputs(np.arange(cfg.num_tokens), xb, res["topk_idx"], res["topk_w"],
                               lambda e: W[e], experts[0], len(experts))
    np.testing.assert_allclose(res["out"], tok, rtol=1e-12, atol=1e-12)
    checks.check_layout(res["topk_idx"], res["layout"], cfg.num_experts, cfg.ep_size,
                        share, cfg.align)


# ---------------------------------------------------------------- combine variants

def test_combine_rows_fp32_is_the_fp32_sum():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((10, 6))
    dst = np.array([[0, 3], [1, -1], [2, 9], [-1, -1], [4, 5]])
    w = rng.random((5, 2))
    np.testing.assert_array_equal(ocombine.combine_rows(y, dst, w, row_dtype="fp32"),
                                  ocombine.combine(y, dst, w).astype(np.float64))


def test_combine_rows_rounds_once_to_the_row_dtype():
    # fp16: 1 + 2^-11 is a tie between 1 and 1 + 2^-10 -> 1 (even); bf16: 1 + 2^-8 -> 1
    y = np.array([[1.0], [2.0 ** -11], [2.0 ** -8]])
    dst = np.array([[0, 1]])
    assert ocombine.combine_rows(y, dst, row_dtype="fp16")[0, 0] == 1.0
    dst2 = np.array([[0, 2]])
    assert ocombine.combine_rows(y, dst2, row_dtype="bf16")[0, 0] == 1.0
    # just above the fp16 tie rounds up
    y3 = np.array([[1.0], [2.0 ** -11 + 2.0 ** -20]])
    assert ocombine.combine_rows(y3, np.array([[0, 1]]), row_dtype="fp16")[0, 0] == 1.0 + 2.0 ** -10


def test_shared_rows_join_before_the_one_rounding():
    # routed sum 1 + 3*2^-9 and shared rows -2^-9: the fp32 sum 1 + 2^-8 is a
    # bf16 tie that rounds to even, 1.0; rounding the routed part first would
    # give 1 + 2^-7 and keep it
    y = np.array([[1.0 + 3 * 2.0 ** -9]])
    dst = np.array([[0]])
    shared = np.array([[-2.0 ** -9]])
    assert ocombine.combine_rows(y, dst, shared=shared)[0, 0] == 1.0
    routed_first = bf16.round_to_bf16(bf16.round_to_bf16(1.0 + 3 * 2.0 ** -9) - 2.0 ** -9)
    assert routed_first == 1.0 + 2.0 ** -7


def test_score_before_and_after_the_experts_agree_for_identity_experts():
    # with identity experts, applying the score before (permute_weighted, then a
    # unit-weight combine) and after (the weighted combine) give the same
    # sum up to the roundings each path makes
    rng = np.random.default_rng(9)
    T, k, E, H = 12, 2, 4, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx = oroute.select(logits, k)
    w = oroute.weights(logits, idx)
    L = olayout.layout(idx, E, 1, -1, 4)
    x = bf16.round_to_bf16(rng.standard_normal((T, H)))
    rows = int(L["offsets"][-1])
    xp_pre, _ = opermute.permute_weighted(x, L["dst_row"], w, rows)
    pre = ocombine.combine_rows(xp_pre, L["dst_row"], None)
    post = ocombine.combine_rows(opermute.permute(x, L["src_row"], k), L["dst_row"], w)
    exact = ocombine.combine_exact(opermute.permute(x, L["src_row"], k), L["dst_row"], w)
    assert np.abs(pre - exact).max() <= 2.0 ** -6 * np.abs(exact).max()
    assert np.abs(post - exact).max() <= 2.0 ** -7 * np.abs(exact).max()


def test_permute_weighted_rounds_the_fp32_product_once():
    # Score applied before the experts (DeepSpeed PR #8847, section "Change",
    # score_apply="pre"): the row is the fp32 product w * x rounded once to
    # bf16. Worked by hand, w = 1 + 2^-9 + 2^-17 (an fp32 number) and
    # x = 2 - 2^-7 (a bf16 number): the exact product is
    # 2 - 2^-7 + 2^-8 - 2^-16 + 2^-16 - 2^-24 = 2 - 2^-8 - 2^-24. It sits half
    # way between the fp32 neighbours 2 - 2^-8 - 2^-23 (odd significand) and
    # 2 - 2^-8 (even), so the fp32 product is 2 - 2^-8: the midpoint of the
    # bf16 neighbours 2 - 2^-7 (odd) and 2, which ties to the even 2.0.
    # The two other readings give 2 - 2^-7 = 1.9921875 here:
    #  * rounding the weight to bf16 first: w is below the midpoint 1 + 2^-8,
    #    so bf16(w) = 1 and bf16(1 * x) = x;
    #  * rounding the exact product straight to bf16: it lies below the
    #    midpoint 2 - 2^-8.
    # (No single input can make all three readings differ: rounding w to bf16
    # moves the product by at most one bf16 unit of it, so the weight-first
    # value always equals one of the other two. The second case below covers
    # the weight-first reading where the other two agree.)
    w = np.array([[1 + 2.0 ** -9 + 2.0 ** -17]], dtype=np.float32)
    assert float(w[0, 0]) == 1 + 2.0 ** -9 + 2.0 ** -17
    x = np.array([[2 - 2.0 ** -7]])
    rows, written = opermute.permute_weighted(x, np.array([[0]]), w, 1)
    assert written.tolist() == [True]
    assert rows[0, 0] == 2.0
    # Second case: w = 1 + 2^-8 + 2^-10, x = 1.5. The product 1.50732421875 is
    # exact in fp32 and above the bf16 midpoint 1.50390625, so the row is
    # 1.5078125. Rounding the weight first gives bf16(w) = 1 + 2^-7 (w lies
    # above the midpoint 1 + 2^-8), and 1.5 * (1 + 2^-7) = 1.51171875 is the
    # midpoint of 1.5078125 (odd) and 1.515625 (even): 1.515625.
    w2 = np.array([[1 + 2.0 ** -8 + 2.0 ** -10]], dtype=np.float32)
    rows2, _ = opermute.permute_weighted(np.array([[1.5]]), np.array([[0]]), w2, 1)
    assert rows2[0, 0] == 1.5078125
    # rows no slot points at stay unwritten
    rows3, written3 = opermute.permute_weighted(np.array([[1.0], [2.0]]), np.array([[1], [-1]]),
                                                np.ones((2, 1), np.float32), 3)
    assert written3.tolist() == [False, True, False] and rows3[1, 0] == 1.0


# ---------------------------------------------------------------- combine error bound

def test_combine_bound_holds_for_the_fp32_sum():
    # a-priori bound of the fused restore against the exact sum: gamma_n
    # (n = local slots) times sum |w y|, plus half a bf16 unit of the result
    rng = np.random.default_rng(21)
    T, k, H, R = 512, 8, 64, 4096
    dst = np.stack([rng.permutation(R)[:k] for _ in range(T)])
    dst[::7, 3] = -1  # some slots of other shares
    w = rng.random((T, k)).astype(np.float32)
    y = bf16.round_to_bf16(rng.standard_normal((R, H)))
    exact = ocombine.combine_exact(y, dst, w)
    bound = ocombine.combine_error_bound(y, dst, w)
    fused = ocombine.combine_bf16(y, dst, w)
    assert (np.abs(fused - exact) <= bound).all()
    # a sum on a bf16 midpoint: 1 + 2^-8 ties to 1.0, an error of exactly
    # half a bf16 unit, which is all but the whole bound
    y1, w1, d1 = np.array([[1.0], [2.0 ** -8]]), np.ones((1, 2), np.float32), np.array([[0, 1]])
    err1 = abs(ocombine.combine_bf16(y1, d1, w1)[0, 0] - (1 + 2.0 ** -8))
    b1 = ocombine.combine_error_bound(y1, d1, w1)[0, 0]
    assert err1 == 2.0 ** -8 and 0.99 * b1 < err1 <= b1
    # rows that cancel: the fp32 product (1 + 2^-23)(1 + 2^-7) loses its 2^-30
    # term, the sum with -(1 + 2^-7) is 2^-23 where the exact value is
    # 2^-23 + 2^-30. That error is twice half a bf16 unit of the result
    # (2^-31): a bound of half a unit alone would reject the FP32 restore,
    # the gamma_n term admits it
    y2 = np.array([[1.0 + 2.0 ** -7], [-(1.0 + 2.0 ** -7)]])
    w2 = np.array([[1.0 + 2.0 ** -23, 1.0]], dtype=np.float32)
    d2 = np.array([[0, 1]])
    err2 = abs(ocombine.combine_bf16(y2, d2, w2)[0, 0] - ocombine.combine_exact(y2, d2, w2)[0, 0])
    assert err2 == 2.0 ** -30
    assert err2 <= ocombine.combine_error_bound(y2, d2, w2)[0, 0]


def test_combine_bound_rejects_plausible_mistakes():
    # the bound is tight enough that a dropped slot, a bf16 running sum (the
    # default restore) or bf16-rounded weights break it on Gaussian rows
    rng = np.random.default_rng(22)
    T, E, k, H = 2048, 64, 8, 128
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oroute.route(logits, k)
    L = olayout.layout(idx, E, 1, -1, 1)
    y = bf16.round_to_bf16(rng.standard_normal((L["m_cap"], H)))
    dst = L["dst_row"]
    exact = ocombine.combine_exact(y, dst, w)
    bound = ocombine.combine_error_bound(y, dst, w)
    assert not (np.abs(ocombine.restore_default(y, dst, w) - exact) <= bound).all()
    dropped = dst.copy()
    dropped[:, -1] = -1
    assert not (np.abs(ocombine.combine_bf16(y, dropped, w) - exact) <= bound).all()
    wb = bf16.round_to_bf16(w.astype(np.float64))
    assert not (np.abs(ocombine.combine_bf16(y, dst, wb) - exact) <= bound).all()
    # the exact sum rounded once obeys it (half a unit is inside the bound)
    assert (np.abs(bf16.round_to_bf16(exact) - exact) <= bound).all()
