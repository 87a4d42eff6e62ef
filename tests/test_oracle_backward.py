"""Pins of the backward oracle (oracle/backward.py): each gradient is checked
against something other than its own formula -- the forward oracles through
an adjoint identity or a finite difference, invariants of the softmax, and
the size of the FP32 score-gradient error the pages report."""
import json
import os

import numpy as np
import pytest

from oracle import backward as ob, bf16, combine as ocombine, layout as olayout
from oracle import permute as opermute, route as oroute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, T=24, E=8, k=3, ep=2, share=1, H=16, align=4):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx = oroute.select(logits, k)
    w = oroute.weights(logits, idx)
    L = olayout.layout(idx, E, ep, share, align)
    rows = int(L["offsets"][-1])
    y = bf16.round_to_bf16(rng.standard_normal((max(rows, 1), H)))
    G = bf16.round_to_bf16(rng.standard_normal((T, H)))
    return logits, idx, w, L, y, G


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_score_gradient_is_the_derivative_of_the_combine(seed):
    # combine_exact is linear in the weights: moving w[t, s] by eps moves
    # <G, out> by eps * <G[t], y[dst_row[t, s]]> -- the forward, not the formula
    _, idx, w, L, y, G = _case(seed)
    dst = L["dst_row"]
    gw = ob.combine_backward_scores(G, y, dst)
    base = (ocombine.combine_exact(y, dst, w) * G).sum()
    eps = 2.0 ** -10
    for t, s in [(0, 0), (3, 1), (7, 2), (11, 0), (23, 2)]:
        w2 = w.copy()
        w2[t, s] += eps
        fd = ((ocombine.combine_exact(y, dst, w2) * G).sum() - base) / eps
        assert fd == pytest.approx(gw[t, s], rel=1e-9, abs=1e-9), (t, s)
        if dst[t, s] < 0:
            assert gw[t, s] == 0.0


@pytest.mark.parametrize("seed", [3, 4])
def test_row_gradient_is_the_adjoint_of_the_combine(seed):
    # with weights that are powers of two, w * G is exact in bf16, so the
    # rounded row gradient must satisfy <combine(y), G> = <y, grad_y> exactly
    _, _, _, L, y, G = _case(seed)
    dst = L["dst_row"]
    rng = np.random.default_rng(seed + 100)
    w = 2.0 ** -rng.integers(0, 4, size=dst.shape).astype(np.float64)
    gy, written = ob.combine_backward_rows(G, dst, w, y.shape[0])
    lhs = (ocombine.combine_exact(y, dst, w) * G).sum()
    rhs = (y[written] * gy[written]).sum()
    assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-12)
    # exactly the local rows are written, padding and other shares' rows are not
    assert set(np.nonzero(written)[0]) == set(dst[dst >= 0].tolist())


def test_row_gradient_rounds_the_fp32_product_once():
    # w = 1/3 (fp32) times G = 1 + 2^-7: the fp32 product rounds to bf16 once
    w = np.array([[1.0 / 3.0]])
    G = np.array([[1.0 + 2.0 ** -7]])
    dst = np.array([[0]])
    gy, _ = ob.combine_backward_rows(G, dst, w, 1)
    want = bf16.round_to_bf16(float(np.float32(np.float32(1.0 / 3.0) * np.float32(1.0 + 2.0 ** -7))))
    assert gy[0, 0] == want


def test_worked_example_gradients():
    # the hand-computed layout of tests/golden (all experts local); y[r] = r + 1
    # and G = 1 in one column make every gradient a small closed form
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    idx = np.array(g["topk_idx"], dtype=np.int32)
    w = np.array(g["topk_w"], dtype=np.float64)
    dst = np.array(g["shares"]["-1"]["dst_row"], dtype=np.int64)
    rows = len(g["shares"]["-1"]["src_row"])
    y = (np.arange(rows, dtype=np.float64) + 1.0)[:, None]
    G = np.ones((4, 1))
    gw = ob.combine_backward_scores(G, y, dst)
    np.testing.assert_array_equal(gw, dst + 1.0)  # <1, y[r]> = r + 1
    gy, written = ob.combine_backward_rows(G, dst, w, rows)
    for t in range(4):
        for s in range(2):
            assert gy[dst[t, s], 0] == bf16.round_to_bf16(float(np.float32(w[t, s])))
    assert written.sum() == 8
    # routing gradient of token 0 (weights sigma(1), 1 - sigma(1)): with g = (r0+1, r1+1)
    gl = ob.route_backward(idx, w, gw, 4)
    w0, w1 = w[0]
    g0, g1 = gw[0]
    assert gl[0, idx[0, 0]] == pytest.approx(w0 * w1 * (g0 - g1), rel=1e-12)
    assert gl[0, idx[0, 1]] == pytest.approx(w0 * w1 * (g1 - g0), rel=1e-12)


@pytest.mark.parametrize("seed", [5, 6])
def test_permute_gradient_is_the_adjoint_of_the_permute(seed):
    # small integers: every sum is exact, so <permute(x), Gp> = <x, grad_x>
    rng = np.random.default_rng(seed)
    _, _, _, L, _, _ = _case(seed)
    dst, src = L["dst_row"], L["src_row"]
    T, k = dst.shape
    x = rng.integers(-4, 5, size=(T, 8)).astype(np.float64)
    Gp = rng.integers(-4, 5, size=(src.shape[0], 8)).astype(np.float64)
    xp = opermute.permute(x, src, k)
    valid = src >= 0
    lhs = (xp[valid] * Gp[valid]).sum()
    rhs = (x * ob.permute_backward(Gp, dst)).sum()
    assert lhs == rhs
    # a token with no local slot gets a zero row
    none_local = (dst < 0).all(axis=1)
    assert not ob.permute_backward(Gp, dst)[none_local].any()


def test_permute_gradient_sums_in_fp32_slot_order():
    # 1 + 2^-24 + 2^-24: slot order in fp32 keeps 1.0 (each addition rounds
    # back); an fp64 sum would give 1 + 2^-23
    Gp = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]])
    dst = np.array([[0, 1, 2]])
    assert ob.permute_backward(Gp, dst)[0, 0] == np.float32(1.0)


@pytest.mark.parametrize("seed", [7, 8])
def test_routing_gradient_matches_finite_differences(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 6, 10, 4
    # well separated logits: small moves never change the selection
    logits = np.stack([rng.permutation(E) * 0.7 for _ in range(T)]).astype(np.float64)
    idx = oroute.select(logits.astype(np.float32), k)
    g = rng.standard_normal((T, k))
    gl = ob.route_backward(idx, oroute.weights(logits, idx), g, E)

    def loss(lg):
        return (oroute.weights(lg, idx) * g).sum()

    eps = 1e-6
    for t in range(T):
        for e in range(E):
            lp, lm = logits.copy(), logits.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            fd = (loss(lp) - loss(lm)) / (2 * eps)
            assert fd == pytest.approx(gl[t, e], abs=1e-8), (t, e)
    np.testing.assert_allclose(gl.sum(axis=1), 0.0, atol=1e-15)


def test_routing_gradient_special_cases():
    # top-1: the weight is 1 whatever the logit, so no gradient reaches it
    idx = np.array([[2], [0]], dtype=np.int32)
    gl = ob.route_backward(idx, np.ones((2, 1)), np.array([[3.0], [-1.0]]), 4)
    assert not gl.any()
    # equal upstream gradients on every slot: the softmax is shift invariant
    idx = np.array([[0, 1, 2]], dtype=np.int32)
    w = np.array([[0.5, 0.3, 0.2]])
    gl = ob.route_backward(idx, w, np.full((1, 3), 2.5), 3)
    np.testing.assert_allclose(gl, 0.0, atol=1e-15)


def test_fp32_score_gradient_error_is_the_pages_size():
    # the pages: FP32 score gradient at hidden 6144, relative L2 error about
    # 8.4e-8 against FP64. An fp32 pairwise reduction of the exact products
    # lands in that range; a bf16 rounding of the result would be ~1e-3.
    rng = np.random.default_rng(11)
    H, n = 6144, 64
    G = bf16.round_to_bf16(rng.standard_normal((n, H)))
    y = bf16.round_to_bf16(rng.standard_normal((n, H)))
    exact = np.einsum("th,th->t", G, y)
    fp32 = np.array([ob.pairwise_fp32_sum((G[t] * y[t]).astype(np.float32)) for t in range(n)],
                    dtype=np.float64)
    rel = np.linalg.norm(fp32 - exact) / np.linalg.norm(exact)
    assert 1e-9 < rel < 5e-7
    dst = np.arange(n)[:, None]
    assert (np.abs(fp32 - exact) <= ob.score_bound(G, y, dst)[:, 0]).all()
    as_bf16 = bf16.round_to_bf16(exact)
    assert np.linalg.norm(as_bf16 - exact) / np.linalg.norm(exact) > 1e-4


# ---------------------------------------------------------------- experts

from oracle import experts as oexperts  # noqa: E402


@pytest.mark.parametrize("seed", [21, 22])
def test_expert_gradients_match_finite_differences(seed):
    # every gradient of swiglu_backward against central differences of the
    # forward swiglu (fp64): a swapped gate/up, a missing silu' term or a
    # transposed weight would fail
    rng = np.random.default_rng(seed)
    m, H, I = 5, 6, 4
    x = rng.standard_normal((m, H))
    w1 = rng.standard_normal((H, I)) * 0.5
    w3 = rng.standard_normal((H, I)) * 0.5
    w2 = rng.standard_normal((I, H)) * 0.5
    dy = rng.standard_normal((m, H))
    dx, dw1, dw3, dw2 = oexperts.swiglu_backward(x, w1, w3, w2, dy)

    def loss(x_, w1_, w3_, w2_):
        return (oexperts.swiglu(x_, w1_, w3_, w2_) * dy).sum()

    eps = 1e-6
    for name, arr, grad in (("x", x, dx), ("w1", w1, dw1), ("w3", w3, dw3), ("w2", w2, dw2)):
        for _ in range(6):
            i = tuple(rng.integers(0, n) for n in arr.shape)
            args = {"x": x, "w1": w1, "w3": w3, "w2": w2}
            plus = {k: v.copy() for k, v in args.items()}
            minus = {k: v.copy() for k, v in args.items()}
            plus[name][i] += eps
            minus[name][i] -= eps
            fd = (loss(plus["x"], plus["w1"], plus["w3"], plus["w2"]) -
                  loss(minus["x"], minus["w1"], minus["w3"], minus["w2"])) / (2 * eps)
            assert fd == pytest.approx(grad[i], rel=1e-6, abs=1e-8), (name, i)


def test_expert_data_gradient_closed_form():
    # H = I = 1: y = silu(a x) (b x) c, so dy/dx = c (a b x) (2 s + a x s (1 - s))
    # with s = sigmoid(a x): checks silu' and the product rule by hand
    a, b, c, x = 0.7, -1.3, 2.0, 0.9
    dx = oexperts.swiglu_backward([[x]], [[a]], [[b]], [[c]], [[1.0]])[0][0, 0]
    s = 1.0 / (1.0 + np.exp(-a * x))
    assert dx == pytest.approx(c * a * b * x * (2 * s + a * x * s * (1 - s)), rel=1e-12)


def test_grouped_data_gradient_leaves_padding_zero():
    rng = np.random.default_rng(3)
    H, I = 4, 3
    ws = [tuple(rng.standard_normal(s) for s in ((H, I), (H, I), (I, H))) for _ in range(2)]
    offsets, counts = [0, 4, 8], [3, 2]
    xp = rng.standard_normal((8, H))
    dy = rng.standard_normal((8, H))
    dx = oexperts.grouped_swiglu_backward_data(xp, dy, offsets, counts, lambda e: ws[e])
    assert not dx[3].any() and not dx[6:].any()
    np.testing.assert_allclose(dx[4:6], oexperts.swiglu_backward(xp[4:6], *ws[1], dy[4:6])[0])


def test_row_gradient_is_the_fp32_product_rounded_once_more():
    # The row gradient is w * G as an fp32 product, then rounded to the bf16
    # row dtype. Worked by hand: w = 11228502 * 2^-24 (an fp32 number) and
    # G = 3 give the exact product 2 + 2^-7 + 2^-23, half an fp32 unit above
    # the fp32 number 2 + 2^-7; that tie goes to 2 + 2^-7 (even significand),
    # which is the midpoint between the bf16 numbers 2 and 2 + 2^-6 and ties
    # to 2. Rounding the exact product to bf16 directly would give 2 + 2^-6.
    w = np.array([[11228502 * 2.0 ** -24]], dtype=np.float32)
    rows, written = ob.combine_backward_rows(np.array([[3.0]]), np.array([[0]]), w, 1)
    assert written[0] and rows[0, 0] == 2.0
