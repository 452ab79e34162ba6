"""Pins of the oracle's router projection and router backward: a selection special
case of the projection, a selection special case of the routing-weight gradient,
the shift invariance of softmax scores, the equality of the two softmax orders, and
central finite differences of the whole layer through the router; no GPU."""
import numpy as np
import pytest

import oracle as O


def test_gate_logits_unit_rows_select_columns():
    # W_r rows that are unit vectors pick one hidden column each: logits are those
    # columns exactly (and a factor of 2 scales them exactly)
    rng = np.random.default_rng(3)
    T, H, E = 9, 16, 5
    x_bits = O.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x = O.bf16_bits_to_f64(x_bits)
    cols = np.array([7, 0, 15, 3, 7])
    w = np.zeros((E, H))
    w[np.arange(E), cols] = 1.0
    got = O.gate_logits(x_bits, O.f32_to_bf16_bits(w.astype(np.float32)))
    assert got.shape == (T, E)
    assert np.array_equal(got, x[:, cols])
    got2 = O.gate_logits(x_bits, O.f32_to_bf16_bits((2 * w).astype(np.float32)))
    assert np.array_equal(got2, 2 * x[:, cols])


def test_prob_grad_unit_upstream_selects_output_column():
    # dy[t] = unit vector at column a_t: d_prob[t,j] = out[row_of[t,j], a_t]
    rng = np.random.default_rng(4)
    T, H, k = 6, 8, 3
    row_of = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    out = rng.standard_normal((T * k, H))
    a = rng.integers(0, H, size=T)
    dy = np.zeros((T, H))
    dy[np.arange(T), a] = 1.0
    got = O.prob_grad(dy, out, row_of, exact=True)
    assert np.array_equal(got, out[row_of, a[:, None]])


def _router_case(seed, T=7, E=9, k=3):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E))
    idx = O.topk_select(logits, k)
    dq = rng.standard_normal((T, k))
    return logits, idx, dq


def test_softmax_gradients_sum_to_zero_and_orders_agree():
    # adding a constant to a token's logits leaves softmax weights unchanged, so each
    # row of d_logits sums to 0; softmax-then-renormalise and softmax-of-the-kept
    # are one function of the kept logits, so their gradients agree and the
    # unselected logits get none
    logits, idx, dq = _router_case(11)
    pre = O.router_backward(logits, idx, dq, O.SOFTMAX_PRE_RENORM, exact=True)
    post = O.router_backward(logits, idx, dq, O.SOFTMAX_POST, exact=True)
    scale = np.abs(pre).max()
    assert scale > 0.05
    assert np.abs(pre.sum(axis=1)).max() < 1e-14
    assert np.abs(post.sum(axis=1)).max() < 1e-14
    assert np.abs(pre - post).max() < 1e-14
    mask = np.ones_like(pre, dtype=bool)
    mask[np.arange(len(idx))[:, None], idx] = False
    assert np.abs(pre[mask]).max() < 1e-15 and not post[mask].any()


def test_sigmoid_gradient_is_derivative_of_each_weight():
    # q_j = sigmoid(l_j) on its own: central differences of each weight
    logits, idx, dq = _router_case(12, k=2)
    got = O.router_backward(logits, idx, dq, O.SIGMOID, exact=True)
    eps = 1e-6
    rows = np.arange(len(idx))[:, None]
    for j in range(idx.shape[1]):
        lp, lm = logits.copy(), logits.copy()
        lp[rows[:, 0], idx[:, j]] += eps
        lm[rows[:, 0], idx[:, j]] -= eps
        qp = O.topk_probs(lp, idx, O.SIGMOID, exact=True)[:, j]
        qm = O.topk_probs(lm, idx, O.SIGMOID, exact=True)[:, j]
        fd = dq[:, j] * (qp - qm) / (2 * eps)
        assert np.allclose(got[rows[:, 0], idx[:, j]], fd, rtol=1e-7, atol=1e-10)


def _layer(x, w_r, wgu, wd, dy, k, score, I, logits=None, placement=O.PLACE_COMBINE):
    if logits is None:
        logits = O.gate_logits(x, w_r, exact=True)
    f = O.moe_forward(x, logits, wgu, wd, k, score, I, exact=True, placement=placement)
    return float((f["y"] * dy).sum()), f


def _margin(logits, k):
    s = -np.sort(-logits, axis=1)
    return (s[:, k - 1] - s[:, k]).min()


@pytest.mark.parametrize("score,k,placement", [(O.SOFTMAX_PRE_RENORM, 3, O.PLACE_COMBINE),
                                               (O.SOFTMAX_POST, 2, O.PLACE_COMBINE),
                                               (O.SIGMOID, 2, O.PLACE_COMBINE),
                                               (O.SQRTSOFTPLUS, 2, O.PLACE_COMBINE),
                                               (O.SOFTMAX_PRE_RENORM, 3, O.PLACE_INPUT),
                                               (O.SIGMOID, 1, O.PLACE_INPUT),
                                               (O.SOFTMAX_PRE_RENORM, 3, O.PLACE_ACTIVATION),
                                               (O.SIGMOID, 1, O.PLACE_ACTIVATION),
                                               (O.SOFTMAX_PRE, 2, O.PLACE_ACTIVATION)])
def test_layer_gradients_through_router_match_finite_differences(score, k, placement):
    T, H, E, I = 6, 16, 7, 8
    rng = np.random.default_rng(30 + score)
    x = rng.standard_normal((T, H))
    w_r = rng.standard_normal((E, H)) * 0.5
    wgu = rng.standard_normal((E, H, 2 * I)) * 0.5
    wd = rng.standard_normal((E, I, H)) * 0.5
    dy = rng.standard_normal((T, H))
    _, fwd = _layer(x, w_r, wgu, wd, dy, k, score, I, placement=placement)
    # the top-k choice must not move under the perturbations below
    assert _margin(fwd["logits"], k) > 1e-3
    g = O.moe_backward(fwd, dy, wgu, wd, I, exact=True, w_router_bits=w_r)
    eps = 1e-6

    def check(name, arr, grad, loss):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        scale = np.abs(gflat).max()
        assert scale > 1e-3
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp = loss()
            flat[i] = old - eps
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gflat[i]) <= 1e-7 * scale + 1e-6 * abs(fd), (name, i, fd, gflat[i])

    P = placement
    logits = fwd["logits"].copy()
    check("logits", logits, g["d_logits"], lambda: _layer(x, w_r, wgu, wd, dy, k, score, I, logits, P)[0])
    check("w_router", w_r, g["dw_router"], lambda: _layer(x, w_r, wgu, wd, dy, k, score, I, None, P)[0])
    check("x", x, g["dx"], lambda: _layer(x, w_r, wgu, wd, dy, k, score, I, None, P)[0])
    check("w_gu", wgu, g["dw_gu"], lambda: _layer(x, w_r, wgu, wd, dy, k, score, I, None, P)[0])
    check("w_down", wd, g["dw_down"], lambda: _layer(x, w_r, wgu, wd, dy, k, score, I, None, P)[0])


def test_backward_without_router_weight_is_unchanged():
    # the router term of dx is d_logits . W_r: with W_r = 0 it vanishes and dx is the
    # expert path's alone, while dW_r = d_logits^T x does not depend on W_r
    T, H, E, I, k = 5, 8, 4, 4, 2
    rng = np.random.default_rng(40)
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E))
    wgu = rng.standard_normal((E, H, 2 * I))
    wd = rng.standard_normal((E, I, H))
    dy = rng.standard_normal((T, H))
    f = O.moe_forward(x, logits, wgu, wd, k, O.SOFTMAX_PRE_RENORM, I, exact=True)
    a = O.moe_backward(f, dy, wgu, wd, I, exact=True)
    b = O.moe_backward(f, dy, wgu, wd, I, exact=True, w_router_bits=np.zeros((E, H)))
    assert np.array_equal(a["dx"], b["dx"])
    assert np.array_equal(b["dw_router"], b["d_logits"].T @ x) and b["dw_router"].any()


def test_input_placement_equals_combine_placement_for_unit_weights():
    # top-1 with softmax after the top-k: every weight is exactly 1, so scaling the inputs
    # or the outputs by it gives bit-identical layers (rounded mode)
    rng = np.random.default_rng(50)
    T, H, E, I = 12, 32, 4, 16
    x = O.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    wgu = O.f32_to_bf16_bits((rng.standard_normal((E, H, 2 * I)) * 0.1).astype(np.float32))
    wd = O.f32_to_bf16_bits((rng.standard_normal((E, I, H)) * 0.1).astype(np.float32))
    a = O.moe_forward(x, lg, wgu, wd, 1, O.SOFTMAX_POST, I)
    b = O.moe_forward(x, lg, wgu, wd, 1, O.SOFTMAX_POST, I, placement=O.PLACE_INPUT)
    assert (a["topk_prob"] == 1.0).all()
    assert np.array_equal(a["y"], b["y"])


def test_activation_placement_equals_combine_placement():
    # ScaledSwiGLU with a bias-free FC2: (p h) W = p (h W), so in exact arithmetic the
    # weights on the SwiGLU output give the layer of weights in the combine; with unit
    # weights (top-1, softmax after the top-k) the rounded layers are bit-identical too,
    # forward and backward
    rng = np.random.default_rng(51)
    T, H, E, I, k = 10, 16, 5, 8, 3
    x = rng.standard_normal((T, H))
    lg = rng.standard_normal((T, E))
    wgu = rng.standard_normal((E, H, 2 * I)) * 0.5
    wd = rng.standard_normal((E, I, H)) * 0.5
    dy = rng.standard_normal((T, H))
    a = O.moe_forward(x, lg, wgu, wd, k, O.SOFTMAX_PRE_RENORM, I, exact=True)
    b = O.moe_forward(x, lg, wgu, wd, k, O.SOFTMAX_PRE_RENORM, I, exact=True,
                      placement=O.PLACE_ACTIVATION)
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-14)
    # the expert outputs differ by exactly the weight factor
    rw = O.row_weights(a["topk_prob"], a["row_of"], T * k)
    assert np.allclose(b["out"], a["out"] * rw[:, None], rtol=1e-12, atol=1e-14)
    ga = O.moe_backward(a, dy, wgu, wd, I, exact=True)
    gb = O.moe_backward(b, dy, wgu, wd, I, exact=True)
    for key in ("dx", "dw_gu"):
        assert np.allclose(ga[key], gb[key], rtol=1e-10, atol=1e-12), key
    # dW_down differs: it pairs the scaled h with the unweighted d_out, which is the same
    # product in exact arithmetic
    assert np.allclose(ga["dw_down"], gb["dw_down"], rtol=1e-10, atol=1e-12)
    xb = O.f32_to_bf16_bits(x.astype(np.float32))
    lg32 = lg.astype(np.float32)
    wgub = O.f32_to_bf16_bits((wgu * 0.2).astype(np.float32))
    wdb = O.f32_to_bf16_bits((wd * 0.2).astype(np.float32))
    dyb = O.f32_to_bf16_bits(dy.astype(np.float32))
    a = O.moe_forward(xb, lg32, wgub, wdb, 1, O.SOFTMAX_POST, I)
    b = O.moe_forward(xb, lg32, wgub, wdb, 1, O.SOFTMAX_POST, I, placement=O.PLACE_ACTIVATION)
    assert (a["topk_prob"] == 1.0).all()
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["y"], b["y"])
    ga = O.moe_backward(a, dyb, wgub, wdb, I)
    gb = O.moe_backward(b, dyb, wgub, wdb, I)
    for key in ("dx", "dw_gu", "dw_down", "dgu"):
        assert np.array_equal(ga[key], gb[key]), key
