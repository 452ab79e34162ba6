"""Pins of the oracle's auxiliary load-balancing loss (Transformer Engine guide "Mixture of
Experts", Load balancing: dense scores from the auxiliary-score helper, the loss from the
token counts, a gradient for every expert's logit), read as the Switch Transformer balance
loss coeff * E * sum_e f_e P_e with f_e = c_e / (k T); no GPU."""
import numpy as np
import pytest

import oracle as O

SCORES = [O.SOFTMAX_PRE_RENORM, O.SOFTMAX_POST, O.SOFTMAX_PRE, O.SIGMOID, O.SQRTSOFTPLUS]


@pytest.mark.parametrize("score", SCORES)
def test_dense_scores_are_a_distribution_over_the_experts(score):
    rng = np.random.default_rng(score)
    lg = rng.standard_normal((30, 9)).astype(np.float32)
    s = O.aux_scores(lg, score, exact=True)
    assert (s > 0).all() and np.allclose(s.sum(axis=1), 1.0, rtol=1e-14)
    # the order follows the logits (every score function here is increasing)
    assert np.array_equal(np.argsort(-s, axis=1, kind="stable"),
                          np.argsort(-lg.astype(np.float64), axis=1, kind="stable"))


@pytest.mark.parametrize("score", SCORES)
def test_balanced_routing_gives_coeff_and_no_gradient(score):
    # equal logits: every score 1/E; counts T k / E each: loss = coeff exactly, and with
    # uniform counts the loss is coeff whatever the scores, so the softmax-type gradient
    # vanishes (sum_e s_te = 1 for every token)
    T, E, k, coeff = 64, 8, 2, 1e-2
    lg = np.zeros((T, E), np.float32)
    counts = np.full(E, T * k // E)
    s = O.aux_scores(lg, score, exact=True)
    assert O.aux_loss(s, counts, T, k, coeff, exact=True) == pytest.approx(coeff, rel=1e-15)
    lg2 = np.random.default_rng(9).standard_normal((T, E)).astype(np.float32)
    s2 = O.aux_scores(lg2, score, exact=True)
    assert O.aux_loss(s2, counts, T, k, coeff, exact=True) == pytest.approx(coeff, rel=1e-14)
    g = O.aux_loss_backward(lg2, counts, T, k, coeff, score, exact=True)
    assert np.abs(g).max() < 1e-16


def test_all_tokens_on_one_expert():
    # every pair routed to expert 0: f_0 = 1, so loss = coeff E P_0 (the Switch form with
    # all load on one expert), which with uniform scores is coeff and with scores
    # concentrated on expert 0 approaches coeff E
    T, E, k, coeff = 16, 4, 1, 0.5
    counts = np.array([T * k, 0, 0, 0])
    s = np.full((T, E), 1.0 / E)
    assert O.aux_loss(s, counts, T, k, coeff, exact=True) == pytest.approx(coeff)
    s = np.zeros((T, E))
    s[:, 0] = 1.0
    assert O.aux_loss(s, counts, T, k, coeff, exact=True) == pytest.approx(coeff * E)


def test_loss_is_bilinear_in_counts_and_scores():
    rng = np.random.default_rng(4)
    T, E, k = 20, 6, 2
    s = O.aux_scores(rng.standard_normal((T, E)).astype(np.float32), O.SOFTMAX_PRE_RENORM)
    c1, c2 = rng.integers(0, 10, E), rng.integers(0, 10, E)
    a = O.aux_loss(s, c1, T, k, 1.0, exact=True) + O.aux_loss(s, c2, T, k, 1.0, exact=True)
    assert O.aux_loss(s, c1 + c2, T, k, 1.0, exact=True) == pytest.approx(a, rel=1e-14)
    # doubling the token total at fixed counts and scores of twice the tokens: f halves
    s2 = np.concatenate([s, s])
    assert O.aux_loss(s2, c1, 2 * T, k, 1.0, exact=True) == pytest.approx(
        O.aux_loss(s, c1, T, k, 1.0, exact=True) / 2, rel=1e-14)


@pytest.mark.parametrize("score", SCORES)
def test_gradient_matches_finite_differences(score):
    rng = np.random.default_rng(10 + score)
    T, E, k, coeff, dl = 6, 5, 2, 0.3, 1.7
    lg = rng.standard_normal((T, E))
    counts = rng.integers(0, 7, E)
    got = O.aux_loss_backward(lg, counts, T, k, coeff, score, d_loss=dl, exact=True)
    assert np.abs(got).max() > 0
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            fp = O.aux_loss(O.aux_scores(lp, score, exact=True), counts, T, k, coeff, exact=True)
            fm = O.aux_loss(O.aux_scores(lm, score, exact=True), counts, T, k, coeff, exact=True)
            fd = dl * (fp - fm) / (2 * eps)
            assert abs(fd - got[t, e]) <= 1e-9 * np.abs(got).max() + 1e-6 * abs(fd), (t, e, fd, got[t, e])
    if score in O.SOFTMAX_KINDS:  # shift invariance of a softmax row
        assert np.allclose(got.sum(axis=1), 0.0, atol=1e-15)
