"""Pins of the oracle's router for non-finite logits (a masked expert at -inf, a NaN logit
counted as -inf) and for the softmax before the top-k without renormalisation (Transformer
Engine guide "Mixture of Experts", Router: use_pre_softmax; Token combine: pre-softmax top-1
weights are not one); no GPU."""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O


def _brute_topk(row, k):
    # plain Python: sort (key descending, id ascending) with NaN as -inf
    keyed = [(-(-math.inf if math.isnan(v) else v), e) for e, v in enumerate(row)]
    return [e for _, e in sorted(keyed)[:k]]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # the all-masked rows
def test_masked_and_nan_logits_still_give_k_valid_ids():
    rng = np.random.default_rng(0)
    T, E, k = 64, 12, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    # rows with fewer than k finite logits: the -inf / NaN experts fill the rest, lowest id
    # first; a fully masked row; a NaN row
    for t in range(0, T, 2):
        nmask = rng.integers(E - k, E + 1)
        cols = rng.choice(E, size=nmask, replace=False)
        lg[t, cols[: nmask // 2]] = -np.inf
        lg[t, cols[nmask // 2:]] = np.nan
    lg[1, :] = -np.inf
    lg[3, :] = np.nan
    idx = O.topk_select(lg, k)
    assert ((idx >= 0) & (idx < E)).all()
    for t in range(T):
        assert len(set(idx[t].tolist())) == k
        assert idx[t].tolist() == _brute_topk([float(v) for v in lg[t]], k), t
    assert idx[1].tolist() == list(range(k)) and idx[3].tolist() == list(range(k))
    # with the group option (every group kept) and without it the choice is the same
    assert np.array_equal(O.topk_select_ext(lg, k, O.SOFTMAX_POST, None, 3, 3), idx)
    # the kept -inf / NaN experts get weight 0 when a finite logit remains
    for score in (O.SOFTMAX_PRE_RENORM, O.SOFTMAX_POST, O.SOFTMAX_PRE, O.SIGMOID,
                  O.SQRTSOFTPLUS):
        q = O.topk_probs(lg, idx, score)
        sel = np.take_along_axis(np.where(np.isnan(lg), -np.inf, lg), idx.astype(np.int64), 1)
        fin = np.isfinite(sel).any(axis=1)
        assert (q[fin][~np.isfinite(sel[fin])] == 0).all()
        assert np.isfinite(q[fin]).all()


def test_pre_softmax_weights_are_the_full_softmax_probabilities():
    rng = np.random.default_rng(1)
    T, E, k = 40, 10, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx = O.topk_select(lg, k)
    q = O.topk_probs(lg, idx, O.SOFTMAX_PRE, exact=True)
    p = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(q, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=1e-14, atol=0)
    # k = E: the kept weights are the whole softmax and sum to one
    qa = O.topk_probs(lg, O.topk_select(lg, E), O.SOFTMAX_PRE, exact=True)
    assert np.allclose(qa.sum(axis=1), 1.0, rtol=1e-14)
    # renormalising them gives the renormalised score function
    qr = O.topk_probs(lg, idx, O.SOFTMAX_PRE_RENORM, exact=True)
    assert np.allclose(q / q.sum(axis=1, keepdims=True), qr, rtol=1e-14)
    # top-1: not one (the guide's point that these weights must still be applied)
    q1 = O.topk_probs(lg, O.topk_select(lg, 1), O.SOFTMAX_PRE)
    assert (q1 < 1.0).all() and (q1 > 1.0 / E).all()
    # group values before the top-k are the same probabilities as with renormalisation
    assert np.array_equal(O.selection_keys(lg, O.SOFTMAX_PRE)[1],
                          O.selection_keys(lg, O.SOFTMAX_PRE_RENORM)[1])


def test_pre_softmax_backward_matches_finite_differences():
    rng = np.random.default_rng(2)
    T, E, k = 5, 7, 2
    lg = rng.standard_normal((T, E))
    idx = O.topk_select(lg, k)
    dq = rng.standard_normal((T, k))
    got = O.router_backward(lg, idx, dq, O.SOFTMAX_PRE, exact=True)
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            fd = ((O.topk_probs(lp, idx, O.SOFTMAX_PRE, exact=True) -
                   O.topk_probs(lm, idx, O.SOFTMAX_PRE, exact=True)) * dq).sum() / (2 * eps)
            assert abs(fd - got[t, e]) <= 1e-8 + 1e-6 * abs(fd), (t, e, fd, got[t, e])
    # unlike the renormalised form, the experts not kept get a gradient: -p_e sum_j q_j dq_j
    kept = np.zeros((T, E), bool)
    kept[np.arange(T)[:, None], idx] = True
    p = softmax(lg, axis=1)
    q = np.take_along_axis(p, idx.astype(np.int64), 1)
    want = -p * (q * dq).sum(axis=1, keepdims=True)
    assert np.allclose(got[~kept], want[~kept], rtol=1e-12, atol=1e-15)
    # and each row sums to zero (a softmax is shift invariant)
    assert np.allclose(got.sum(axis=1), 0.0, atol=1e-14)


@pytest.mark.parametrize("score", [O.SOFTMAX_PRE])
def test_pre_softmax_layer_backward_through_the_router(score):
    # central differences of the whole layer through the router projection
    import workloads as W
    w = W.custom("fdp", T=5, H=8, E=4, k=2, I=4, score=score)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((w.T, w.H))
    wgu = rng.standard_normal((w.E, w.H, 2 * w.I)) * 0.5
    wd = rng.standard_normal((w.E, w.I, w.H)) * 0.5
    wr = rng.standard_normal((w.E, w.H)) * 0.5
    dy = rng.standard_normal((w.T, w.H))

    def loss(wr_):
        lg = O.gate_logits(x, wr_, exact=True)
        r = O.moe_forward(x, lg, wgu, wd, w.k, score, w.I, exact=True)
        return float((r["y"] * dy).sum()), r

    _, fwd = loss(wr)
    g = O.moe_backward(fwd, dy, wgu, wd, w.I, exact=True, w_router_bits=wr)
    eps = 1e-6
    for i in range(wr.size):
        old = wr.flat[i]
        wr.flat[i] = old + eps
        lp, rp = loss(wr)
        wr.flat[i] = old - eps
        lm, rm = loss(wr)
        wr.flat[i] = old
        assert np.array_equal(rp["topk_idx"], rm["topk_idx"])
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - g["dw_router"].flat[i]) <= 1e-7 * np.abs(g["dw_router"]).max() + 1e-6 * abs(fd)
