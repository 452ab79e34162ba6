"""Pins of the oracle's router options: sqrtsoftplus against closed forms and a library
identity, scaling, expert bias (selection only), grouped routing (special cases that
reduce to plain top-k, a hand-worked example, and a brute-force check of the group
choice), the bit-packed routing map, the expert-bias update, and the backward of the
new score function and of scaling by central differences; no GPU."""
import itertools

import numpy as np
import pytest

import oracle as O


def test_sqrtsoftplus_closed_forms():
    l = np.array([0.0, 30.0, -30.0, 1.5, -2.25])
    s = O.score_values(l, O.SQRTSOFTPLUS)
    assert np.allclose(s ** 2, np.logaddexp(0.0, l), rtol=1e-14, atol=0)
    assert abs(s[0] - np.sqrt(np.log(2.0))) < 1e-15
    assert abs(s[1] - np.sqrt(30.0)) < 1e-12                  # log(1 + e^30) = 30 + e^-30
    assert abs(s[2] / np.exp(-15.0) - 1.0) < 1e-12            # sqrt(log(1 + e^-30)) ~ e^-15


def test_scaling_multiplies_the_weights():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((20, 12)).astype(np.float32)
    for score in (O.SOFTMAX_PRE_RENORM, O.SOFTMAX_POST, O.SIGMOID, O.SQRTSOFTPLUS):
        _, q1, *_ = O.router_topk(lg, 3, score)
        _, q2, *_ = O.router_topk(lg, 3, score, scaling_factor=2.0)
        assert np.array_equal(q2, 2.0 * q1)


def test_expert_bias_moves_the_choice_not_the_weights():
    rng = np.random.default_rng(1)
    T, E, k = 30, 10, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for score in (O.SIGMOID, O.SQRTSOFTPLUS):
        bias = np.zeros(E, np.float32)
        bias[7] = 100.0                                       # expert 7 always wins
        idx, q, counts, *_ = O.router_topk(lg, k, score, expert_bias=bias)
        assert (idx[:, 0] == 7).all() and counts[7] == T
        # weights are the unbiased scores of the chosen experts
        want = O.to_f32(O.score_values(np.take_along_axis(lg.astype(np.float64), idx.astype(np.int64), 1), score))
        assert np.array_equal(q, want)
        # the rest of the choice is the plain top-(k-1) of the other experts
        rest = np.where(np.arange(E) == 7, -np.inf, lg.astype(np.float64))
        assert np.array_equal(idx[:, 1], np.argmax(rest, axis=1))
    with pytest.raises(ValueError):
        O.router_topk(lg, k, O.SOFTMAX_POST, expert_bias=np.zeros(E, np.float32))


@pytest.mark.parametrize("score", [O.SOFTMAX_PRE_RENORM, O.SOFTMAX_POST, O.SIGMOID, O.SQRTSOFTPLUS])
def test_grouping_special_cases_reduce_to_plain_topk(score):
    rng = np.random.default_rng(2 + score)
    T, E, k = 40, 16, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    plain = O.topk_select(lg, k)
    # every group kept: no restriction
    assert np.array_equal(O.topk_select_ext(lg, k, score, None, 4, 4), plain)
    # one expert per group, k groups kept (m = 1): the k best experts
    assert np.array_equal(O.topk_select_ext(lg, k, score, None, E, k), plain)


def test_grouping_worked_example():
    # 8 experts in 4 groups of 2, k = 2 from 1 group (m = 2), scores = logits (softmax
    # after the top-k): group sums 5, 6, 5, 0, so group 1 (experts 2, 3) wins although
    # experts 0 and 4 have the larger logits; the tie 3 = 3 goes to expert 2 first
    lg = np.array([[5.0, 0.0, 3.0, 3.0, 4.0, 1.0, 0.0, 0.0]], np.float32)
    assert O.topk_select_ext(lg, 2, O.SOFTMAX_POST, None, 4, 1).tolist() == [[2, 3]]
    # with k = 4 from 2 groups (m = 2): groups 1 and 0 (6, then 5 at the lower id)
    assert O.topk_select_ext(lg, 4, O.SOFTMAX_POST, None, 4, 2).tolist() == [[0, 2, 3, 1]]


def test_grouping_brute_force():
    # plain Python: score every group by its m best values, enumerate every set of
    # group_topk groups, and check the chosen experts sit in a best set and are that
    # set's k best
    rng = np.random.default_rng(5)
    T, E, G, gt, k = 25, 12, 4, 2, 4
    m = k // gt
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx = O.topk_select_ext(lg, k, O.SOFTMAX_POST, None, G, gt)
    gs = E // G
    for t in range(T):
        row = [float(v) for v in lg[t]]
        gscore = [sum(sorted(row[g * gs:(g + 1) * gs], reverse=True)[:m]) for g in range(G)]
        best = max(sum(gscore[g] for g in c) for c in itertools.combinations(range(G), gt))
        groups = {int(e) // gs for e in idx[t]}
        assert len(groups) <= gt
        chosen = sorted(groups)
        while len(chosen) < gt:  # the remaining kept group(s) need not hold a choice
            chosen.append(max((g for g in range(G) if g not in chosen), key=lambda g: gscore[g]))
        assert abs(sum(gscore[g] for g in chosen) - best) < 1e-6
        pool = sorted((row[e], -e) for g in chosen for e in range(g * gs, (g + 1) * gs))[::-1]
        assert [int(e) for e in idx[t]] == [-p[1] for p in pool[:k]]


def test_pack_routing_map_bit_order():
    rmap = np.zeros((2, 12), np.uint8)
    rmap[0, 0] = rmap[0, 9] = 1
    rmap[1, 7] = rmap[1, 8] = rmap[1, 11] = 1
    packed = O.pack_routing_map(rmap)
    assert packed.tolist() == [[1, 2], [128, 1 + 8]]


def test_expert_bias_update_worked_example():
    b = np.zeros(4, np.float32)
    assert np.array_equal(O.expert_bias_update(b, [10, 10, 10, 10], 1e-3), b)
    # mean 15: signs -1, +1, +1, +1 -> minus their mean 0.5
    got = O.expert_bias_update(b, [30, 10, 10, 10], 0.25)
    assert np.array_equal(got, np.array([-0.375, 0.125, 0.125, 0.125]))


@pytest.mark.parametrize("score", [O.SQRTSOFTPLUS, O.SIGMOID, O.SOFTMAX_POST])
def test_router_backward_with_scaling_matches_finite_differences(score):
    rng = np.random.default_rng(7 + score)
    T, E, k, c = 6, 9, 3, 2.5
    lg = rng.standard_normal((T, E))
    idx = O.topk_select(lg, k)
    dq = rng.standard_normal((T, k))
    got = O.router_backward(lg, idx, dq, score, exact=True, scaling_factor=c)
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            fp = (O.topk_probs(lp, idx, score, exact=True, scaling_factor=c) * dq).sum()
            fm = (O.topk_probs(lm, idx, score, exact=True, scaling_factor=c) * dq).sum()
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - got[t, e]) <= 1e-7 * np.abs(got).max() + 1e-6 * abs(fd), (t, e, fd, got[t, e])


def test_grouping_softmax_before_topk_sums_probabilities():
    # 4 experts in 2 groups of 2, k = 2 from one group (m = 2), softmax before the top-k:
    # a group's value is the sum of its experts' softmax probabilities.
    # Groups [2, 2] and [3, -10]: on probabilities the second wins (e^3 + e^-10 > 2 e^2)
    # while summed logits would keep the first (4 > -7).
    lg = np.array([[2.0, 2.0, 3.0, -10.0]], np.float32)
    assert O.topk_select_ext(lg, 2, O.SOFTMAX_PRE_RENORM, None, 2, 1).tolist() == [[2, 3]]
    assert O.topk_select_ext(lg, 2, O.SOFTMAX_POST, None, 2, 1).tolist() == [[0, 1]]
    # groups [2, 2] and [2.5, -10]: the sum keeps the first (2 e^2 > e^2.5), the best single
    # probability would keep the second
    lg = np.array([[2.0, 2.0, 2.5, -10.0]], np.float32)
    assert O.topk_select_ext(lg, 2, O.SOFTMAX_PRE_RENORM, None, 2, 1).tolist() == [[0, 1]]


def test_grouping_softmax_before_topk_brute_force():
    # plain Python with math.exp: every group scored by the sum of the softmax
    # probabilities of its m best experts, every set of group_topk groups enumerated
    import math
    rng = np.random.default_rng(6)
    T, E, G, gt, k = 25, 12, 4, 2, 4
    m = k // gt
    lg = (rng.standard_normal((T, E)) * 2.0).astype(np.float32)
    idx = O.topk_select_ext(lg, k, O.SOFTMAX_PRE_RENORM, None, G, gt)
    gs = E // G
    for t in range(T):
        row = [float(v) for v in lg[t]]
        mx = max(row)
        z = sum(math.exp(v - mx) for v in row)
        prob = [math.exp(v - mx) / z for v in row]
        gscore = [sum(sorted(prob[g * gs:(g + 1) * gs], reverse=True)[:m]) for g in range(G)]
        best = max(sum(gscore[g] for g in c) for c in itertools.combinations(range(G), gt))
        groups = {int(e) // gs for e in idx[t]}
        chosen = sorted(groups)
        while len(chosen) < gt:
            chosen.append(max((g for g in range(G) if g not in chosen), key=lambda g: gscore[g]))
        assert abs(sum(gscore[g] for g in chosen) - best) < 1e-6
        pool = sorted((row[e], -e) for g in chosen for e in range(g * gs, (g + 1) * gs))[::-1]
        assert [int(e) for e in idx[t]] == [-p[1] for p in pool[:k]]
