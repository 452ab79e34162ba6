"""Pins of the oracle's router and dispatch against brute force, library routines
and closed forms; no GPU."""
import numpy as np
import pytest
import scipy.special as sp

import oracle as O
import workloads as W


def _brute_topk(l, k):
    # full sort of (-logit, expert) per row: lowest index wins a tie
    return np.array([[e for e in sorted(range(l.shape[1]), key=lambda e: (-float(l[t, e]), e))[:k]]
                     for t in range(l.shape[0])], dtype=np.int32)


@pytest.mark.parametrize("T,E,k", [(50, 4, 2), (40, 16, 1), (30, 128, 8), (20, 8, 8), (10, 256, 32)])
def test_topk_matches_full_sort(T, E, k):
    rng = np.random.default_rng(T * E + k)
    l = rng.standard_normal((T, E)).astype(np.float32)
    assert np.array_equal(O.topk_select(l, k), _brute_topk(l, k))
    # library cross-check: a stable argsort of the negated keys
    assert np.array_equal(O.topk_select(l, k), np.argsort(-l, axis=1, kind="stable")[:, :k])


def test_topk_ties_go_to_lower_index():
    l = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0],
                  [-1.0, 5.0, -1.0, 5.0, -1.0]], np.float32)
    idx = O.topk_select(l, 3)
    assert idx.tolist() == [[1, 2, 4], [0, 1, 2], [1, 3, 0]]
    assert np.array_equal(idx, _brute_topk(l, 3))


def test_topk_quantized_logits_many_ties():
    rng = np.random.default_rng(7)
    l = rng.integers(-2, 3, (200, 32)).astype(np.float32)
    for k in (1, 4, 8):
        assert np.array_equal(O.topk_select(l, k), _brute_topk(l, k))


def test_router_outputs_consistent():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((300, 16)).astype(np.float32)
    idx, q, counts, rmap, dense = O.router_topk(l, 4, O.SOFTMAX_PRE_RENORM)
    assert (rmap.sum(1) == 4).all()                      # k ones per row
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=16))
    assert np.array_equal(counts, rmap.sum(0))
    assert (dense[rmap == 0] == 0).all()                 # zero outside the selection
    assert np.array_equal(np.take_along_axis(dense, idx.astype(np.int64), 1), q)


@pytest.mark.parametrize("k", [1, 2, 8])
def test_softmax_pre_renorm_equals_post(k):
    # top-k then softmax over the k == softmax over all, top-k, renormalise (in R);
    # after one rounding each to fp32 the two agree within a few ulp
    rng = np.random.default_rng(k)
    l = (rng.standard_normal((500, 64)) * 3).astype(np.float32)
    idx = O.topk_select(l, k)
    a = O.topk_probs(l, idx, O.SOFTMAX_PRE_RENORM)
    b = O.topk_probs(l, idx, O.SOFTMAX_POST)
    assert np.all(np.abs(a - b) <= 4 * np.spacing(np.abs(b).astype(np.float32)))
    # rows sum to one within k * 2^-23
    assert np.all(np.abs(a.sum(1) - 1.0) <= k * 2.0 ** -23)
    # library cross-check of the post-top-k softmax
    sel = np.take_along_axis(l.astype(np.float64), idx.astype(np.int64), 1)
    assert np.allclose(b, sp.softmax(sel, axis=1), rtol=2 ** -23, atol=0)


def test_softmax_closed_form_values():
    # two experts with logits 0 and ln 3 -> weights 3/4 and 1/4 (top-2 of 3)
    l = np.array([[np.log(3.0), -50.0, 0.0]], np.float32)
    idx, q, *_ = O.router_topk(l, 2, O.SOFTMAX_POST)
    assert idx.tolist() == [[0, 2]]
    assert np.allclose(q, [[0.75, 0.25]], rtol=1e-7)
    # top-1 softmax after top-k is exactly one
    _, q1, *_ = O.router_topk(l, 1, O.SOFTMAX_POST)
    assert q1[0, 0] == 1.0


def test_sigmoid_top1_not_renormalised():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((100, 16)).astype(np.float32)
    idx, q, *_ = O.router_topk(l, 1, O.SIGMOID)
    ref = sp.expit(np.take_along_axis(l.astype(np.float64), idx.astype(np.int64), 1))
    assert np.allclose(q, ref, rtol=2 ** -23, atol=0)
    assert (q < 1.0).all()
    # sigmoid(0) = 1/2 exactly
    _, q0, *_ = O.router_topk(np.zeros((1, 4), np.float32), 1, O.SIGMOID)
    assert q0[0, 0] == 0.5


def _check_meta(idx, E):
    T, k = idx.shape
    offsets, row_of, src_of = O.dispatch_meta(idx, E)
    flat = idx.ravel()
    counts = np.bincount(flat, minlength=E)
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    # library cross-check: a stable sort of the flattened choices by expert id
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(src_of, order // k)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(row_of.ravel(), inv)
    # bijection, and every row of block e belongs to expert e
    assert np.array_equal(np.sort(row_of.ravel()), np.arange(T * k))
    blk = np.repeat(np.arange(E), counts)
    assert np.array_equal(flat[order], blk)
    return offsets, row_of, src_of


@pytest.mark.parametrize("T,E,k", [(64, 4, 2), (100, 128, 8), (8, 16, 1), (1, 8, 2), (37, 5, 5)])
def test_dispatch_meta_is_stable_counting_sort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    l = rng.standard_normal((T, E)).astype(np.float32)
    _check_meta(O.topk_select(l, k), E)


def test_dispatch_meta_empty_and_hot_experts():
    # every token to experts 0 and 1: the other blocks are empty
    T, E, k = 33, 6, 2
    idx = np.tile(np.array([[1, 0]], np.int32), (T, 1))
    offsets, row_of, src_of = _check_meta(idx, E)
    assert offsets.tolist() == [0, T, 2 * T, 2 * T, 2 * T, 2 * T, 2 * T]
    assert row_of[:, 1].tolist() == list(range(T)) and row_of[:, 0].tolist() == list(range(T, 2 * T))


def test_dispatch_worked_example():
    # 4 tokens, 3 experts, top-2, choices t0:(2,0) t1:(0,1) t2:(2,1) t3:(0,2)
    idx = np.array([[2, 0], [0, 1], [2, 1], [0, 2]], np.int32)
    offsets, row_of, src_of = O.dispatch_meta(idx, 3)
    assert offsets.tolist() == [0, 3, 5, 8]
    assert src_of.tolist() == [0, 1, 3, 1, 2, 0, 2, 3]
    assert row_of.tolist() == [[5, 0], [1, 3], [6, 4], [2, 7]]


@pytest.mark.parametrize("k", [1, 2, 8])
def test_identity_experts_unit_probs_give_k_x(k):
    # dispatch then combine with identity experts and unit weights returns k * x
    # exactly (k is a power of two, so the bf16 result is exact)
    rng = np.random.default_rng(k)
    T, E, H = 50, 16, 64
    x_bits = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    offsets, row_of, src_of = O.dispatch_meta(idx, E)
    xp = O.bf16_bits_to_f64(O.permute(x_bits, src_of))
    y = O.combine(xp, row_of, np.ones((T, k)))
    assert np.array_equal(y, k * O.bf16_bits_to_f64(x_bits))


def test_weights_applied_once():
    # weighting in combine == weighting the expert outputs before an unweighted combine
    rng = np.random.default_rng(9)
    T, E, H, k = 40, 8, 32, 2
    idx, q, *_ = O.router_topk(rng.standard_normal((T, E)).astype(np.float32), k, O.SOFTMAX_PRE_RENORM)
    offsets, row_of, src_of = O.dispatch_meta(idx, E)
    out = rng.standard_normal((T * k, H))
    qp = np.zeros(T * k)
    qp[row_of.ravel()] = q.ravel()
    a = O.combine(out, row_of, q, exact=True)
    b = O.combine(out * qp[:, None], row_of, None, exact=True)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-15)
    # applying them twice is not the same thing
    c = O.combine(out * qp[:, None], row_of, q, exact=True)
    assert not np.allclose(a, c)


def test_padded_dispatch_receive_buffer_example():
    # the pages' example: counts of 129 and 127 need 384 rows at alignment 128
    idx = np.array([[0]] * 129 + [[1]] * 127, dtype=np.int32)
    offsets, pad, row_of, src_of = O.dispatch_meta_padded(idx, 2, 128)
    assert offsets.tolist() == [0, 256, 384]
    assert pad.tolist() == [0, 127]
    assert row_of[128, 0] == 128 and row_of[129, 0] == 256 and row_of[-1, 0] == 382
    assert (src_of[129:256] == -1).all() and src_of[383] == -1 and src_of[256] == 129


def test_padded_dispatch_shifts_the_plain_layout():
    rng = np.random.default_rng(9)
    T, E, k = 97, 10, 3
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    off_u, row_u, src_u = O.dispatch_meta(idx, E)
    for align in (1, 8, 64):
        offsets, pad, row_of, src_of = O.dispatch_meta_padded(idx, E, align)
        assert (offsets % align == 0).all() and (np.diff(offsets) >= np.diff(off_u)).all()
        assert (np.diff(offsets) - np.diff(off_u) < align).all()
        assert np.array_equal(row_of - pad[idx], row_u)          # same order, shifted blocks
        assert np.array_equal(src_of[src_of >= 0], src_u)        # token rows in plain order
        assert (src_of >= 0).sum() == T * k
    offsets1, pad1, row1, src1 = O.dispatch_meta_padded(idx, E, 1)
    assert np.array_equal(offsets1, off_u) and not pad1.any() and np.array_equal(row1, row_u)
