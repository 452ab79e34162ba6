"""GPU parity (through the C ABI) of the router on masked (-inf) and NaN logits and of the
softmax before the top-k without renormalisation (Transformer Engine guide "Mixture of
Experts", Router: use_pre_softmax; Token combine: pre-softmax top-1 weights are not one):
the fast one-token-per-16-lanes kernel (k <= 16), the one-wave-per-token kernel (k > 16)
and the kernel with options, the router backward with the full-softmax gradient, and the
dispatch backward with a dense d_logits.

Without an expert bias or groups the selection keys are the logits themselves, so the ids
must match the oracle bit for bit, ties and -inf included; the weights are fp32 results
of exp and a sum and must agree within 1e-6 relative (NaN where the oracle has NaN: a row
with no finite logit)."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
from gpu_helpers import check_bf16, check_close, combine_slack, dev, dev_bf16, host_vals

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _masked_logits(rng, T, E, k):
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(0, T, 3):   # every third row: fewer than k finite logits left
        nmask = int(rng.integers(E - k + 1, E + 1))
        cols = rng.choice(E, size=nmask, replace=False)
        lg[t, cols[: nmask // 2]] = -np.inf
        lg[t, cols[nmask // 2:]] = np.nan
    lg[1, :] = -np.inf
    lg[2, :] = np.nan
    lg[4, : E // 2] = -np.inf   # ties at -inf among the last k
    return lg


def _run_router(lg, k, score, opts=None):
    T, E = lg.shape
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    q = torch.full((T, k), 7.0, device="cuda")
    counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    rmap = torch.full((T, E), 9, dtype=torch.uint8, device="cuda")
    dense = torch.full((T, E), 7.0, device="cuda")
    if opts is None:
        M.moe_router_topk(dev(lg), k, score, idx, q, counts, rmap, dense)
    else:
        M.moe_router_topk_ex(dev(lg), k, score, opts, idx, q, counts, rmap, dense)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), host_vals(q), counts.cpu().numpy(), rmap.cpu().numpy(),
            host_vals(dense))


def _compare(lg, k, score, got, name, num_groups=0, group_topk=0, scaling=1.0):
    idx, q, counts, rmap, dense = got
    E = lg.shape[1]
    ridx, rq, rcounts, rrmap, rdense = O.router_topk(lg, k, score, num_groups=num_groups,
                                                     group_topk=group_topk,
                                                     scaling_factor=scaling)
    assert ((idx >= 0) & (idx < E)).all(), f"{name}: id out of range"
    assert np.array_equal(idx, ridx), f"{name}: ids differ in rows {np.nonzero((idx != ridx).any(1))[0][:8]}"
    assert np.array_equal(counts, rcounts) and np.array_equal(rmap, rrmap), name
    ok = np.isclose(q, rq, rtol=1e-6, atol=0, equal_nan=True)
    assert ok.all(), (name, q[~ok][:4], rq[~ok][:4])
    okd = np.isclose(dense, rdense, rtol=1e-6, atol=0, equal_nan=True)
    assert okd.all(), name
    _say(f"{name}: ok, NaN weights in {int(np.isnan(q).any(1).sum())} rows")


@pytest.mark.parametrize("T,E,k", [(200, 16, 4), (130, 128, 8), (77, 40, 20), (65, 256, 32),
                                   (33, 7, 7)])
@pytest.mark.parametrize("score", [O.SOFTMAX_PRE_RENORM, O.SOFTMAX_POST, O.SOFTMAX_PRE,
                                   O.SIGMOID, O.SQRTSOFTPLUS])
def test_router_masked_and_nan_logits(T, E, k, score):
    _say("router masked/NaN", T, E, k, score)
    rng = np.random.default_rng(T * 7 + E + k + score)
    lg = _masked_logits(rng, T, E, k)
    _compare(lg, k, score, _run_router(lg, k, score), f"plain {T}x{E} k={k} s={score}")
    # the options kernel: a scaling factor (same keys), and grouped routing after the
    # top-k (group values = logits, summed best first in fp32 on both sides)
    opts = M.router_opts(scaling_factor=2.0)
    _compare(lg, k, score, _run_router(lg, k, score, opts), f"scaled {T}x{E} k={k} s={score}",
             scaling=2.0)
    if score == O.SOFTMAX_POST and E % 4 == 0 and k <= 2 * (E // 4):
        opts = M.router_opts(num_groups=4, group_topk=2)
        _compare(lg, k, score, _run_router(lg, k, score, opts), f"grouped {T}x{E} k={k}",
                 num_groups=4, group_topk=2)


@pytest.mark.parametrize("T,E,k", [(300, 16, 4), (129, 128, 8), (70, 64, 24), (40, 8, 1)])
def test_router_softmax_pre(T, E, k):
    _say("router softmax before the top-k, no renormalisation", T, E, k)
    rng = np.random.default_rng(3 * T + E)
    lg = (rng.standard_normal((T, E)) * 2.0).astype(np.float32)
    got = _run_router(lg, k, O.SOFTMAX_PRE)
    _compare(lg, k, O.SOFTMAX_PRE, got, f"pre {T}x{E} k={k}")
    assert (got[1].sum(axis=1) < 1.0 + 1e-6).all()
    if k == 1:
        assert (got[1] < 1.0).all()    # non-unit top-1 weights
    opts = M.router_opts(scaling_factor=0.5)
    _compare(lg, k, O.SOFTMAX_PRE, _run_router(lg, k, O.SOFTMAX_PRE, opts), "pre scaled",
             scaling=0.5)


def test_router_softmax_pre_grouped():
    # groups of the softmax probabilities; group scores are fp32 sums on both sides, so
    # only tokens decided by a clear margin are compared
    from test_gpu_router_opts import _firm
    rng = np.random.default_rng(11)
    T, E, k, G, gt = 400, 64, 8, 8, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, q, *_ = _run_router(lg, k, O.SOFTMAX_PRE, M.router_opts(num_groups=G, group_topk=gt))
    ridx, rq, *_ = O.router_topk(lg, k, O.SOFTMAX_PRE, num_groups=G, group_topk=gt)
    firm = _firm(lg, k, O.SOFTMAX_PRE, None, G, gt)
    assert firm.mean() > 0.9
    assert np.array_equal(idx[firm], ridx[firm])
    assert np.allclose(q[firm], rq[firm], rtol=1e-6, atol=0)


@pytest.mark.parametrize("T,H,E,k,scaling", [(300, 256, 16, 4, 1.0), (65, 512, 128, 8, 2.5),
                                             (40, 128, 8, 1, 1.0)])
def test_combine_backward_router_softmax_pre(T, H, E, k, scaling):
    _say("combine backward router, softmax before the top-k", T, H, E, k)
    rng = np.random.default_rng(5 * T + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, q, _, _, _ = O.router_topk(lg, k, O.SOFTMAX_PRE, scaling_factor=scaling)
    _, row_of, _ = O.dispatch_meta(idx, E)
    N = T * k
    bf = lambda shape: O.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    dy, out = bf((T, H)), bf((N, H))
    d_out = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
    d_prob = torch.full((T, k), float("nan"), device="cuda")
    d_logits = torch.full((T, E), float("nan"), device="cuda")
    M.moe_combine_backward_router(dev_bf16(dy), dev_bf16(out), dev(row_of), dev(idx),
                                  dev(q.astype(np.float32)), O.SOFTMAX_PRE, d_out, d_logits, d_prob,
                                  scaling_factor=scaling, logits=dev(lg))
    torch.cuda.synchronize()
    dyv, outv = O.as_values(dy), O.as_values(out)
    ref_dq = O.prob_grad(dy, outv, row_of)
    absdot = np.stack([(np.abs(dyv) * np.abs(outv[row_of[:, j]])).sum(axis=1) for j in range(k)], 1)
    u = 2.0 ** -24
    b_dq = H * u * absdot + u * np.abs(ref_dq)
    check_close(host_vals(d_prob), ref_dq, b_dq, "d_prob")
    ref_dl = O.router_backward(lg, idx, ref_dq, O.SOFTMAX_PRE, scaling_factor=scaling)
    # with s = q / c the kept probabilities and S = sum_j s_j d_prob_j: kept experts
    # c s_j (d_prob_j - S), the others -c p_e S; the bounds carry the d_prob error and a
    # few fp32 roundings of exp, the softmax sum (E terms) and the products
    s = q / scaling
    S_b = (s * b_dq).sum(axis=1, keepdims=True)
    S_abs = (s * np.abs(ref_dq)).sum(axis=1, keepdims=True)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    bound = scaling * p * (S_b + (E + k + 16) * u * S_abs)
    rows = np.arange(T)[:, None]
    bound[rows, idx] = scaling * s * (b_dq + S_b) + (k + 16) * u * scaling * s * (np.abs(ref_dq) + S_abs)
    got = host_vals(d_logits)
    kept = np.zeros((T, E), bool)
    kept[rows, idx] = True
    assert (got[~kept] != 0).mean() > 0.99   # the experts not kept get a gradient
    check_close(got, ref_dl, bound, "d_logits (pre)", floor=1e-12 * np.abs(ref_dl).max())


@pytest.mark.parametrize("T,H,E,k", [(200, 256, 16, 4), (33, 512, 128, 8)])
def test_dispatch_backward_router_dense(T, H, E, k):
    # a d_logits with every expert nonzero (softmax before the top-k): the router's dx term
    # runs over all of them
    _say("dispatch backward router, dense d_logits", T, H, E, k)
    rng = np.random.default_rng(T + E)
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    _, row_of, _ = O.dispatch_meta(idx, E)
    bf = lambda shape, sd=1.0: O.f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    dxp, w = bf((T * k, H)), bf((E, H), 0.02)
    dl = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    dl[0, :] = 0.0            # a token with no router gradient at all
    dl[1, ::2] = 0.0
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    M.moe_dispatch_backward_router(dev_bf16(dxp), dev(row_of), dev(idx), dev(dl), dev_bf16(w), dx)
    torch.cuda.synchronize()
    dxpv = O.as_values(dxp)
    ref = O.combine(dxpv, row_of, None, dl.astype(np.float64) @ O.as_values(w))
    check_bf16(host_vals(dx), ref, "dx (dense router term)", slack=combine_slack(dxpv, row_of))
