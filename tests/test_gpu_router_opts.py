"""GPU parity of the router options (sqrtsoftplus, expert bias, grouped routing, scaling,
bit-packed routing map), the expert-bias update, and the router backward with the new
score function and scaling, against the oracle through the C ABI.

The selection keys and group scores are fp32 values computed from exp/log on both sides
(the oracle rounds its float64 values once; the device's exp, log1p and sqrt are within
a few ulps), so a token whose k-th and (k+1)-th key, or whose group_topk-th and next
group score, are closer than the tolerance below may choose differently: such tokens are
left out of the comparisons, and at least 90% of the tokens must be decided by a clear
margin. Everything else is compared bit-exactly (ids, counts, maps) or within 1e-6
relative (weights).
"""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
import workloads as W
from gpu_helpers import (GpuMoE, check_bf16, check_close, combine_slack, dev, dev_bf16,
                         fp32_sum_bound, host_vals, topk_gap)

pytestmark = pytest.mark.gpu

KEY_ULPS = 16  # device exp / log1p / sqrt and the bias add, in fp32 ulps of the value


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _firm(lg, k, score, bias, G, gt):
    """Tokens whose choice (groups, then experts) is decided by more than the tolerance."""
    key, gval = O.selection_keys(lg, score, bias)
    T, E = key.shape
    tol_k = KEY_ULPS * 2.0 ** -24 * (np.abs(key).max(axis=1) + 1.0)
    allowed = np.ones((T, E), bool)
    firm = np.ones(T, bool)
    if G and G > 1:
        gs, m = E // G, k // gt
        gscore = np.zeros((T, G))
        for g in range(G):
            kg, vg = key[:, g * gs:(g + 1) * gs], gval[:, g * gs:(g + 1) * gs]
            best = O.topk_select(kg, m)
            gscore[:, g] = np.take_along_axis(vg, best.astype(np.int64), 1).sum(axis=1)
            # the m-th and (m+1)-th key inside a group decide which values are summed
            if m < gs:
                firm &= topk_gap(kg, m) > 2 * tol_k
        tol_g = (m + 2) * KEY_ULPS * 2.0 ** -24 * (np.abs(gval).max(axis=1) * m + 1.0)
        firm &= topk_gap(gscore, gt) > 2 * tol_g
        kept = O.topk_select(gscore, gt)
        allowed[:] = False
        for j in range(gt):
            for g in range(G):
                allowed[kept[:, j] == g, g * gs:(g + 1) * gs] = True
    masked = np.where(allowed, key, -np.inf)
    firm &= topk_gap(masked, k) > 2 * tol_k
    return firm


CASES = [
    # name, T, E, k, score, bias, groups, group_topk, scaling, bitmap
    ("pre_grouped", 300, 64, 6, O.SOFTMAX_PRE_RENORM, False, 8, 3, 2.5, False),
    ("post_grouped_bitmap", 257, 16, 4, O.SOFTMAX_POST, False, 4, 2, 1.0, True),
    ("sigmoid_bias", 200, 32, 2, O.SIGMOID, True, 0, 0, 1.0, False),
    ("sqrt_bias_grouped", 333, 256, 8, O.SQRTSOFTPLUS, True, 8, 4, 2.5, True),
    ("sqrt_plain", 129, 128, 8, O.SQRTSOFTPLUS, False, 0, 0, 1.0, False),
    ("sqrt_top1_scaled", 64, 40, 1, O.SQRTSOFTPLUS, False, 0, 0, 0.5, True),
    ("sigmoid_grouped", 96, 60, 4, O.SIGMOID, False, 5, 2, 1.0, False),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_router_topk_ex(ci):
    name, T, E, k, score, use_bias, G, gt, scale, bitmap = CASES[ci]
    _say("router options", name)
    rng = np.random.default_rng(100 + ci)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32) if use_bias else None
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    prob = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    cols = (E + 7) // 8 if bitmap else E
    rmap = torch.full((T, cols), 0xAB, dtype=torch.uint8, device="cuda")
    dense = torch.full((T, E), float("nan"), device="cuda")
    bias_d = dev(bias) if use_bias else None
    opts = M.router_opts(bias_d, G, gt, scale, bitmap)
    M.moe_router_topk_ex(dev(lg), k, score, opts, idx, prob, counts, rmap, dense)
    torch.cuda.synchronize()
    gi, gq, gc = idx.cpu().numpy(), prob.cpu().numpy(), counts.cpu().numpy()
    rid, rq, rc, rmap_ref, _ = O.router_topk(lg, k, score, expert_bias=bias, num_groups=G,
                                             group_topk=gt, scaling_factor=scale)
    firm = _firm(lg, k, score, bias, G, gt)
    _say(f"{name}: firm {int(firm.sum())}/{T}")
    assert firm.mean() >= 0.9
    assert np.array_equal(gi[firm], rid[firm])
    assert np.allclose(gq[firm], rq[firm], rtol=1e-6, atol=0)
    # the device's own choice is consistent everywhere
    assert np.array_equal(gc, np.bincount(gi.reshape(-1), minlength=E))
    if firm.all():
        assert np.array_equal(gc, rc)
    own = np.zeros((T, E), np.uint8)
    own[np.arange(T)[:, None], gi] = 1
    got_map = rmap.cpu().numpy()
    assert np.array_equal(got_map, O.pack_routing_map(own) if bitmap else own)
    gd = dense.cpu().numpy()
    want = np.zeros((T, E), np.float32)
    want[np.arange(T)[:, None], gi] = gq
    assert np.array_equal(gd, want)
    if G and G > 1:  # every choice inside group_topk groups
        assert all(len({int(e) // (E // G) for e in row}) <= gt for row in gi)


def test_router_options_rejected_on_the_host():
    lg = torch.zeros((4, 16), device="cuda")
    idx = torch.empty((4, 3), dtype=torch.int32, device="cuda")
    prob = torch.empty((4, 3), dtype=torch.float32, device="cuda")
    counts = torch.empty((16,), dtype=torch.int32, device="cuda")
    bias = torch.zeros(16, device="cuda")
    for k, opts, status in ((2, M.router_opts(bias), M.MOE_ERR_UNSUPPORTED),        # bias + softmax
                            (2, M.router_opts(None, 3, 1), M.MOE_ERR_UNSUPPORTED),  # 16 % 3
                            (2, M.router_opts(None, 4, 5), M.MOE_ERR_INVALID_ARG),  # 5 > 4 groups
                            (3, M.router_opts(None, 8, 1), M.MOE_ERR_INVALID_ARG)):  # 3 > 1 x 2
        with pytest.raises(M.MoeError) as e:
            M.moe_router_topk_ex(lg, k, O.SOFTMAX_POST, opts, idx[:, :k].contiguous(),
                                 prob[:, :k].contiguous(), counts)
        assert e.value.status == status


@pytest.mark.parametrize("counts,coeff", [([10, 10, 10, 10], 1e-3), ([30, 10, 10, 10], 0.25),
                                          (list(range(128)), 1e-3),
                                          ([5_000_001, 3, 0, 77, 123456, 9], 0.01)])
def test_expert_bias_update(counts, coeff):
    E = len(counts)
    rng = np.random.default_rng(E)
    b0 = (rng.standard_normal(E) * 0.1).astype(np.float32)
    bias = dev(b0)
    M.moe_expert_bias_update(bias, dev(np.array(counts, np.int32)), np.float32(coeff))
    torch.cuda.synchronize()
    want = O.expert_bias_update(b0, counts, float(np.float32(coeff)))
    assert np.array_equal(bias.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("score,scale", [(O.SQRTSOFTPLUS, 2.5), (O.SIGMOID, 0.5),
                                         (O.SOFTMAX_PRE_RENORM, 2.0), (O.SQRTSOFTPLUS, 1.0)])
def test_combine_backward_router_scaled(score, scale):
    T, H, E, k = 150, 256, 32, 4
    _say("combine backward router", score, scale)
    rng = np.random.default_rng(13 + score)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, q, _, _, _ = O.router_topk(lg, k, score, scaling_factor=scale)
    _, row_of, _ = O.dispatch_meta(idx, E)
    N = T * k
    dy = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out = W.to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    d_out = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
    d_prob = torch.empty((T, k), device="cuda")
    d_logits = torch.full((T, E), float("nan"), device="cuda")
    M.moe_combine_backward_router(dev_bf16(dy), dev_bf16(out), dev(row_of), dev(idx),
                                  dev(q.astype(np.float32)), score, d_out, d_logits, d_prob,
                                  scaling_factor=scale)
    torch.cuda.synchronize()
    dyv, outv = O.as_values(dy), O.as_values(out)
    ref_dq = O.prob_grad(dy, outv, row_of)
    absdot = np.stack([(np.abs(dyv) * np.abs(outv[row_of[:, j]])).sum(axis=1) for j in range(k)], 1)
    b_dq = H * 2.0 ** -24 * absdot + 2.0 ** -24 * np.abs(ref_dq)
    check_close(host_vals(d_prob), ref_dq, b_dq, "d_prob")
    ref_dl = O.router_backward(lg, idx, ref_dq, score, scaling_factor=scale)
    u = 2.0 ** -24
    s = q / scale
    if score == O.SIGMOID:
        b_sel = scale * (s * (1 - s) * b_dq + 8 * u * s * np.abs(ref_dq))
    elif score == O.SQRTSOFTPLUS:
        g = -np.expm1(-s * s) / (2 * s)
        b_sel = scale * g * (b_dq + 24 * u * np.abs(ref_dq))
    else:
        s_b = (s * b_dq).sum(axis=1, keepdims=True)
        s_abs = (s * np.abs(ref_dq)).sum(axis=1, keepdims=True)
        b_sel = scale * (s * (b_dq + s_b) + (k + 8) * u * s * (np.abs(ref_dq) + s_abs))
    bound = np.zeros((T, E))
    bound[np.arange(T)[:, None], idx] = b_sel
    check_close(host_vals(d_logits), ref_dl, bound, "d_logits", floor=1e-12 * np.abs(ref_dl).max())


def test_layer_with_router_options():
    """Forward + backward of the layer with sqrtsoftplus, an expert bias, grouped routing
    and scaling (logits given, so both sides start from the same fp32 logits)."""
    w = W.custom("opts", T=300, H=256, E=64, k=6, I=128, score=O.SQRTSOFTPLUS, training=True)
    G, gt, scale = 8, 3, 2.5
    _say("layer with router options")
    d = W.make_inputs(w)
    bias = (np.random.default_rng(3).standard_normal(w.E) * 0.3).astype(np.float32)
    g = GpuMoE(w, d)
    g.prob.num_groups, g.prob.group_topk, g.prob.scaling_factor = G, gt, scale
    bias_d = dev(bias)
    g.tens.expert_bias = bias_d.data_ptr()
    y = host_vals(g.forward())
    firm = _firm(d["logits"], w.k, w.score, bias, G, gt)
    assert firm.all(), np.nonzero(~firm)[0]
    idx, q, counts, _, _ = O.router_topk(d["logits"], w.k, w.score, expert_bias=bias,
                                         num_groups=G, group_topk=gt, scaling_factor=scale)
    offsets, row_of, src_of = O.dispatch_meta(idx, w.E)
    ints = g.ints()
    assert np.array_equal(ints["topk_idx"], idx) and np.array_equal(ints["offsets"], offsets)
    assert np.array_equal(ints["row_of"], row_of) and np.array_equal(ints["src_of"], src_of)
    assert np.allclose(ints["topk_prob"], q, rtol=1e-6, atol=0)
    # the oracle layer on the options' choice: dispatch, MLP and combine as usual
    xp = O.as_values(d["x"])[src_of.astype(np.int64)]
    mlp = O.expert_mlp(xp, d["w_gu"], d["w_down"], offsets, w.I)
    yr = O.combine(mlp["out"], row_of, q)
    check_bf16(y, yr, "opts y", slack=combine_slack(mlp["out"], row_of, q))
    g.backward(d["dy"])
    fwd = dict(topk_idx=idx, topk_prob=q, offsets=offsets, row_of=row_of, src_of=src_of,
               xp=xp, **mlp)
    rb = O.moe_backward(fwd, d["dy"], d["w_gu"], d["w_down"], w.I)
    check_bf16(host_vals(g.dx), rb["dx"], "opts dx", slack=combine_slack(rb["dxp"], row_of))
    check_bf16(host_vals(g.dw_gu), rb["dw_gu"], "opts dw_gu")
    check_bf16(host_vals(g.dw_down), rb["dw_down"], "opts dw_down")


def test_layer_router_projection_sqrtsoftplus_scaled():
    """The layer owning its router projection with sqrtsoftplus weights scaled by 2.5:
    d_logits and dW_r through the new score function."""
    w = W.custom("r_sqrt", T=200, H=256, E=32, k=4, I=128, score=O.SQRTSOFTPLUS, training=True)
    scale = 2.5
    _say("layer router sqrtsoftplus scaled")
    d = W.make_inputs(w)
    g = GpuMoE(w, d, router=True)
    g.prob.scaling_factor = scale
    g.forward()
    ref_logits = O.gate_logits(d["x"], d["w_router"])
    xa, wa = np.abs(O.as_values(d["x"])), np.abs(O.as_values(d["w_router"]))
    bound = fp32_sum_bound(xa, wa.T, w.H) + 2.0 ** -24 * np.abs(ref_logits)
    assert (topk_gap(ref_logits, w.k) > 2 * bound.max(axis=1)).all()
    idx, q, _, _, _ = O.router_topk(ref_logits, w.k, w.score, scaling_factor=scale)
    assert np.array_equal(g.ints()["topk_idx"], idx)
    offsets, row_of, src_of = O.dispatch_meta(idx, w.E)
    xp = O.as_values(d["x"])[src_of.astype(np.int64)]
    mlp = O.expert_mlp(xp, d["w_gu"], d["w_down"], offsets, w.I)
    fwd = dict(topk_idx=idx, topk_prob=q, offsets=offsets, row_of=row_of, src_of=src_of, xp=xp,
               x=O.as_values(d["x"]), logits=ref_logits, score=w.score, **mlp)
    g.backward(d["dy"])
    # the oracle's backward with the scaled weights: the router term sees c * d_prob
    dq = O.prob_grad(d["dy"], mlp["out"], row_of)
    dl = O.router_backward(ref_logits, idx, dq, w.score, scaling_factor=scale)
    dwr = O.to_f32(dl.T @ O.as_values(d["x"]))
    for key, got, r in (("d_logits", host_vals(g.view("d_logits", (w.T, w.E), torch.float32)), dl),
                        ("dw_router", host_vals(g.dw_router), dwr)):
        rel = np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30)
        _say(f"sqrtsoftplus scaled {key}: rel_l2={rel:.3e}")
        assert np.isfinite(got).all() and rel <= 1e-2, (key, rel)
    rb = O.moe_backward(fwd, d["dy"], d["w_gu"], d["w_down"], w.I)
    dx_ref = O.combine(rb["dxp"], row_of, None, dl @ O.as_values(d["w_router"]))
    check_bf16(host_vals(g.dx), dx_ref, "sqrtsoftplus scaled dx", slack=combine_slack(rb["dxp"], row_of))
