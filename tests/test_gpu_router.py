"""GPU parity of the router projection and the router backward (through the C ABI)
against the oracle: stage calls on seeded inputs spanning several blocks with ragged
tails, then the whole layer with its own router projection, forward and backward.

Tolerances of the fp32 results follow from the arithmetic: a sum of n exact products
in fp32 is within n * 2^-24 * sum|terms| of the exact sum (the recursive-summation
bound); the router weight gradient also carries the two-half bf16 split of each
d_logits value, within 2^-18 of the value. Logits decide the top-k choice: a token
whose k-th and (k+1)-th oracle logits are further apart than twice the logits bound
must select the same experts on both sides; closer ones may differ and are left out of
the comparisons that depend on the choice, and the dispatch layout is then checked
for consistency with the device's own choice.
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


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf(rng, shape, std=1.0):
    return W.to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


@pytest.mark.parametrize("T,H,E", [(333, 256, 8), (64, 128, 4), (257, 512, 200), (1, 64, 3),
                                   (97, 2048, 128)])
def test_router_logits(T, H, E):
    _say("router logits", T, H, E)
    rng = np.random.default_rng(T + H + E)
    x, w = _bf(rng, (T, H)), _bf(rng, (E, H), 0.02)
    logits = torch.full((T, E), float("nan"), device="cuda")
    M.moe_router_logits(dev_bf16(x), dev_bf16(w), logits)
    torch.cuda.synchronize()
    ref = O.gate_logits(x, w)
    bound = fp32_sum_bound(np.abs(O.as_values(x)), np.abs(O.as_values(w)).T, H) + 2.0 ** -24 * np.abs(ref)
    check_close(host_vals(logits), ref, bound, f"logits {T}x{H}x{E}")


def _routing(rng, T, E, k, score):
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, q, _, _, _ = O.router_topk(logits, k, score)
    _, row_of, _ = O.dispatch_meta(idx, E)
    return logits, idx, q, row_of


@pytest.mark.parametrize("T,H,E,k,score", [(300, 256, 16, 4, O.SOFTMAX_PRE_RENORM),
                                           (77, 512, 8, 2, O.SOFTMAX_POST),
                                           (65, 256, 16, 1, O.SIGMOID),
                                           (40, 128, 64, 12, O.SOFTMAX_PRE_RENORM),
                                           (33, 128, 32, 3, O.SIGMOID)])
def test_combine_backward_router(T, H, E, k, score):
    _say("combine backward router", T, H, E, k, score)
    rng = np.random.default_rng(7 * T + k)
    logits, idx, q, row_of = _routing(rng, T, E, k, score)
    N = T * k
    dy, out = _bf(rng, (T, H)), _bf(rng, (N, H))
    d_out = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
    d_prob = torch.full((T, k), float("nan"), device="cuda")
    d_logits = torch.full((T, E), float("nan"), device="cuda")
    M.moe_combine_backward_router(dev_bf16(dy), dev_bf16(out), dev(row_of), dev(idx),
                                  dev(q.astype(np.float32)), score, d_out, d_logits, d_prob)
    torch.cuda.synchronize()
    # d_out = bf16(q * dy): one fp32 product, then bf16 -- bit-exact
    dyv = O.as_values(dy)
    ref_out = np.zeros((N, H))
    for j in range(k):
        ref_out[row_of[:, j]] = O.to_bf16(dyv * q[:, j:j + 1])
    assert np.array_equal(host_vals(d_out), ref_out)
    # d_prob: fp32 sums of H exact products
    ref_dq = O.prob_grad(dy, O.as_values(out), row_of)
    outv = O.as_values(out)
    absdot = np.stack([(np.abs(dyv) * np.abs(outv[row_of[:, j]])).sum(axis=1) for j in range(k)], 1)
    b_dq = H * 2.0 ** -24 * absdot + 2.0 ** -24 * np.abs(ref_dq)
    check_close(host_vals(d_prob), ref_dq, b_dq, "d_prob")
    # d_logits: the score backward on the kept experts, 0 elsewhere. Its error follows
    # from the d_prob error B and a few fp32 roundings of the products
    ref_dl = O.router_backward(logits, idx, ref_dq, score)
    rows = np.arange(T)[:, None]
    if score == O.SIGMOID:
        b_sel = q * (1 - q) * b_dq + 8 * 2.0 ** -24 * q * np.abs(ref_dq)
    else:
        s_b = (q * b_dq).sum(axis=1, keepdims=True)
        s_abs = (q * np.abs(ref_dq)).sum(axis=1, keepdims=True)
        b_sel = q * (b_dq + s_b) + (k + 8) * 2.0 ** -24 * q * (np.abs(ref_dq) + s_abs)
    bound = np.zeros((T, E))
    bound[rows, idx] = b_sel
    got = host_vals(d_logits)
    # experts not kept: exactly 0 on the device (the oracle's full-softmax chain rule
    # leaves float64 residues there, far below the floor)
    mask = np.ones((T, E), bool)
    mask[rows, idx] = False
    assert not got[mask].any()
    check_close(got, ref_dl, bound, "d_logits", floor=1e-12 * np.abs(ref_dl).max())


@pytest.mark.parametrize("T,H,E,k", [(1000, 256, 8, 2), (64, 128, 4, 2), (4096, 512, 128, 8),
                                     (300, 192, 24, 3), (0, 128, 8, 2)])
def test_router_weight_grad(T, H, E, k):
    _say("router weight grad", T, H, E, k)
    rng = np.random.default_rng(11 + T + E)
    x = _bf(rng, (T, H))
    # a d_logits of the layer's shape: k nonzero fp32 values per token
    dl = np.zeros((T, E), np.float32)
    if T:
        idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
        dl[np.arange(T)[:, None], idx] = rng.standard_normal((T, k)).astype(np.float32) * 0.3
    dw = torch.full((E, H), float("nan"), device="cuda")
    ws = torch.empty(M.moe_router_weight_grad_workspace_bytes(T, H, E), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xFF)
    xd = dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    M.moe_router_weight_grad(xd, dev(dl), dw, ws)
    torch.cuda.synchronize()
    got = host_vals(dw)
    if T == 0:
        assert not got.any()
        return
    xv = O.as_values(x)
    ref = O.to_f32(dl.astype(np.float64).T @ xv)
    absdot = np.abs(dl.astype(np.float64)).T @ np.abs(xv)
    bound = (2.0 ** -17 + 2 * T * 2.0 ** -24) * absdot + 2.0 ** -24 * np.abs(ref)
    check_close(got, ref, bound, f"dw_router {T}x{H}x{E}")


@pytest.mark.parametrize("T,H,E,k", [(300, 256, 16, 4), (77, 512, 8, 2), (5, 128, 64, 12)])
def test_dispatch_backward_router(T, H, E, k):
    _say("dispatch backward router", T, H, E, k)
    rng = np.random.default_rng(3 * T + k)
    _, idx, _, row_of = _routing(rng, T, E, k, O.SOFTMAX_PRE_RENORM)
    dxp, w = _bf(rng, (T * k, H)), _bf(rng, (E, H), 0.02)
    dl = np.zeros((T, E), np.float32)
    dl[np.arange(T)[:, None], idx] = rng.standard_normal((T, k)).astype(np.float32)
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    M.moe_dispatch_backward_router(dev_bf16(dxp), dev(row_of), dev(idx), dev(dl), dev_bf16(w), dx)
    torch.cuda.synchronize()
    dxpv = O.as_values(dxp)
    ref = O.combine(dxpv, row_of, None, dl.astype(np.float64) @ O.as_values(w))
    check_bf16(host_vals(dx), ref, "dx (router)", slack=combine_slack(dxpv, row_of))


# ---- whole layer with the router projection -----------------------------------------------

LAYER = {
    "qwen_like": W.custom("r_qwen", T=257, H=256, E=32, k=8, I=192, training=True),
    "post": W.custom("r_post", T=300, H=384, E=8, k=2, I=256, score=O.SOFTMAX_POST, training=True),
    "sigmoid": W.custom("r_sig", T=96, H=256, E=16, k=2, I=128, score=O.SIGMOID, training=True),
    "t1": W.custom("r_t1", T=1, H=128, E=8, k=2, I=128, training=True),
    "pre": W.custom("r_pre", T=200, H=256, E=16, k=4, I=128, score=O.SOFTMAX_PRE, training=True),
}


def _router_choice(w, d, g):
    """Oracle logits and the device's top-k choice. Tokens whose k-th and (k+1)-th oracle
    logits are more than twice the logits bound apart must choose the same experts on
    both sides; a closer (near-tie) token may choose differently, but only among experts
    whose oracle logit is within that distance of its k-th largest. Returns the oracle
    logits, the tokens whose choice matches, and the experts no differing token chose
    on either side."""
    ref_logits = O.gate_logits(d["x"], d["w_router"])
    got_logits = host_vals(g.view("logits", (w.T, w.E), torch.float32))
    xa, wa = np.abs(O.as_values(d["x"])), np.abs(O.as_values(d["w_router"]))
    bound = fp32_sum_bound(xa, wa.T, w.H) + 2.0 ** -24 * np.abs(ref_logits)
    check_close(got_logits, ref_logits, bound, f"{w.name} logits")
    tol = 2 * bound.max(axis=1)
    firm = topk_gap(ref_logits, w.k) > tol
    idx_ref = O.topk_select(ref_logits, w.k)
    idx_got = g.ints()["topk_idx"]
    same = (idx_got == idx_ref).all(axis=1)
    assert same[firm].all(), np.nonzero(firm & ~same)[0]
    kth = -np.sort(-ref_logits, axis=1)[:, w.k - 1]
    chosen = np.take_along_axis(ref_logits, idx_got.astype(np.int64), axis=1)
    assert (chosen >= (kth - tol)[:, None]).all()
    clean = np.ones(w.E, bool)
    clean[idx_got[~same].reshape(-1)] = False
    clean[idx_ref[~same].reshape(-1)] = False
    _say(f"{w.name}: near-tie tokens {int((~firm).sum())}, differing choices {int((~same).sum())}")
    return ref_logits, same, clean


def _valid_dispatch(ints, E):
    """Dispatch metadata consistent with the device's own choice (used when a near-tie
    token chose differently, so the oracle's layout is not the device's)."""
    idx, row_of, src_of, offsets = ints["topk_idx"], ints["row_of"], ints["src_of"], ints["offsets"]
    T, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert np.array_equal(ints["counts"], counts)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(np.sort(row_of.reshape(-1)), np.arange(T * k))
    tok = np.repeat(np.arange(T), k)
    assert np.array_equal(src_of[row_of.reshape(-1)], tok)
    for e in range(E):  # inside a block rows follow ascending token index
        blk = src_of[offsets[e]:offsets[e + 1]]
        assert (np.diff(blk) > 0).all() and (idx[blk] == e).any(axis=1).all()


@pytest.mark.parametrize("name", list(LAYER))
def test_layer_with_router(name):
    w = LAYER[name]
    _say("layer with router", name)
    d = W.make_inputs(w)
    g = GpuMoE(w, d, router=True)
    y = host_vals(g.forward())
    ref_logits, same, clean = _router_choice(w, d, g)
    ref = O.moe_forward(d["x"], ref_logits, d["w_gu"], d["w_down"], w.k, w.score, w.I)
    ints = g.ints()
    if same.all():
        for key in ("topk_idx", "counts", "offsets", "row_of", "src_of"):
            assert np.array_equal(ints[key], ref[key]), key
    else:
        _valid_dispatch(ints, w.E)
    S = np.nonzero(same)[0]
    slack = combine_slack(ref["out"], ref["row_of"], ref["topk_prob"])
    check_bf16(y[S], ref["y"][S], f"{name} y", slack=slack[S])
    g.backward(d["dy"])
    rb = O.moe_backward(ref, d["dy"], d["w_gu"], d["w_down"], w.I, w_router_bits=d["w_router"])
    check_bf16(host_vals(g.dx)[S], rb["dx"][S], f"{name} dx",
               slack=combine_slack(rb["dxp"], ref["row_of"])[S])
    C = np.nonzero(clean)[0]
    check_bf16(host_vals(g.dw_gu)[C], rb["dw_gu"][C], f"{name} dw_gu")
    check_bf16(host_vals(g.dw_down)[C], rb["dw_down"][C], f"{name} dw_down")
    # d_logits and dW_r: fp32 results computed from the bf16 expert outputs, whose
    # elements may each sit one bf16 rounding away from the oracle's, so no per-element
    # fp32 bound applies: the float-output rule, relative L2 within 1e-2
    dl = host_vals(g.view("d_logits", (w.T, w.E), torch.float32))
    for key, got, r in (("d_logits", dl[S], rb["d_logits"][S]),
                        ("dw_router", host_vals(g.dw_router)[C], rb["dw_router"][C])):
        rel = np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30)
        _say(f"{name} {key}: rel_l2={rel:.3e}")
        assert np.isfinite(got).all() and rel <= 1e-2, (key, rel)


# ---- routing weights applied to the expert inputs ------------------------------------------

@pytest.mark.parametrize("T,H,E,k,score", [(300, 256, 16, 4, O.SOFTMAX_PRE_RENORM),
                                           (65, 512, 8, 1, O.SIGMOID)])
def test_dispatch_backward_router_input(T, H, E, k, score):
    _say("dispatch backward router (input placement)", T, H, E, k, score)
    rng = np.random.default_rng(5 * T + k)
    logits, idx, q, row_of = _routing(rng, T, E, k, score)
    dxp, x, w = _bf(rng, (T * k, H)), _bf(rng, (T, H)), _bf(rng, (E, H), 0.02)
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    d_logits = torch.full((T, E), float("nan"), device="cuda")
    M.moe_dispatch_backward_router_input(dev_bf16(dxp), dev_bf16(x), dev(row_of), dev(idx),
                                         dev(q.astype(np.float32)), dev_bf16(w), score, dx, d_logits)
    torch.cuda.synchronize()
    dxpv, xv = O.as_values(dxp), O.as_values(x)
    ref_dq = O.prob_grad(dxpv, xv, row_of, rows_first=True)
    ref_dl = O.router_backward(logits, idx, ref_dq, score)
    absdot = np.stack([(np.abs(xv) * np.abs(dxpv[row_of[:, j]])).sum(axis=1) for j in range(k)], 1)
    b_dq = H * 2.0 ** -24 * absdot + 2.0 ** -24 * np.abs(ref_dq)
    u = 2.0 ** -24
    if score == O.SIGMOID:
        b_sel = q * (1 - q) * b_dq + 8 * u * q * np.abs(ref_dq)
    else:
        s_b = (q * b_dq).sum(axis=1, keepdims=True)
        s_abs = (q * np.abs(ref_dq)).sum(axis=1, keepdims=True)
        b_sel = q * (b_dq + s_b) + (k + 8) * u * q * (np.abs(ref_dq) + s_abs)
    bound = np.zeros((T, E))
    bound[np.arange(T)[:, None], idx] = b_sel
    got_dl = host_vals(d_logits)
    check_close(got_dl, ref_dl, bound, "d_logits (input)", floor=1e-12 * np.abs(ref_dl).max())
    # dx from the device's own d_logits would feed a device value into the reference;
    # the oracle's d_logits differs from it by at most `bound`, far below a bf16 ulp of dx
    ref_dx = O.combine(dxpv, row_of, q, ref_dl @ O.as_values(w))
    check_bf16(host_vals(dx), ref_dx, "dx (input)", slack=combine_slack(dxpv, row_of, q))


@pytest.mark.parametrize("router", [False, True])
def test_layer_input_placement(router):
    w = W.custom("inp", T=257, H=256, E=32, k=8, I=192, training=True)
    _say("layer, weights on the inputs, router", router)
    d = W.make_inputs(w)
    g = GpuMoE(w, d, router=router)
    g.prob.weight_placement = M.MOE_PLACE_INPUT
    y = host_vals(g.forward())
    if router:
        ref_logits, same, clean = _router_choice(w, d, g)
    else:
        ref_logits, same, clean = d["logits"], np.ones(w.T, bool), np.ones(w.E, bool)
    ref = O.moe_forward(d["x"], ref_logits, d["w_gu"], d["w_down"], w.k, w.score, w.I,
                        placement=O.PLACE_INPUT)
    if same.all():
        ints = g.ints()
        for key in ("topk_idx", "offsets", "row_of"):
            assert np.array_equal(ints[key], ref[key]), key
        # the scaled input rows: one fp32 product and one bf16 rounding, with the device's
        # weight within 1e-6 of the oracle's, so at most one bf16 ulp apart
        xp = host_vals(g.view("xp", (w.T * w.k, w.H), torch.bfloat16))
        from gpu_helpers import bf16_ulp
        assert (np.abs(xp - ref["xp"]) <= bf16_ulp(ref["xp"]) * (1 + 1e-9)).all()
    S = np.nonzero(same)[0]
    check_bf16(y[S], ref["y"][S], "input-placement y",
               slack=combine_slack(ref["out"], ref["row_of"])[S])
    g.backward(d["dy"])
    rb = O.moe_backward(ref, d["dy"], d["w_gu"], d["w_down"], w.I,
                        w_router_bits=d["w_router"] if router else None)
    check_bf16(host_vals(g.dx)[S], rb["dx"][S], "input-placement dx",
               slack=combine_slack(rb["dxp"], ref["row_of"], ref["topk_prob"])[S])
    C = np.nonzero(clean)[0]
    check_bf16(host_vals(g.dw_gu)[C], rb["dw_gu"][C], "input-placement dw_gu")
    check_bf16(host_vals(g.dw_down)[C], rb["dw_down"][C], "input-placement dw_down")
    if router:
        dl = host_vals(g.view("d_logits", (w.T, w.E), torch.float32))
        for key, got, r in (("d_logits", dl[S], rb["d_logits"][S]),
                            ("dw_router", host_vals(g.dw_router)[C], rb["dw_router"][C])):
            rel = np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30)
            _say(f"input placement {key}: rel_l2={rel:.3e}")
            assert np.isfinite(got).all() and rel <= 1e-2, (key, rel)
