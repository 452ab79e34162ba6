"""Pins of the oracle's MXFP8 recipe (e4m3 elements, one power-of-two scale per block
of 32 along K, after the OCP Microscaling v1.0 conversion): worked blocks, saturation,
the zero block, scale invariance under powers of two, the element error bound, and the
grouped GEMM against a plain-Python block-form sum; no GPU."""
import numpy as np

import oracle as O


def test_worked_blocks():
    ones = np.ones((1, 32))
    q, s = O.quantize_mx_e4m3(ones)
    # floor(log2 1) - 8 = -8: scale byte 119, every element 256 = 2^8 (code 0x78)
    assert s.tolist() == [[119]] and (q == 0x78).all()
    assert np.array_equal(O.mx_decode(q, s), ones)
    # amax exactly 448: X = 1 and e4m3-representable values come back unchanged
    v = np.zeros((1, 32))
    v[0, :6] = [448.0, -1.5, 0.125, 3.0, -448.0, 2.0 ** -9]
    q, s = O.quantize_mx_e4m3(v)
    assert s.tolist() == [[127]] and np.array_equal(O.mx_decode(q, s), v)
    # amax 500: X = 1 still (floor(log2 500) = 8), so 500 saturates to 448 (code 0x7E)
    v[0, 0] = 500.0
    q, s = O.quantize_mx_e4m3(v)
    assert s.tolist() == [[127]] and q[0, 0] == 0x7E and O.mx_decode(q, s)[0, 0] == 448.0
    # an all-zero block: scale byte 0, zero codes
    q, s = O.quantize_mx_e4m3(np.zeros((2, 64)))
    assert not s.any() and not q.any()


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(0)
    v = O.as_values(O.f32_to_bf16_bits(rng.standard_normal((5, 96)).astype(np.float32)))
    q0, s0 = O.quantize_mx_e4m3(v)
    for j in (-20, -3, 1, 7):
        q, s = O.quantize_mx_e4m3(v * 2.0 ** j)
        assert np.array_equal(q, q0) and np.array_equal(s.astype(int), s0.astype(int) + j)


def test_element_error_bound():
    rng = np.random.default_rng(1)
    v = O.as_values(O.f32_to_bf16_bits((rng.standard_normal((40, 128)) *
                                        np.exp(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)))
    q, s = O.quantize_mx_e4m3(v)
    d = O.mx_decode(q, s)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    t = np.abs(v) / X
    ok = t <= 448                     # not saturated
    # nearest-even e4m3: half an ulp, relative 2^-4 for normals, 2^-10 absolute (times X)
    # on the subnormal grid
    bound = np.maximum(np.abs(v) * 2.0 ** -4, X * 2.0 ** -10)
    assert (np.abs(d - v)[ok] <= bound[ok] * (1 + 1e-12)).all()
    assert (np.abs(d[~ok]) == 448 * X[~ok]).all()


def test_grouped_gemm_mx_block_form():
    rng = np.random.default_rng(2)
    counts = [3, 0, 2]
    offs = np.concatenate([[0], np.cumsum(counts)])
    K, N = 64, 3
    a = rng.standard_normal((5, K))
    b = rng.standard_normal((3, N, K)) * 0.1
    qa, sa = O.quantize_mx_e4m3(a)
    qb, sb = zip(*[O.quantize_mx_e4m3(b[e]) for e in range(3)])
    qb, sb = np.stack(qb), np.stack(sb)
    got = O.grouped_gemm_mx(qa, sa, qb, sb, offs, exact=True)
    ea, eb = O.e4m3_decode(qa), O.e4m3_decode(qb)
    for e in range(3):
        for r in range(offs[e], offs[e + 1]):
            for n in range(N):
                tot = 0.0
                for blk in range(K // 32):
                    part = sum(float(ea[r, k]) * float(eb[e, n, k]) for k in range(32 * blk, 32 * blk + 32))
                    tot += part * 2.0 ** (int(sa[r, blk]) - 127) * 2.0 ** (int(sb[e, n, blk]) - 127)
                assert got[r, n] == tot


def test_mx_forward_close_to_bf16_forward():
    import workloads as W
    w = W.custom("mx", T=64, H=128, E=4, k=2, I=128)
    d = W.make_inputs(w)
    a = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I)
    b = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, mx=True)
    rel = np.linalg.norm(b["y"] - a["y"]) / np.linalg.norm(a["y"])
    assert 1e-3 < rel < 0.1


# ---- the MXFP8 backward: token-axis blocks and the four backward GEMMs ----------------------

def _ocp_block(vals):
    """One block by the OCP rule, scalar arithmetic: (scale byte, codes)."""
    import math
    amax = max(abs(float(v)) for v in vals)
    if amax == 0:
        se = -127
    else:
        se = max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
    codes = O.e4m3_encode(np.array([float(v) / 2.0 ** se for v in vals], np.float32))
    return se + 127, codes


def test_mx_cols_brute_force():
    rng = np.random.default_rng(3)
    counts = [5, 0, 70, 32]
    offs = np.concatenate([[0], np.cumsum(counts)])
    C = 3
    v = O.as_values(O.f32_to_bf16_bits(rng.standard_normal((offs[-1], C)).astype(np.float32)))
    v[offs[2] + 40] *= 2.0 ** 30      # one large row: its block's scale, not its neighbours'
    q, s, co = O.quantize_mx_cols(v, offs)
    assert co.tolist() == [0, 64, 64, 192, 256]
    assert q.shape == (C, 256) and s.shape == (C, 8)
    for e in range(4):
        n = counts[e]
        for c in range(C):
            for b in range((co[e + 1] - co[e]) // 32):
                blk = [v[offs[e] + 32 * b + i, c] if 32 * b + i < n else 0.0 for i in range(32)]
                byte, codes = _ocp_block(blk)
                p = co[e] + 32 * b
                assert s[c, p // 32] == byte
                assert np.array_equal(q[c, p:p + 32], codes)


def test_mx_wgrad_block_form():
    rng = np.random.default_rng(4)
    counts = [40, 0, 7]
    offs = np.concatenate([[0], np.cumsum(counts)])
    M, N = 2, 3
    a = rng.standard_normal((offs[-1], M))
    b = rng.standard_normal((offs[-1], N)) * 0.01
    qa, sa, co = O.quantize_mx_cols(a, offs)
    qb, sb, _ = O.quantize_mx_cols(b, offs)
    got = O.grouped_gemm_mx_wgrad(qa, sa, qb, sb, co, exact=True)
    ea, eb = O.e4m3_decode(qa), O.e4m3_decode(qb)
    assert not got[1].any()
    for e in range(3):
        for m in range(M):
            for n in range(N):
                tot = 0.0
                for p0 in range(co[e], co[e + 1], 32):
                    part = sum(float(ea[m, p]) * float(eb[n, p]) for p in range(p0, p0 + 32))
                    tot += part * 2.0 ** (int(sa[m, p0 // 32]) - 127) * 2.0 ** (int(sb[n, p0 // 32]) - 127)
                assert got[e, m, n] == tot


def _mx_case():
    import workloads as W
    w = W.custom("mxb", T=48, H=128, E=4, k=2, I=64)
    d = W.make_inputs(w)
    fwd = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, mx=True)
    rng = np.random.default_rng(5)
    dy = O.f32_to_bf16_bits(rng.standard_normal((w.T, w.H)).astype(np.float32))
    bwd = O.moe_backward(fwd, dy, d["w_gu"], d["w_down"], w.I, mx=True)
    return w, d, fwd, bwd


def _quant_bound(a, b, axis_a, axis_b):
    """sum_k |a_k b_k - qa_k qb_k| bound: per element |q - v| <= max(|v|/8, X/1024), X the
    block scale (2^(floor(log2 amax) - 8)) of 32 consecutive values along the given axis."""
    def err(v, axis):
        v = np.moveaxis(np.asarray(v, np.float64), axis, -1)
        L = v.shape[-1]
        pad = (-L) % 32
        vp = np.concatenate([v, np.zeros(v.shape[:-1] + (pad,))], axis=-1)
        blk = vp.reshape(v.shape[:-1] + (-1, 32))
        amax = np.abs(blk).max(axis=-1, keepdims=True)
        X = np.where(amax > 0, np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8), 0)
        e = np.maximum(np.abs(blk) / 8, X / 1024).reshape(vp.shape)[..., :L]
        return np.moveaxis(e, -1, axis)
    return err(a, axis_a), err(b, axis_b)


def test_mx_backward_gemms_within_quantisation_bound():
    w, d, fwd, bwd = _mx_case()
    offs = fwd["offsets"]
    wgu = [O.as_values(d["w_gu"][e]) for e in range(w.E)]
    wdn = [O.as_values(d["w_down"][e]) for e in range(w.E)]
    d_out, dgu = bwd["d_out"], bwd["dgu"]
    for e in range(w.E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 == r0:
            continue
        # dh = d_out W_down^T: blocks along H for both
        a, b = d_out[r0:r1], wdn[e]                 # [n, H], [I, H]
        ea, eb = _quant_bound(a, b, 1, 1)
        bound = ea @ np.abs(b).T + np.abs(a) @ eb.T + ea @ eb.T
        exact = a @ b.T
        assert (np.abs(bwd["dh"][r0:r1] - exact) <= bound + 2.0 ** -23 * np.abs(exact) + 1e-30).all()
        # dxp = dGU W_gu^T: blocks along 2I
        a, b = dgu[r0:r1], wgu[e]                   # [n, 2I], [H, 2I]
        ea, eb = _quant_bound(a, b, 1, 1)
        bound = ea @ np.abs(b).T + np.abs(a) @ eb.T + ea @ eb.T
        exact = a @ b.T
        assert (np.abs(bwd["dxp"][r0:r1] - exact) <= bound * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(exact) + 1e-30).all()
        # dW_down = h^T d_out, dW_gu = xp^T dGU: blocks along the expert's tokens
        for got, a, b in ((bwd["dw_down"][e], fwd["h"][r0:r1], d_out[r0:r1]),
                          (bwd["dw_gu"][e], fwd["xp"][r0:r1], dgu[r0:r1])):
            ea, eb = _quant_bound(a, b, 0, 0)
            bound = ea.T @ np.abs(b) + np.abs(a).T @ eb + ea.T @ eb
            exact = a.T @ b
            assert (np.abs(got - exact) <= bound * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(exact) + 1e-30).all()


def test_mx_backward_block_axes():
    """Scaling a tensor by 2 along the axis its blocks do NOT run along changes only the
    matching output slice (exactly doubled): routed rows for the data gradients (blocks
    along K), channels for the weight gradients (blocks along the tokens)."""
    w, d, fwd, bwd = _mx_case()
    offs = fwd["offsets"]
    wg, wd = np.asarray(d["w_gu"]), np.asarray(d["w_down"])
    r = int(offs[1]) + 1                                        # a row of expert 1
    d2 = bwd["d_out"].copy()
    d2[r] *= 2
    b2 = O.expert_mlp_mx_backward(fwd, fwd["xp"], d2, wg, wd, offs, w.I)
    for key in ("dh", "dgu", "dxp"):
        assert np.array_equal(b2[key][r], 2 * bwd[key][r])
        keep = np.arange(len(d2)) != r
        assert np.array_equal(b2[key][keep], bwd[key][keep])
    c = 5
    f2 = dict(fwd)
    f2["h"] = fwd["h"].copy()
    f2["h"][:, c] *= 2
    xp2 = fwd["xp"].copy()
    xp2[:, c] *= 2
    b3 = O.expert_mlp_mx_backward(f2, xp2, bwd["d_out"], wg, wd, offs, w.I)
    for key in ("dw_down", "dw_gu"):
        assert np.array_equal(b3[key][:, c], 2 * bwd[key][:, c])
        keep = np.arange(b3[key].shape[1]) != c
        assert np.array_equal(b3[key][:, keep], bwd[key][:, keep])


def test_mx_backward_close_to_bf16_backward():
    w, d, fwd, bwd = _mx_case()
    ref_f = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I)
    rng = np.random.default_rng(5)
    dy = O.f32_to_bf16_bits(rng.standard_normal((w.T, w.H)).astype(np.float32))
    ref = O.moe_backward(ref_f, dy, d["w_gu"], d["w_down"], w.I)
    for key in ("dx", "dw_gu", "dw_down"):
        rel = np.linalg.norm(bwd[key] - ref[key]) / np.linalg.norm(ref[key])
        assert 1e-3 < rel < 0.15, (key, rel)
