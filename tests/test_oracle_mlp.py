"""Pins of the oracle's grouped expert MLP, combine and backward: brute-force loops,
a per-token dense reference that shares no step with the permuted path, row
independence, library SiLU, and central finite differences; no GPU."""
import numpy as np
import pytest
import scipy.special as sp

import oracle as O
import workloads as W


def _bf(a):
    return O.bf16_bits_to_f64(O.f32_to_bf16_bits(np.asarray(a, np.float32)))


def test_grouped_gemm_matches_triple_loop():
    rng = np.random.default_rng(0)
    E, K, N = 3, 5, 4
    counts = [2, 0, 3]
    offs = np.concatenate([[0], np.cumsum(counts)])
    a = rng.standard_normal((offs[-1], K))
    b = rng.standard_normal((E, K, N))
    got = O.grouped_gemm(a, b, offs, exact=True)
    ref = np.zeros_like(got)
    for e in range(E):
        for r in range(offs[e], offs[e + 1]):
            for c in range(N):
                s = 0.0
                for kk in range(K):
                    s += a[r, kk] * b[e, kk, c]
                ref[r, c] = s
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-14)


def test_grouped_gemm_dw_matches_loop_and_zero_for_empty():
    rng = np.random.default_rng(1)
    counts = [3, 0, 2, 1]
    offs = np.concatenate([[0], np.cumsum(counts)])
    a = rng.standard_normal((6, 4))
    b = rng.standard_normal((6, 5))
    got = O.grouped_gemm_dw(a, b, offs, exact=True)
    for e in range(4):
        ref = np.zeros((4, 5))
        for r in range(offs[e], offs[e + 1]):
            ref += np.outer(a[r], b[r])
        assert np.allclose(got[e], ref, rtol=1e-14, atol=1e-14)
    assert not got[1].any()


def test_silu_matches_library():
    g = np.linspace(-30, 30, 10001)
    assert np.allclose(O.silu(g), g * sp.expit(g), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def _dense_reference(x, logits, w_gu, w_d, k, score, I, shared=None, exact=False):
    """Per token, no dispatch: y[t] = sum_j q_j * MLP_{e_j}(x[t]) (+ shared MLP(x[t]))."""
    idx = O.topk_select(logits, k)
    q = O.topk_probs(logits, idx, score, exact)
    T, H = x.shape
    y = np.zeros((T, H))
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = idx[t, j]
            gu = O.to_f32(x[t] @ w_gu[e], exact)
            h = O.to_bf16(O.silu(gu[:I]) * gu[I:], exact)
            out = O.to_bf16(O.to_f32(h @ w_d[e], exact), exact)
            acc += q[t, j] * out
        if shared is not None:
            sgu, sd = shared
            Is = sd.shape[0]
            gu = O.to_f32(x[t] @ sgu, exact)
            h = O.to_bf16(O.silu(gu[:Is]) * gu[Is:], exact)
            acc += O.to_bf16(O.to_f32(h @ sd, exact), exact)
        y[t] = O.to_bf16(acc, exact)
    return y


@pytest.mark.parametrize("name", ["tiny", "small_shared", "small_post"])
def test_forward_matches_dense_per_token_reference(name):
    if name == "tiny":
        w = W.WORKLOADS["tiny"]
    elif name == "small_shared":
        w = W.custom("s", T=24, H=64, E=16, k=1, I=64, score=O.SIGMOID, shared_I=128,
                     hot_experts=(0, 1, 2), hot_bias=2.0)
    else:
        w = W.custom("p", T=40, H=64, E=8, k=2, I=128, score=O.SOFTMAX_POST)
    d = W.make_inputs(w)
    x = O.bf16_bits_to_f64(d["x"])
    wgu, wd = O.bf16_bits_to_f64(d["w_gu"]), O.bf16_bits_to_f64(d["w_down"])
    shared = None
    if w.shared_I:
        shared = (O.bf16_bits_to_f64(d["shared_gu"]), O.bf16_bits_to_f64(d["shared_down"]))
    for exact in (True, False):
        r = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I,
                          d.get("shared_gu"), d.get("shared_down"), exact=exact)
        ref = _dense_reference(x, d["logits"], wgu, wd, w.k, w.score, w.I, shared, exact)
        if exact:
            assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-15)
        else:
            # same rounding points; only float64 summation order differs
            ulp = np.spacing(np.abs(ref).astype(np.float32)) * 65536
            assert np.all(np.abs(r["y"] - ref) <= ulp)
            assert np.mean(r["y"] == ref) > 0.999


def test_row_independence_under_token_shuffle():
    w = W.custom("r", T=48, H=64, E=8, k=2, I=64)
    d = W.make_inputs(w)
    perm = np.random.default_rng(3).permutation(w.T)
    a = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, exact=True)
    b = O.moe_forward(d["x"][perm], d["logits"][perm], d["w_gu"], d["w_down"], w.k, w.score, w.I,
                      exact=True)
    assert np.allclose(a["y"][perm], b["y"], rtol=1e-13, atol=1e-16)


def test_fp8_gemm_uses_decoded_codes_and_scales():
    rng = np.random.default_rng(11)
    E, K, N = 2, 32, 16
    offs = np.array([0, 5, 9])
    a = _bf(rng.standard_normal((9, K)))
    b = _bf(rng.standard_normal((E, K, N)) * 0.02)
    qa, sa = O.quantize_rows_e4m3(a)
    qb, sb = O.quantize_cols_e4m3(b)
    got = O.grouped_gemm(O.e4m3_decode(qa), O.e4m3_decode(qb), offs, False, sa, sb)
    for e in range(E):
        for r in range(offs[e], offs[e + 1]):
            for c in range(N):
                s = sum(O.e4m3_decode(qa[r, kk]) * O.e4m3_decode(qb[e, kk, c]) for kk in range(K))
                ref = np.float32(s * float(sa[r]) * float(sb[e, c]))
                assert got[r, c] == ref
    # and it approximates the bf16 product to fp8 accuracy
    ref = O.grouped_gemm(a, b, offs, exact=True)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 0.08


def test_fp8_forward_close_to_bf16_forward():
    w = W.custom("f", T=64, H=256, E=8, k=2, I=128)
    d = W.make_inputs(w)
    a = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I)
    b = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, fp8=True)
    rel = np.linalg.norm(a["y"] - b["y"]) / np.linalg.norm(a["y"])
    assert 1e-3 < rel < 0.1


def _loss(x, wgu, wd, logits, dy, w):
    r = O.moe_forward(x, logits, wgu, wd, w.k, w.score, w.I, exact=True)
    return float((r["y"] * dy).sum()), r


@pytest.mark.parametrize("score", [O.SOFTMAX_PRE_RENORM, O.SIGMOID])
def test_backward_matches_finite_differences(score):
    w = W.custom("fd", T=6, H=8, E=3, k=2 if score != O.SIGMOID else 1, I=4, score=score)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((w.T, w.H))
    wgu = rng.standard_normal((w.E, w.H, 2 * w.I)) * 0.5
    wd = rng.standard_normal((w.E, w.I, w.H)) * 0.5
    logits = rng.standard_normal((w.T, w.E)).astype(np.float32)
    dy = rng.standard_normal((w.T, w.H))
    _, fwd = _loss(x, wgu, wd, logits, dy, w)
    g = O.moe_backward(fwd, dy, wgu, wd, w.I, exact=True)
    eps = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("w_gu", wgu, g["dw_gu"]), ("w_down", wd, g["dw_down"])):
        flat = arr.reshape(-1)
        gflat = grad.reshape(-1)
        scale = np.abs(gflat).max()
        for i in np.random.default_rng(5).choice(flat.size, size=min(40, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp, _ = _loss(x, wgu, wd, logits, dy, w)
            flat[i] = old - eps
            lm, _ = _loss(x, wgu, wd, logits, dy, w)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gflat[i]) <= 1e-7 * scale + 1e-6 * abs(fd), (name, i, fd, gflat[i])


def test_backward_empty_expert_has_zero_gradient():
    w = W.custom("z", T=16, H=64, E=4, k=1, I=64, training=True)
    d = W.make_inputs(w)
    logits = d["logits"].copy()
    logits[:, 3] = -100.0      # expert 3 never chosen
    r = O.moe_forward(d["x"], logits, d["w_gu"], d["w_down"], w.k, w.score, w.I)
    assert r["counts"][3] == 0
    g = O.moe_backward(r, d["dy"], d["w_gu"], d["w_down"], w.I)
    assert not g["dw_gu"][3].any() and not g["dw_down"][3].any()
    assert g["dw_gu"][0].any()
