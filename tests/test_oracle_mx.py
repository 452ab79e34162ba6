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
