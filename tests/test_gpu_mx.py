"""GPU parity of the MXFP8 recipe (e4m3 codes, one power-of-two scale per 32 along K)
against the oracle, through the C ABI: quantisation bit-exact (codes and scale bytes),
the block-scaled grouped GEMM and its SwiGLU epilogue against the oracle fed the same
codes (only the fp32 accumulation order differs), and the layer forward."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
import workloads as W
from gpu_helpers import GpuMoE, check_bf16, check_fp8, dev, dev_bf16, host_vals, mx_gemm_slack

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _rows(rng, R, C):
    # magnitudes from 2^-60 to 2^60 per row, zero blocks, and blocks whose amax sits in
    # [448, 512) times a power of two (their largest values saturate)
    v = rng.standard_normal((R, C)) * np.exp2(rng.integers(-60, 60, (R, 1)))
    v[0, :32] = 0.0
    v[1, :32] = rng.uniform(-1, 1, 32)
    v[1, 5] = 500.0
    v[2, 32:64] *= 0.0
    v[2, 40] = -2.0 ** -130  # fp32-subnormal block
    return W.to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("R,C", [(67, 64), (300, 2048), (5, 768)])
def test_quantize_mxfp8_rows_bit_exact(R, C):
    rng = np.random.default_rng(R + C)
    x = _rows(rng, R, C)
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    s = torch.empty((R, C // 32), dtype=torch.uint8, device="cuda")
    M.moe_quantize_mxfp8_rows(dev_bf16(x), q, s)
    torch.cuda.synchronize()
    rq, rs = O.quantize_mx_e4m3(O.as_values(x))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def test_quantize_mxfp8_weights_bit_exact():
    G, K, N = 3, 256, 96
    rng = np.random.default_rng(4)
    w = W.to_bf16_bits((rng.standard_normal((G, K, N)) * 0.02).astype(np.float32))
    q = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((G, N, K // 32), dtype=torch.uint8, device="cuda")
    M.moe_quantize_mxfp8_weights(dev_bf16(w), q, s)
    torch.cuda.synchronize()
    for g in range(G):
        rq, rs = O.quantize_mx_e4m3(O.as_values(w[g]).T)
        assert np.array_equal(q[g].cpu().numpy(), rq) and np.array_equal(s[g].cpu().numpy(), rs)


def _acc_bound(qa, sa, qb, sb, offs, K):
    """Accumulation slack of each output (mx_gemm_slack), from the decoded codes."""
    a = np.abs(O.mx_decode(qa, sa))
    out = np.zeros((a.shape[0], qb.shape[1]))
    for e in range(qb.shape[0]):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 > r0:
            out[r0:r1] = mx_gemm_slack(a[r0:r1], np.abs(O.mx_decode(qb[e], sb[e])))
    return out


def _groups(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _mx_operands(rng, counts, K, N):
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    a = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-8, 8, (rows, 1)))
    b = rng.standard_normal((G, N, K)) * 0.05
    qa, sa = O.quantize_mx_e4m3(a)
    qb, sb = zip(*[O.quantize_mx_e4m3(b[g]) for g in range(G)])
    return offs, rows, G, qa, sa, np.stack(qb), np.stack(sb)


@pytest.mark.parametrize("counts,K,N", [([130, 0, 1, 255, 64], 256, 384), ([7], 64, 64),
                                        ([300, 129, 0, 128], 2048, 192)])
def test_grouped_gemm_mxfp8(counts, K, N):
    _say("mx gemm", counts, K, N)
    rng = np.random.default_rng(K + N)
    offs, rows, G, qa, sa, qb, sb = _mx_operands(rng, counts, K, N)
    c = torch.full((rows, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_mxfp8(dev(qa), dev(sa), dev(qb), dev(sb), dev(offs), c)
    torch.cuda.synchronize()
    ref = O.to_bf16(O.grouped_gemm_mx(qa, sa, qb, sb, offs))
    # same codes and scales: only the accumulation differs. Every element is within one
    # bf16 ulp plus the accumulation slack (no max-abs excuse), and the relative L2 of the
    # rounding flips stays near 2^-9 of their share
    check_bf16(host_vals(c), ref, "mx gemm", max_abs=0.0, rel_l2=1e-3,
               slack=_acc_bound(qa, sa, qb, sb, offs, K))


@pytest.mark.parametrize("counts,K,I", [([130, 0, 1, 255, 64], 256, 192), ([40, 300], 512, 64)])
def test_grouped_gemm_mxfp8_swiglu(counts, K, I):
    _say("mx gemm swiglu", counts, K, I)
    rng = np.random.default_rng(K + I + 1)
    offs, rows, G, qa, sa, qb, sb = _mx_operands(rng, counts, K, 2 * I)
    h = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_mxfp8(dev(qa), dev(sa), dev(qb), dev(sb), dev(offs), h, swiglu=True)
    torch.cuda.synchronize()
    gu = O.grouped_gemm_mx(qa, sa, qb, sb, offs)
    ref = O.swiglu_from_gu(gu[:, :I], gu[:, I:])
    # h = silu(g) u: the g and u bounds carried through |d h| <= |u| |silu'(g)| dg + |silu(g)| du
    bgu = _acc_bound(qa, sa, qb, sb, offs, K)
    g, u = gu[:, :I], gu[:, I:]
    sg = 1 / (1 + np.exp(-g))
    dsilu = np.abs(sg * (1 + g * (1 - sg)))
    # plus the device sigmoid (2^x and a reciprocal, a few ulps; its argument g log2(e) is
    # rounded in fp32, an absolute error that makes the relative error grow with |g|)
    slack = (np.abs(u) * dsilu * bgu[:, :I] + np.abs(g * sg) * bgu[:, I:] +
             2.0 ** -24 * (2 * np.abs(g) + 8) * np.abs(ref))
    # the device sigmoid underflows to 0 for g below about -88, where |h| < 1e-30: an
    # absolute floor of 1e-30 (no other excuse)
    check_bf16(host_vals(h), ref, "mx swiglu", max_abs=1e-30, rel_l2=1e-3, slack=slack)


@pytest.mark.parametrize("name,T,E,k,H,I", [("mx_small", 300, 16, 4, 256, 192),
                                            ("mx_skewed", 600, 32, 8, 512, 256)])
def test_layer_mxfp8_forward(name, T, E, k, H, I):
    w = W.custom(name, T=T, H=H, E=E, k=k, I=I, zipf_s=1.2 if name == "mx_skewed" else 0.0,
                 n_empty=3 if name == "mx_skewed" else 0)
    _say("layer mxfp8", name)
    d = W.make_inputs(w)
    g = GpuMoE(w, d, training=False, mx=True)
    y = host_vals(g.forward())
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, mx=True)
    ints = g.ints()
    assert np.array_equal(ints["offsets"], ref["offsets"])
    # the GEMM2 input is re-quantised from the bf16 h, which may sit one bf16 rounding away
    # from the oracle's: the fp8 rule, relative L2 within 5e-2 of the quantised oracle
    check_fp8(y, ref["y"], f"{name} y")
    bf = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I)
    rel = np.linalg.norm(y - bf["y"]) / np.linalg.norm(bf["y"])
    _say(f"{name}: mxfp8 against the bf16 layer rel_l2={rel:.3e}")
