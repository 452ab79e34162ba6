"""GPU parity of the MXFP8 backward against the oracle, through the C ABI: the token-axis
quantisation of the weight-gradient operands bit-exact (codes, scale bytes, expert starts),
the weight-gradient GEMM and the SwiGLU-backward GEMM against the oracle fed the same
codes (only the fp32 accumulation order differs), and the layer's training step."""
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


def _groups(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _rows(rng, R, C):
    # magnitudes from 2^-60 to 2^60 per column, one huge row, a zero stretch, saturating
    # blocks ([448, 512) times a power of two)
    v = rng.standard_normal((R, C)) * np.exp2(rng.integers(-60, 60, (1, C)))
    if R > 40:
        v[3, :] *= 2.0 ** 20
        v[8:40, 0] = 0.0
        v[10, 1] = 500.0 * 2.0 ** 10
        v[11:42, 1] = rng.uniform(-1, 1, 31) * 2.0 ** 10
    return W.to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("counts,C", [([130, 0, 1, 255, 64, 33], 64), ([7], 200),
                                      ([300, 129, 0, 128], 768),
                                      ([(i * 37) % 70 for i in range(600)], 64)])
def test_quantize_mxfp8_cols_bit_exact(counts, C):
    _say("mx cols", counts, C)
    rng = np.random.default_rng(C + len(counts))
    offs = _groups(counts)
    R, G = int(offs[-1]), len(counts)
    x = _rows(rng, R, C)
    Kp = M.moe_mxfp8_cols_capacity(R, G)
    co = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
    qt = torch.full((C, Kp), 0xEE, dtype=torch.uint8, device="cuda")
    st = torch.full((C, Kp // 32), 0xEE, dtype=torch.uint8, device="cuda")
    d_offs = dev(offs)
    M.moe_mxfp8_col_offsets(d_offs, co)
    M.moe_quantize_mxfp8_cols(dev_bf16(x), d_offs, co, qt, st)
    torch.cuda.synchronize()
    rq, rs, rco = O.quantize_mx_cols(O.as_values(x), offs)
    assert np.array_equal(co.cpu().numpy(), rco)
    n = int(rco[-1])
    assert np.array_equal(st.cpu().numpy()[:, :n // 32], rs)
    assert np.array_equal(qt.cpu().numpy()[:, :n], rq)
    # nothing written past the last expert's range
    assert (qt.cpu().numpy()[:, n:] == 0xEE).all()


def _acc_bound_wgrad(qa, sa, qb, sb, co):
    a, b = np.abs(O.mx_decode(qa, sa)), np.abs(O.mx_decode(qb, sb))
    G = len(co) - 1
    out = np.zeros((G, a.shape[0], b.shape[0]))
    for g in range(G):
        c0, c1 = int(co[g]), int(co[g + 1])
        if c1 > c0:
            out[g] = mx_gemm_slack(a[:, c0:c1], b[:, c0:c1])
    return out


@pytest.mark.parametrize("counts,M_,N", [([130, 0, 1, 255, 64], 192, 256), ([7], 64, 64),
                                         ([300, 129, 0, 128], 256, 192)])
def test_grouped_gemm_mxfp8_wgrad(counts, M_, N):
    _say("mx wgrad", counts, M_, N)
    rng = np.random.default_rng(M_ + N)
    offs = _groups(counts)
    R, G = int(offs[-1]), len(counts)
    a = rng.standard_normal((R, M_)) * np.exp2(rng.integers(-8, 8, (1, M_)))
    b = rng.standard_normal((R, N)) * 0.05
    qa, sa, co = O.quantize_mx_cols(a, offs)
    qb, sb, _ = O.quantize_mx_cols(b, offs)
    Kp = M.moe_mxfp8_cols_capacity(R, G)
    pad = Kp - qa.shape[1]
    # the device buffers are Kp wide; the columns past the last expert are never read
    fill = lambda q: np.concatenate([q, np.full((q.shape[0], pad), 0x7F, np.uint8)], axis=1)
    fills = lambda s: np.concatenate([s, np.full((s.shape[0], pad // 32), 0xFF, np.uint8)], axis=1)
    c = torch.full((G, M_, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_mxfp8_wgrad(dev(fill(qa)), dev(fills(sa)), dev(fill(qb)), dev(fills(sb)),
                                   dev(co.astype(np.int32)), c)
    torch.cuda.synchronize()
    ref = O.to_bf16(O.grouped_gemm_mx_wgrad(qa, sa, qb, sb, co))
    check_bf16(host_vals(c), ref, "mx wgrad", max_abs=0.0, rel_l2=1e-3,
               slack=_acc_bound_wgrad(qa, sa, qb, sb, co))


@pytest.mark.parametrize("counts,K,I", [([130, 0, 1, 255, 64], 256, 192), ([40, 300], 512, 64)])
def test_grouped_gemm_mxfp8_swiglu_bwd(counts, K, I):
    _say("mx swiglu bwd", counts, K, I)
    rng = np.random.default_rng(K + I + 2)
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    a = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-8, 8, (rows, 1)))
    b = rng.standard_normal((G, I, K)) * 0.05
    qa, sa = O.quantize_mx_e4m3(a)
    qb, sb = zip(*[O.quantize_mx_e4m3(b[g]) for g in range(G)])
    qb, sb = np.stack(qb), np.stack(sb)
    gu = W.to_bf16_bits((rng.standard_normal((rows, 2 * I)) * 3).astype(np.float32))
    dgu = torch.full((rows, 2 * I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_mxfp8_swiglu_bwd(dev(qa), dev(sa), dev(qb), dev(sb), dev(offs),
                                        dev_bf16(gu), dgu)
    torch.cuda.synchronize()
    dh = O.grouped_gemm_mx(qa, sa, qb, sb, offs)
    guv = O.as_values(gu)
    g, u = guv[:, :I], guv[:, I:]
    dg, du = O.swiglu_backward(dh, g, u)
    # the dh accumulation bound carried through the (linear in dh) SwiGLU backward, plus the
    # device sigmoid's few ulps (its argument rounded in fp32: relative error growing with |g|)
    aa = np.abs(O.mx_decode(qa, sa))
    bdh = np.zeros_like(dh)
    for e in range(G):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 > r0:
            bdh[r0:r1] = mx_gemm_slack(aa[r0:r1], np.abs(O.mx_decode(qb[e], sb[e])))
    s = 1 / (1 + np.exp(-g))
    cg, cu = np.abs(u * s * (1 + g * (1 - s))), np.abs(g * s)
    sig = 2.0 ** -24 * (2 * np.abs(g) + 8)
    got = host_vals(dgu)
    check_bf16(got[:, :I], dg, "mx dg", max_abs=1e-30, rel_l2=1e-3,
               slack=cg * bdh + sig * (1 + np.abs(g)) * np.abs(dg))
    check_bf16(got[:, I:], du, "mx du", max_abs=1e-30, rel_l2=1e-3,
               slack=cu * bdh + sig * np.abs(du))


@pytest.mark.parametrize("name,T,E,k,H,I", [("mx_small", 300, 16, 4, 256, 192),
                                            ("mx_skewed", 600, 32, 8, 512, 256)])
def test_layer_mxfp8_training(name, T, E, k, H, I):
    w = W.custom(name, T=T, H=H, E=E, k=k, I=I, zipf_s=1.2 if name == "mx_skewed" else 0.0,
                 n_empty=3 if name == "mx_skewed" else 0)
    _say("layer mxfp8 training", name)
    d = W.make_inputs(w)
    rng = np.random.default_rng(T)
    dy = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = GpuMoE(w, d, training=True, mx=True)
    y = host_vals(g.forward())
    g.backward(dy)
    fwd = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, mx=True)
    ref = O.moe_backward(fwd, dy, d["w_gu"], d["w_down"], w.I, mx=True)
    ints = g.ints()
    assert np.array_equal(ints["offsets"], fwd["offsets"])
    check_fp8(y, fwd["y"], f"{name} y")
    N = T * k
    gu = host_vals(g.view("gu", (N, 2 * I), torch.bfloat16))
    check_fp8(gu, np.concatenate([O.to_bf16(fwd["g"]), O.to_bf16(fwd["u"])], axis=1), f"{name} gu",
              rel_l2=1e-3)
    dgu = host_vals(g.view("dgu", (N, 2 * I), torch.bfloat16))
    # Both sides run the same recipe; they part only where a value the GPU rounded one bf16
    # ulp away from the oracle's (an accumulation-order difference) crosses an e4m3 rounding
    # boundary when it is quantised for the next GEMM, moving that operand by up to 2^-3 of
    # itself. Such flips are rare: relative L2 1e-2 (the MXFP8 layer differs from the bf16
    # layer by about 7e-2, so a result that skipped the recipe fails).
    rels = {}
    rels["dgu"] = check_fp8(dgu, ref["dgu"], f"{name} dgu", rel_l2=1e-2)
    rels["dx"] = check_fp8(host_vals(g.dx), ref["dx"], f"{name} dx", rel_l2=1e-2)
    rels["dw_gu"] = check_fp8(host_vals(g.dw_gu), ref["dw_gu"], f"{name} dw_gu", rel_l2=1e-2)
    rels["dw_down"] = check_fp8(host_vals(g.dw_down), ref["dw_down"], f"{name} dw_down", rel_l2=1e-2)
    # experts with no rows: zero weight gradients
    empty = np.flatnonzero(np.diff(fwd["offsets"]) == 0)
    assert not host_vals(g.dw_gu)[empty].any() and not host_vals(g.dw_down)[empty].any()
    _say(name, {k_: f"{v:.2e}" for k_, v in rels.items()})


def test_layer_mxfp8_training_full_size_qwen3():
    """The Qwen3-shaped block (T=4096, H=2048, E=128, top-8, I=768) in the launch
    configuration the benchmark times with --mx. Routing and offsets whole (bit-exact); an
    expert's output rows, dgu and dxp rows and weight gradients depend only on the rows
    routed to it, so the oracle runs that expert's MXFP8 MLP forward and backward alone,
    on sampled experts (the most and the least loaded, and one more)."""
    w = W.WORKLOADS["qwen3"]
    _say("layer mxfp8 training full size qwen3")
    d = W.make_inputs("qwen3")
    g = GpuMoE(w, d, training=True, mx=True)
    g.forward()
    g.backward(d["dy"])
    idx, q, counts, _, _ = O.router_topk(d["logits"], w.k, w.score)
    offs, row_of, src_of = O.dispatch_meta(idx, w.E)
    ints = g.ints()
    assert np.array_equal(ints["offsets"], offs) and np.array_equal(ints["row_of"], row_of)
    N, H, I = w.T * w.k, w.H, w.I
    out = g.view("out", (N, H), torch.bfloat16)
    dgu = g.view("dgu", (N, 2 * I), torch.bfloat16)
    dxp = g.view("dxp", (N, H), torch.bfloat16)
    dy = O.as_values(d["dy"])
    x = O.as_values(d["x"])
    qr = np.zeros(N)
    for j in range(w.k):
        qr[row_of[:, j]] = q[:, j]
    n = np.diff(offs)
    for e in (int(np.argmax(n)), int(np.argmin(np.where(n > 0, n, N))), 77):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        _say("expert", e, "rows", r1 - r0)
        eo = np.array([0, r1 - r0])
        xp = x[src_of[r0:r1]]
        mlp = O.expert_mlp_mx(xp, d["w_gu"][e:e + 1], d["w_down"][e:e + 1], eo, I)
        d_out = O.to_bf16(dy[src_of[r0:r1]] * qr[r0:r1, None])
        rb = O.expert_mlp_mx_backward(mlp, xp, d_out, d["w_gu"][e:e + 1], d["w_down"][e:e + 1], eo, I)
        check_fp8(host_vals(out[r0:r1]), mlp["out"], f"out[{e}]", rel_l2=1e-2)
        check_fp8(host_vals(dgu[r0:r1]), rb["dgu"], f"dgu[{e}]", rel_l2=1e-2)
        check_fp8(host_vals(dxp[r0:r1]), rb["dxp"], f"dxp[{e}]", rel_l2=1e-2)
        check_fp8(host_vals(g.dw_down[e]), rb["dw_down"][0], f"dw_down[{e}]", rel_l2=1e-2)
        check_fp8(host_vals(g.dw_gu[e]), rb["dw_gu"][0], f"dw_gu[{e}]", rel_l2=1e-2)
    assert torch.isfinite(g.dx).all().item()
    assert torch.isfinite(g.dw_gu).all().item() and torch.isfinite(g.dw_down).all().item()


@pytest.mark.parametrize("align", [64, 128])
def test_layer_mxfp8_training_padded(align):
    """MXFP8 training on a padded dispatch: the padding rows are zero, which changes no
    block maximum and no sum (the token-axis blocks start at every expert's first row
    either way), so the results are those of the unpadded MXFP8 oracle."""
    w = W.custom("mxpad", T=300, H=256, E=16, k=4, I=192, zipf_s=1.2, n_empty=3)
    _say("layer mxfp8 training padded", align)
    d = W.make_inputs(w)
    rng = np.random.default_rng(align)
    dy = W.to_bf16_bits(rng.standard_normal((w.T, w.H)).astype(np.float32))
    g = GpuMoE(w, d, training=True, mx=True)
    g.prob.align_size = align
    g.ws = torch.empty(M.moe_workspace_bytes(g.prob), dtype=torch.uint8, device="cuda")
    g.ws.fill_(0xFF)
    g.views = M.moe_workspace_views(g.prob, g.ws)
    y = host_vals(g.forward())
    g.backward(dy)
    fwd = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, mx=True)
    ref = O.moe_backward(fwd, dy, d["w_gu"], d["w_down"], w.I, mx=True)
    r_off, _, r_row, _ = O.dispatch_meta_padded(fwd["topk_idx"], w.E, align)
    assert np.array_equal(g.view("offsets", (w.E + 1,), torch.int32).cpu().numpy(), r_off)
    assert np.array_equal(g.view("row_of", (w.T, w.k), torch.int32).cpu().numpy(), r_row)
    check_fp8(y, fwd["y"], f"mx padded{align} y", rel_l2=1e-2)
    check_fp8(host_vals(g.dx), ref["dx"], f"mx padded{align} dx", rel_l2=1e-2)
    check_fp8(host_vals(g.dw_gu), ref["dw_gu"], f"mx padded{align} dw_gu", rel_l2=1e-2)
    check_fp8(host_vals(g.dw_down), ref["dw_down"], f"mx padded{align} dw_down", rel_l2=1e-2)


def test_layer_mxfp8_training_with_router():
    """MXFP8 training with the layer's own router projection: the routing comes from
    device-computed logits, so near-tie tokens may choose differently from the oracle; as
    in the bf16 router test, outputs are compared on the tokens whose choice matches and
    weight gradients on the experts no differing token chose."""
    from test_gpu_router import _router_choice, _valid_dispatch
    w = W.custom("mxrouter", T=300, H=256, E=16, k=4, I=192, training=True)
    _say("layer mxfp8 training with router")
    d = W.make_inputs(w)
    g = GpuMoE(w, d, training=True, mx=True, router=True)
    y = host_vals(g.forward())
    ref_logits, same, clean = _router_choice(w, d, g)
    fwd = O.moe_forward(d["x"], ref_logits, d["w_gu"], d["w_down"], w.k, w.score, w.I, mx=True)
    ints = g.ints()
    if same.all():
        for key in ("topk_idx", "counts", "offsets", "row_of", "src_of"):
            assert np.array_equal(ints[key], fwd[key]), key
    else:
        _valid_dispatch(ints, w.E)
    S, C = np.nonzero(same)[0], np.nonzero(clean)[0]
    check_fp8(y[S], fwd["y"][S], "mx router y", rel_l2=1e-2)
    g.backward(d["dy"])
    rb = O.moe_backward(fwd, d["dy"], d["w_gu"], d["w_down"], w.I, w_router_bits=d["w_router"], mx=True)
    check_fp8(host_vals(g.dx)[S], rb["dx"][S], "mx router dx", rel_l2=1e-2)
    check_fp8(host_vals(g.dw_gu)[C], rb["dw_gu"][C], "mx router dw_gu", rel_l2=1e-2)
    check_fp8(host_vals(g.dw_down)[C], rb["dw_down"][C], "mx router dw_down", rel_l2=1e-2)
    dl = host_vals(g.view("d_logits", (w.T, w.E), torch.float32))
    check_fp8(dl[S], rb["d_logits"][S], "mx router d_logits", rel_l2=1e-2)
    check_fp8(host_vals(g.dw_router)[C], rb["dw_router"][C], "mx router dw_router", rel_l2=1e-2)


def test_layer_mxfp8_fused_codes_bit_exact():
    # the MXFP8 row codes of every row-blocked GEMM operand of the layer: written by the
    # dispatch copies as they go (forward: the x rows; backward: the combine-backward rows
    # d_out = bf16(p dy), one quantisation per weighted copy) or by the row quantiser (h,
    # dgu). Codes and scale bytes equal the oracle's quantisation of the bf16 rows the layer
    # kept (I = 192: the second 128-column h tile half full; skewed routing with empty
    # experts)
    w = W.custom("mx_codes", T=300, H=256, E=16, k=4, I=192, zipf_s=1.2, n_empty=3)
    _say("layer mxfp8 fused codes")
    d = W.make_inputs(w)
    dy = W.to_bf16_bits(np.random.default_rng(2).standard_normal((w.T, w.H)).astype(np.float32))
    g = GpuMoE(w, d, training=True, mx=True)
    g.forward()
    N, H, I = w.T * w.k, w.H, w.I

    def codes_match(rows_name, C, q_name, s_name, label):
        rows = g.view(rows_name, (N, C), torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
        q = g.view(q_name, (N, C), torch.uint8).cpu().numpy()
        s = g.view(s_name, (N, C // 32), torch.uint8).cpu().numpy()
        rq, rs = O.quantize_mx_e4m3(O.as_values(rows))
        assert np.array_equal(s, rs), f"{label}: scale bytes"
        assert np.array_equal(q, rq), f"{label}: codes"

    codes_match("xp", H, "xq", "xq_scale", "forward xp")
    codes_match("h", I, "hq", "hq_scale", "forward h")
    g.backward(dy)
    codes_match("d_out", H, "xq", "xq_scale", "backward d_out")
    codes_match("dgu", 2 * I, "dgq", "dgq_scale", "backward dgu")
