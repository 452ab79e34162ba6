"""GPU parity (through the C ABI) of ScaledSwiGLU (Transformer Engine guide "Mixture of
Experts", Grouped MLP: the routing weights scale the SwiGLU output before FC2, the combine
sums unweighted): the scaled SwiGLU GEMM, its backward with the weight-gradient partials,
the permuted weights, the router's dispatch backward, and the whole layer forward and
backward, with and without the router projection, against the oracle."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
import workloads as W
from gpu_helpers import (GpuMoE, check_bf16, check_close, combine_slack, dev, dev_bf16,
                         host_vals)
from test_gpu_parity import GROUP_CASES, _groups

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture
def grid_cap():
    yield M.moe_set_gemm_max_blocks
    M.moe_set_gemm_max_blocks(0)


@pytest.mark.parametrize("case", list(GROUP_CASES))
@pytest.mark.parametrize("H,I", [(128, 256), (256, 192)])
def test_grouped_gemm_swiglu_scaled(case, H, I):
    counts = GROUP_CASES[case]
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    _say("scaled swiglu", case, H, I)
    rng = np.random.default_rng(15)
    xp = W.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    wgu = W.to_bf16_bits(rng.standard_normal((G, H, 2 * I)).astype(np.float32) * 0.05)
    ps = rng.uniform(0.01, 1.0, rows).astype(np.float32)
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    gu = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    h.view(torch.int16).fill_(0x7FC0)
    M.moe_grouped_gemm_swiglu_scaled(dev_bf16(xp), dev_bf16(wgu), dev(offs), dev(ps), h, gu)
    torch.cuda.synchronize()
    ref = O.expert_mlp(O.bf16_bits_to_f64(xp), wgu, np.zeros((G, I, 8)), offs, I, row_scale=ps)
    check_bf16(host_vals(h), ref["h"], "scaled h")
    check_bf16(host_vals(gu), O.to_bf16(np.concatenate([ref["g"], ref["u"]], 1)), "gu")


@pytest.mark.parametrize("I,cap,counts", [(192, 0, "ragged"), (192, 4, "ragged"), (256, 0, "tile_edges"),
                                          (128, 0, "decode")])
def test_grouped_gemm_swiglu_scaled_bwd(I, cap, counts, grid_cap):
    # a capped grid picks the wide 320x256 tiles, the uncapped one the narrow 320x128; a
    # decode-sized row count the 32-row tiles: every tiling has 64 columns per wave
    if cap:
        grid_cap(cap)
    cnt = [3, 0, 5, 1, 8, 2, 0, 4] if counts == "decode" else GROUP_CASES[counts]
    offs = _groups(cnt)
    rows, G = int(offs[-1]), len(cnt)
    H = 256
    _say("scaled swiglu bwd", I, cap, counts)
    rng = np.random.default_rng(18)
    d_out = W.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    wd = W.to_bf16_bits(rng.standard_normal((G, I, H)).astype(np.float32) * 0.05)
    gu = W.to_bf16_bits(rng.standard_normal((rows, 2 * I)).astype(np.float32))
    ps = rng.uniform(0.01, 1.0, rows).astype(np.float32)
    dgu = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    part = torch.full((rows, I // 64), float("nan"), device="cuda")
    M.moe_grouped_gemm_swiglu_scaled_bwd(dev_bf16(d_out), dev_bf16(wd), dev(offs), dev_bf16(gu),
                                         dev(ps), dgu, part)
    torch.cuda.synchronize()
    dov = O.bf16_bits_to_f64(d_out)
    dh = O.grouped_gemm(dov, np.swapaxes(wd, 1, 2), offs)
    g, u = O.bf16_bits_to_f64(gu[:, :I]), O.bf16_bits_to_f64(gu[:, I:])
    dg, du = O.swiglu_backward(dh * ps[:, None].astype(np.float64), g, u)
    check_bf16(host_vals(dgu), np.concatenate([dg, du], 1), "dgu (scaled)")
    hu = O.silu(g) * u
    ref = (dh * hu).sum(axis=1)
    got = host_vals(part).sum(axis=1)
    # dh carries the GEMM's fp32 error (H terms), then I products summed in fp32
    dh_b = H * U * O.grouped_gemm(np.abs(dov), np.abs(np.swapaxes(O.bf16_bits_to_f64(wd), 1, 2)), offs, exact=True)
    bound = (dh_b * np.abs(hu)).sum(axis=1) + (I + 16) * U * (np.abs(dh * hu)).sum(axis=1)
    check_close(got, ref, bound, "d_scale")


def test_permute_probs():
    rng = np.random.default_rng(3)
    T, E, k = 300, 16, 4
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    _, row_of, _ = O.dispatch_meta(idx, E)
    q = rng.uniform(size=(T, k)).astype(np.float32)
    rp = torch.full((T * k,), float("nan"), device="cuda")
    M.moe_permute_probs(dev(row_of), dev(q), rp)
    torch.cuda.synchronize()
    assert np.array_equal(rp.cpu().numpy(), O.row_weights(q, row_of, T * k).astype(np.float32))


LAYERS = {
    "qwen_like": W.custom("act_q", T=257, H=256, E=32, k=8, I=192, training=True),
    "post": W.custom("act_p", T=300, H=384, E=8, k=2, I=256, score=O.SOFTMAX_POST, training=True),
    "pre": W.custom("act_pre", T=200, H=256, E=16, k=4, I=128, score=O.SOFTMAX_PRE, training=True),
}


@pytest.mark.parametrize("router", [False, True])
@pytest.mark.parametrize("name", list(LAYERS))
def test_layer_scaled_swiglu(name, router):
    from test_gpu_router import _router_choice
    w = LAYERS[name]
    _say("layer, ScaledSwiGLU", name, "router", router)
    d = W.make_inputs(w)
    g = GpuMoE(w, d, router=router, placement=M.MOE_PLACE_ACTIVATION)
    y = host_vals(g.forward())
    if router:
        ref_logits, same, clean = _router_choice(w, d, g)
    else:
        ref_logits, same, clean = d["logits"], np.ones(w.T, bool), np.ones(w.E, bool)
    ref = O.moe_forward(d["x"], ref_logits, d["w_gu"], d["w_down"], w.k, w.score, w.I,
                        placement=O.PLACE_ACTIVATION)
    if same.all():
        ints = g.ints()
        for key in ("topk_idx", "offsets", "row_of"):
            assert np.array_equal(ints[key], ref[key]), key
        h = host_vals(g.view("h", (w.T * w.k, w.I), torch.bfloat16))
        check_bf16(h, ref["h"], f"{name} scaled h")
    S = np.nonzero(same)[0]
    check_bf16(y[S], ref["y"][S], f"{name} y", slack=combine_slack(ref["out"], ref["row_of"])[S])
    g.backward(d["dy"])
    rb = O.moe_backward(ref, d["dy"], d["w_gu"], d["w_down"], w.I,
                        w_router_bits=d["w_router"] if router else None)
    check_bf16(host_vals(g.dx)[S], rb["dx"][S], f"{name} dx",
               slack=combine_slack(rb["dxp"], ref["row_of"])[S])
    C = np.nonzero(clean)[0]
    check_bf16(host_vals(g.dw_gu)[C], rb["dw_gu"][C], f"{name} dw_gu")
    check_bf16(host_vals(g.dw_down)[C], rb["dw_down"][C], f"{name} dw_down")
    if router:
        dl = host_vals(g.view("d_logits", (w.T, w.E), torch.float32))
        for key, got, r in (("d_logits", dl[S], rb["d_logits"][S]),
                            ("dw_router", host_vals(g.dw_router)[C], rb["dw_router"][C])):
            rel = np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30)
            _say(f"{name} {key}: rel_l2={rel:.3e}")
            assert np.isfinite(got).all() and rel <= 1e-2, (key, rel)


def test_layer_scaled_swiglu_unit_weights_equal_combine_placement():
    # top-1, softmax after the top-k: every weight is 1, so both placements run the same
    # arithmetic and the device results are bit-identical
    w = W.custom("act_u", T=130, H=256, E=8, k=1, I=128, score=O.SOFTMAX_POST, training=True)
    d = W.make_inputs(w)
    out = {}
    for place in (M.MOE_PLACE_COMBINE, M.MOE_PLACE_ACTIVATION):
        g = GpuMoE(w, d, placement=place)
        y = host_vals(g.forward())
        g.backward(d["dy"])
        out[place] = (y, host_vals(g.dx), host_vals(g.dw_gu), host_vals(g.dw_down))
    for a, b, key in zip(out[M.MOE_PLACE_COMBINE], out[M.MOE_PLACE_ACTIVATION],
                         ("y", "dx", "dw_gu", "dw_down")):
        assert np.array_equal(a, b), key
