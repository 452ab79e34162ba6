"""GPU parity of the padded dispatch (moe_permute_padded and the layer with align_size)
against the oracle's padded layout, through the C ABI. Integer layout bit-exact; row
copies bit-exact, padding rows zero (fp8: scale 1); the layer's outputs against the
unpadded oracle (padding changes no arithmetic)."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
import workloads as W
from gpu_helpers import GpuMoE, check_bf16, check_fp8, combine_slack, dev, dev_bf16, host_vals

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_padded(x_bits, idx, E, align, fp8=False):
    T, H = x_bits.shape
    k = idx.shape[1]
    R = M.moe_padded_rows(T, E, k, align)
    xp = torch.full((R, H), 0x7F if fp8 else 0, dtype=torch.uint8 if fp8 else torch.bfloat16,
                    device="cuda")
    if not fp8:
        xp.view(torch.int16).fill_(0x7FC0)  # NaN canary
    scale = torch.full((R,), float("nan"), device="cuda") if fp8 else None
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    pad = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    row_of = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src_of = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.moe_permute_workspace_bytes(T, E, k), dtype=torch.uint8, device="cuda")
    M.moe_permute_padded(dev_bf16(x_bits), dev(idx), E, align, xp, offsets, pad, row_of, src_of,
                         ws, M.MOE_FP8_E4M3 if fp8 else M.MOE_BF16, scale)
    torch.cuda.synchronize()
    return xp, scale, offsets.cpu().numpy(), pad.cpu().numpy(), row_of.cpu().numpy(), src_of.cpu().numpy()


def _check_layout(idx, E, align, offsets, pad, row_of, src_of):
    r_off, r_pad, r_row, r_src = O.dispatch_meta_padded(idx, E, align)
    assert np.array_equal(offsets, r_off) and np.array_equal(pad, r_pad)
    assert np.array_equal(row_of, r_row)
    assert np.array_equal(src_of[:r_off[-1]], r_src)
    return r_off


@pytest.mark.parametrize("T,H,E,k,align", [(300, 256, 16, 4, 128), (97, 128, 10, 3, 8),
                                           (1, 64, 4, 2, 256), (1000, 512, 64, 2, 1)])
def test_permute_padded_bf16(T, H, E, k, align):
    _say("permute padded", T, H, E, k, align)
    rng = np.random.default_rng(T + align)
    x = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    xp, _, offsets, pad, row_of, src_of = _run_padded(x, idx, E, align)
    r_off = _check_layout(idx, E, align, offsets, pad, row_of, src_of)
    got = xp.view(torch.int16).cpu().numpy().view(np.uint16)[:r_off[-1]]
    want = np.zeros((r_off[-1], H), np.uint16)
    rows = src_of[:r_off[-1]]
    want[rows >= 0] = x[rows[rows >= 0]]
    assert np.array_equal(got, want)  # token rows bit copies, padding rows zero


def test_permute_padded_receive_buffer_example():
    # counts of 129 and 127 at alignment 128: 384 rows
    idx = np.array([[0]] * 129 + [[1]] * 127, dtype=np.int32)
    rng = np.random.default_rng(1)
    x = W.to_bf16_bits(rng.standard_normal((256, 64)).astype(np.float32))
    xp, _, offsets, pad, row_of, src_of = _run_padded(x, idx, 2, 128)
    assert offsets.tolist() == [0, 256, 384] and pad.tolist() == [0, 127]
    _check_layout(idx, 2, 128, offsets, pad, row_of, src_of)


def test_permute_padded_fp8():
    T, H, E, k, align = 200, 256, 8, 2, 64
    rng = np.random.default_rng(2)
    x = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    xp, scale, offsets, pad, row_of, src_of = _run_padded(x, idx, E, align, fp8=True)
    r_off = _check_layout(idx, E, align, offsets, pad, row_of, src_of)
    q, sc = O.quantize_rows_e4m3(O.as_values(x))
    rows = src_of[:r_off[-1]]
    gq, gs = xp.cpu().numpy()[:r_off[-1]], scale.cpu().numpy()[:r_off[-1]]
    assert np.array_equal(gq[rows >= 0], q[rows[rows >= 0]])
    assert np.array_equal(gs[rows >= 0], sc[rows[rows >= 0]])
    assert not gq[rows < 0].any() and (gs[rows < 0] == 1.0).all()


@pytest.mark.parametrize("align", [64, 256])
def test_layer_padded(align):
    w = W.custom("pad", T=257, H=256, E=32, k=8, I=192, training=True)
    _say("layer padded", align)
    d = W.make_inputs(w)
    g = GpuMoE(w, d)
    g.prob.align_size = align
    # the workspace grows by the padding capacity
    g.ws = torch.empty(M.moe_workspace_bytes(g.prob), dtype=torch.uint8, device="cuda")
    g.ws.fill_(0xFF)
    g.views = M.moe_workspace_views(g.prob, g.ws)
    assert g.views.rows == w.T * w.k + w.E * (align - 1)
    y = host_vals(g.forward())
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I)
    r_off, r_pad, r_row, _ = O.dispatch_meta_padded(ref["topk_idx"], w.E, align)
    offs = g.view("offsets", (w.E + 1,), torch.int32).cpu().numpy()
    assert np.array_equal(offs, r_off)
    assert np.array_equal(g.view("pad_offsets", (w.E,), torch.int32).cpu().numpy(), r_pad)
    assert np.array_equal(g.view("row_of", (w.T, w.k), torch.int32).cpu().numpy(), r_row)
    slack = combine_slack(ref["out"], ref["row_of"], ref["topk_prob"])
    check_bf16(y, ref["y"], f"padded{align} y", slack=slack)
    g.backward(d["dy"])
    rb = O.moe_backward(ref, d["dy"], d["w_gu"], d["w_down"], w.I)
    check_bf16(host_vals(g.dx), rb["dx"], f"padded{align} dx", slack=combine_slack(rb["dxp"], ref["row_of"]))
    check_bf16(host_vals(g.dw_gu), rb["dw_gu"], f"padded{align} dw_gu")
    check_bf16(host_vals(g.dw_down), rb["dw_down"], f"padded{align} dw_down")


def test_layer_padded_fp8_forward():
    w = W.custom("pad8", T=300, H=256, E=32, k=8, I=256, fp8=True, zipf_s=1.2, n_empty=5)
    _say("layer padded fp8")
    d = W.make_inputs(w)
    g = GpuMoE(w, d)
    g.prob.align_size = 128
    g.ws = torch.empty(M.moe_workspace_bytes(g.prob), dtype=torch.uint8, device="cuda")
    g.ws.fill_(0xFF)
    g.views = M.moe_workspace_views(g.prob, g.ws)
    y = host_vals(g.forward())
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I, fp8=True)
    check_fp8(y, ref["y"], "padded fp8 y")
