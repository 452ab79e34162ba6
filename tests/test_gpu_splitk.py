"""Split-K of the decode-sized grouped GEMMs (a few rows per expert on 32-row tiles): each
tile's reduction is cut into K parts on the device, the parts' fp32 sums go to a caller
space and a second launch adds them and applies the epilogue. Parity against the oracle,
against the unsplit launch, and the edges: uneven parts, ragged column tiles, empty
experts, rows past the last group left alone, the shared group and the routing weights of
the layer."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
import workloads as W
from gpu_helpers import GpuMoE, check_bf16, combine_slack, dev, dev_bf16, host_vals

pytestmark = pytest.mark.gpu

# a decode step: a handful of rows per expert, several experts empty
DCOUNTS = [3, 0, 1, 8, 2, 0, 5, 1, 0, 4, 2, 6, 0, 0, 1, 7]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _groups(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _space(rows, G, ncols):
    n = M.moe_grouped_gemm_splitk_workspace_bytes(rows, G, ncols)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # NaN partial sums wherever a part was not written
    return ws


def _parts(ws):
    return int(ws[:4].view(torch.int32).item())


@pytest.fixture
def grid_cap():
    yield M.moe_set_gemm_max_blocks
    M.moe_set_gemm_max_blocks(0)


# H = 1088, 768, 256: 34, 24 and 8 K stages of 32 (with 8 stages, only two parts of at
# least four); a grid of 5 blocks has no idle block, so the launch does not split
@pytest.mark.parametrize("H", [1088, 768, 256])
@pytest.mark.parametrize("cap", [0, 5])
def test_splitk_swiglu(H, cap, grid_cap):
    grid_cap(cap)
    counts = DCOUNTS
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    I = 320  # 2.5 tiles of 128 h columns: a ragged last column tile
    _say("split-K swiglu", H, cap)
    rng = np.random.default_rng(H + cap)
    x = W.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    wgu = W.to_bf16_bits(rng.standard_normal((G, H, 2 * I)).astype(np.float32) * 0.05)
    ws = _space(rows, G, 2 * I)
    h = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    gu = torch.full((rows, 2 * I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_swiglu(dev_bf16(x), dev_bf16(wgu), dev(offs), h, gu, ws=ws)
    h0 = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_swiglu(dev_bf16(x), dev_bf16(wgu), dev(offs), h0)  # unsplit
    torch.cuda.synchronize()
    S = _parts(ws)
    _say("parts", S)
    if cap == 0:
        assert 1 < S <= 8
    else:
        assert S == -1  # not offered a split: the space is left as it was
    r = O.expert_mlp(O.bf16_bits_to_f64(x), wgu, np.zeros((G, I, 8)), offs, I)
    check_bf16(host_vals(h), r["h"], f"split-K h H={H} cap={cap}")
    check_bf16(host_vals(gu), np.concatenate([r["g"], r["u"]], 1), f"split-K gu H={H} cap={cap}")
    # the unsplit launch: the same sums in another fp32 order
    check_bf16(host_vals(h), host_vals(h0), f"split vs unsplit H={H} cap={cap}", max_abs=2e-3, rel_l2=2e-3)


@pytest.mark.parametrize("mode", [M.MOE_GEMM_NN, M.MOE_GEMM_NT])
@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float32])
def test_splitk_store(mode, out_dt):
    counts = DCOUNTS
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    K, N = 1088, 320
    _say("split-K store", mode, out_dt)
    rng = np.random.default_rng(7 + mode)
    a = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((G, K, N)).astype(np.float32) * 0.05)
    bdev = dev_bf16(b) if mode == M.MOE_GEMM_NN else dev_bf16(np.ascontiguousarray(np.swapaxes(b, 1, 2)))
    ws = _space(rows, G, N)
    c = torch.full((rows, N), float("nan"), dtype=out_dt, device="cuda")
    M.moe_grouped_gemm(mode, dev_bf16(a), bdev, dev(offs), c, ws=ws)
    torch.cuda.synchronize()
    assert _parts(ws) > 1
    ref = O.grouped_gemm(O.bf16_bits_to_f64(a), b, offs)
    r = O.to_bf16(ref) if out_dt == torch.bfloat16 else ref
    check_bf16(host_vals(c), r, f"split-K store mode={mode} {out_dt}",
               max_abs=2e-2 if out_dt == torch.bfloat16 else 1e-3)


def test_splitk_rows_past_the_last_group_untouched():
    # offsets[G] < rows: the rows after the last group are not the GEMM's to write
    counts = [2, 0, 5, 1]
    offs = _groups(counts)
    rows, G = 12, len(counts)
    K, N = 768, 256
    rng = np.random.default_rng(3)
    a = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((G, K, N)).astype(np.float32) * 0.05)
    ws = _space(rows, G, N)
    c = torch.full((rows, N), 7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm(M.MOE_GEMM_NN, dev_bf16(a), dev_bf16(b), dev(offs), c, ws=ws)
    torch.cuda.synchronize()
    assert _parts(ws) > 1
    end = int(offs[-1])
    ref = O.grouped_gemm(O.bf16_bits_to_f64(a[:end]), b, offs)
    check_bf16(host_vals(c)[:end], O.to_bf16(ref), "split-K rows in groups")
    assert (host_vals(c)[end:] == 7.0).all()


def test_splitk_space_too_small_is_refused():
    offs = _groups(DCOUNTS)
    rows, G = int(offs[-1]), len(DCOUNTS)
    K, N = 256, 128
    a = torch.zeros((rows, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((G, K, N), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((rows, N), dtype=torch.bfloat16, device="cuda")
    n = M.moe_grouped_gemm_splitk_workspace_bytes(rows, G, N)
    ws = torch.empty(n - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        M.moe_grouped_gemm(M.MOE_GEMM_NN, a, b, dev(offs), c, ws=ws)


# decode-sized layers whose GEMMs split: a shared expert of the routed width (run as one
# more group), the routing weights on the SwiGLU output, and a training step (saved g, u)
DEC = {
    "dec_shared": W.custom("dec_shared", T=8, H=1024, E=16, k=1, I=512, score=O.SIGMOID,
                           shared_I=512, hot_experts=(0, 1, 2), hot_bias=2.0),
    "dec_k4": W.custom("dec_k4", T=12, H=1088, E=32, k=4, I=384, score=O.SOFTMAX_POST),
    "dec_train": W.custom("dec_train", T=16, H=768, E=16, k=2, I=256, training=True),
}


@pytest.mark.parametrize("name", list(DEC))
def test_layer_decode_split(name):
    w = DEC[name]
    _say("layer split-K", name)
    d = W.make_inputs(w)
    g = GpuMoE(w, d)
    y = host_vals(g.forward())
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I,
                        d.get("shared_gu"), d.get("shared_down"))
    slack = combine_slack(ref["out"], ref["row_of"], ref["topk_prob"], ref["shared"])
    check_bf16(y, ref["y"], f"{name} y", slack=slack)
    N = w.T * w.k
    check_bf16(host_vals(g.view("h", (N, w.I), torch.bfloat16)), ref["h"], f"{name} h")
    if w.training:
        g.backward(d["dy"])
        rb = O.moe_backward(ref, d["dy"], d["w_gu"], d["w_down"], w.I)
        check_bf16(host_vals(g.dx), rb["dx"], f"{name} dx", slack=combine_slack(rb["dxp"], ref["row_of"]))
        check_bf16(host_vals(g.dw_gu), rb["dw_gu"], f"{name} dw_gu")
        check_bf16(host_vals(g.dw_down), rb["dw_down"], f"{name} dw_down")


def test_layer_decode_split_scaled_swiglu():
    w = W.custom("dec_act", T=8, H=768, E=16, k=2, I=256, training=False)
    _say("layer split-K, ScaledSwiGLU")
    d = W.make_inputs(w)
    g = GpuMoE(w, d, placement=M.MOE_PLACE_ACTIVATION)
    y = host_vals(g.forward())
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I,
                        placement=O.PLACE_ACTIVATION)
    check_bf16(host_vals(g.view("h", (w.T * w.k, w.I), torch.bfloat16)), ref["h"], "dec_act h")
    check_bf16(y, ref["y"], "dec_act y", slack=combine_slack(ref["out"], ref["row_of"]))
