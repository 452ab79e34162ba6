"""GPU parity of every C-ABI entry point against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails (plus edge cases)."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
import workloads as W
from gpu_helpers import (GpuMoE, check_bf16, check_fp8, combine_slack, dev, dev_bf16, host_bits,
                         host_vals)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---- router ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_router_full_size(name):
    w = W.WORKLOADS[name]
    _say("router", name)
    l = W.make_logits(w)
    T, E, k = l.shape[0], w.E, w.k
    ti = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tp = torch.empty((T, k), dtype=torch.float32, device="cuda")
    cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    rm = torch.full((T, E), 9, dtype=torch.uint8, device="cuda")
    pd = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_router_topk(dev(l), k, w.score, ti, tp, cnt, rm, pd)
    torch.cuda.synchronize()
    idx, q, counts, rmap, dense = O.router_topk(l, k, w.score)
    assert np.array_equal(ti.cpu().numpy(), idx)
    assert np.array_equal(cnt.cpu().numpy(), counts)
    assert np.array_equal(rm.cpu().numpy(), rmap)
    got_q = tp.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_q - q) <= 1e-6 * np.abs(q)), np.max(np.abs(got_q - q) / q)
    got_d = pd.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_d - dense) <= 1e-6 * np.abs(dense))


def test_router_ties_and_k_limits():
    rng = np.random.default_rng(0)
    for (T, E, k, score) in [(100, 32, 32, 0), (77, 256, 8, 1), (5, 3, 3, 2), (64, 200, 17, 0),
                             (50, 64, 16, 0), (33, 16, 1, 2), (19, 129, 16, 1)]:
        l = rng.integers(-3, 3, (T, E)).astype(np.float32)   # many exact ties
        ti = torch.empty((T, k), dtype=torch.int32, device="cuda")
        tp = torch.empty((T, k), dtype=torch.float32, device="cuda")
        cnt = torch.empty((E,), dtype=torch.int32, device="cuda")
        M.moe_router_topk(dev(l), k, score, ti, tp, cnt)
        torch.cuda.synchronize()
        idx, q, counts, _, _ = O.router_topk(l, k, score)
        assert np.array_equal(ti.cpu().numpy(), idx), (T, E, k)
        assert np.array_equal(cnt.cpu().numpy(), counts)
        assert np.allclose(tp.cpu().numpy(), q, rtol=1e-6, atol=0)


# ---- dispatch / combine ------------------------------------------------------------------

def _permute_gpu(x_bits, idx, E, fp8=False):
    T, k = idx.shape
    H = x_bits.shape[1]
    x = dev_bf16(x_bits)
    xp = torch.empty((T * k, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    xs = torch.empty((T * k,), dtype=torch.float32, device="cuda") if fp8 else None
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    row_of = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src_of = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(M.moe_permute_workspace_bytes(T, E, k), 16), dtype=torch.uint8, device="cuda")
    M.moe_permute(x, dev(idx.astype(np.int32)), E, xp, offs, row_of, src_of, ws,
                  M.MOE_FP8_E4M3 if fp8 else M.MOE_BF16, xs)
    torch.cuda.synchronize()
    return xp, xs, offs.cpu().numpy(), row_of.cpu().numpy(), src_of.cpu().numpy()


@pytest.mark.parametrize("T,H,E,k", [(64, 128, 4, 2), (1000, 256, 128, 8), (3000, 64, 16, 1),
                                     (1, 64, 8, 2), (2049, 128, 256, 5)])
def test_permute_bit_exact(T, H, E, k):
    _say("permute", T, H, E, k)
    rng = np.random.default_rng(T + E)
    x_bits = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    xp, _, offs, row_of, src_of = _permute_gpu(x_bits, idx, E)
    r_offs, r_row, r_src = O.dispatch_meta(idx, E)
    assert np.array_equal(offs, r_offs)
    assert np.array_equal(row_of, r_row)
    assert np.array_equal(src_of, r_src)
    assert np.array_equal(host_bits(xp), O.permute(x_bits, r_src))


def test_permute_all_to_one_expert_and_empty_experts():
    T, H, E, k = 1500, 64, 64, 2
    rng = np.random.default_rng(1)
    x_bits = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = np.tile(np.array([[5, 63]], np.int32), (T, 1))
    xp, _, offs, row_of, src_of = _permute_gpu(x_bits, idx, E)
    r_offs, r_row, r_src = O.dispatch_meta(idx, E)
    assert np.array_equal(offs, r_offs) and np.array_equal(row_of, r_row)
    assert np.array_equal(src_of, r_src)
    assert np.array_equal(host_bits(xp), O.permute(x_bits, r_src))


@pytest.mark.parametrize("C", [64, 512, 768, 2048, 4096, 8192])
def test_quantize_rows_bit_exact(C):
    # every register-resident width (1, 2, 4, 8 vectors per lane) and the wide-row path,
    # a row count that is not a multiple of the four rows per block, an all-zero row and
    # rows with widely different ranges
    R = 37
    rng = np.random.default_rng(C)
    xv = rng.standard_normal((R, C)).astype(np.float32) * rng.uniform(1e-3, 300, (R, 1)).astype(np.float32)
    xv[5] = 0.0
    xv[11, C // 3] = 1e4
    x_bits = W.to_bf16_bits(xv)
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sc = torch.empty((R,), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_rows(dev_bf16(x_bits), q, sc)
    torch.cuda.synchronize()
    rq, rs = O.quantize_rows_e4m3(O.bf16_bits_to_f64(x_bits))
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sc.cpu().numpy(), rs)


def test_permute_fp8_codes_and_scales_bit_exact():
    T, H, E, k = 300, 256, 16, 4
    rng = np.random.default_rng(2)
    xv = rng.standard_normal((T, H)).astype(np.float32) * rng.uniform(1e-3, 30, (T, 1)).astype(np.float32)
    xv[7] = 0.0
    x_bits = W.to_bf16_bits(xv)
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    xp, xs, offs, row_of, src_of = _permute_gpu(x_bits, idx, E, fp8=True)
    q, s = O.quantize_rows_e4m3(O.bf16_bits_to_f64(x_bits))
    assert np.array_equal(xp.cpu().numpy(), q[src_of])
    assert np.array_equal(xs.cpu().numpy(), s[src_of])


@pytest.mark.parametrize("k", [1, 2, 8])
def test_identity_experts_give_k_x(k):
    # dispatch -> combine with unit weights and identity experts returns k * x exactly
    T, H, E = 500, 256, 32
    rng = np.random.default_rng(k)
    x_bits = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    xp, _, offs, row_of, src_of = _permute_gpu(x_bits, idx, E)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ones = torch.ones((T, k), dtype=torch.float32, device="cuda")
    M.moe_unpermute_combine(xp, dev(row_of), ones, y)
    torch.cuda.synchronize()
    assert np.array_equal(host_vals(y), k * O.bf16_bits_to_f64(x_bits))


@pytest.mark.parametrize("shared", [False, True])
def test_combine_matches_oracle(shared):
    T, H, E, k = 700, 512, 16, 4
    rng = np.random.default_rng(3)
    idx, q, *_ = O.router_topk(rng.standard_normal((T, E)).astype(np.float32), k, 0)
    _, row_of, _ = O.dispatch_meta(idx, E)
    out_bits = W.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32) * 3)
    sh_bits = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)) if shared else None
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    M.moe_unpermute_combine(dev_bf16(out_bits), dev(row_of), dev(q.astype(np.float32)), y,
                            dev_bf16(sh_bits) if shared else None)
    torch.cuda.synchronize()
    ref = O.combine(O.bf16_bits_to_f64(out_bits), row_of, q,
                    O.bf16_bits_to_f64(sh_bits) if shared else None)
    check_bf16(host_vals(y), ref, "combine")
    # unweighted form (dispatch backward)
    M.moe_unpermute_combine(dev_bf16(out_bits), dev(row_of), None, y)
    torch.cuda.synchronize()
    check_bf16(host_vals(y), O.combine(O.bf16_bits_to_f64(out_bits), row_of, None), "combine_unweighted")


def test_combine_backward_bit_exact():
    T, H, E, k = 400, 128, 8, 2
    rng = np.random.default_rng(4)
    idx, q, *_ = O.router_topk(rng.standard_normal((T, E)).astype(np.float32), k, 0)
    _, row_of, _ = O.dispatch_meta(idx, E)
    dy_bits = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    d_out = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    M.moe_combine_backward(dev_bf16(dy_bits), dev(row_of), dev(q.astype(np.float32)), d_out)
    torch.cuda.synchronize()
    ref = np.zeros((T * k, H))
    dy = O.bf16_bits_to_f64(dy_bits)
    for j in range(k):
        ref[row_of[:, j]] = O.to_bf16(dy * q[:, j:j + 1])
    assert np.array_equal(host_vals(d_out), ref)


# ---- grouped GEMMs --------------------------------------------------------------------------

def _groups(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


GROUP_CASES = {
    "ragged": [130, 0, 1, 255, 64, 300, 0, 17],
    "single": [513],
    "empty_heavy": [0, 0, 0, 200, 0, 0, 1, 0, 0, 0],
    # around the largest M tile (320 rows) and its even splits
    "tile_edges": [320, 321, 641, 32, 0, 319, 960],
}


@pytest.mark.parametrize("case", list(GROUP_CASES))
@pytest.mark.parametrize("H,I", [(128, 256), (256, 192)])
def test_grouped_gemm_swiglu_bf16(case, H, I):
    counts = GROUP_CASES[case]
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    _say("gg_swiglu", case, H, I)
    rng = np.random.default_rng(5)
    xp = W.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    wgu = W.to_bf16_bits(rng.standard_normal((G, H, 2 * I)).astype(np.float32) * 0.05)
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    gu = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    h.view(torch.int16).fill_(0x7FC0)
    M.moe_grouped_gemm_swiglu(dev_bf16(xp), dev_bf16(wgu), dev(offs), h, gu)
    torch.cuda.synchronize()
    ref = O.expert_mlp(O.bf16_bits_to_f64(xp), wgu, np.zeros((G, I, 8)), offs, I)
    check_bf16(host_vals(h), ref["h"], "h")
    check_bf16(host_vals(gu), O.to_bf16(np.concatenate([ref["g"], ref["u"]], 1)), "gu")


@pytest.mark.parametrize("case", list(GROUP_CASES))
@pytest.mark.parametrize("mode", [M.MOE_GEMM_NN, M.MOE_GEMM_NT])
def test_grouped_gemm_nn_nt(case, mode):
    counts = GROUP_CASES[case]
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    K, N = 192, 320
    _say("gg", case, mode)
    rng = np.random.default_rng(6)
    a = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((G, K, N)).astype(np.float32) * 0.05)
    bdev = dev_bf16(b) if mode == M.MOE_GEMM_NN else dev_bf16(np.ascontiguousarray(np.swapaxes(b, 1, 2)))
    for out_dt in (torch.bfloat16, torch.float32):
        c = torch.full((rows, N), float("nan"), dtype=out_dt, device="cuda")
        M.moe_grouped_gemm(mode, dev_bf16(a), bdev, dev(offs), c)
        torch.cuda.synchronize()
        ref = O.grouped_gemm(O.bf16_bits_to_f64(a), b, offs)
        if out_dt == torch.bfloat16:
            ref = O.to_bf16(ref)
        check_bf16(host_vals(c), ref, f"gemm mode={mode} {out_dt}", max_abs=2e-2 if out_dt == torch.bfloat16 else 1e-3)


@pytest.mark.parametrize("case", list(GROUP_CASES))
def test_grouped_gemm_dw(case):
    counts = GROUP_CASES[case]
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    Mdim, N = 192, 256
    _say("gg_dw", case)
    rng = np.random.default_rng(7)
    a = W.to_bf16_bits(rng.standard_normal((rows, Mdim)).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((rows, N)).astype(np.float32) * 0.1)
    c = torch.full((G, Mdim, N), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_grouped_gemm(M.MOE_GEMM_TN_DW, dev_bf16(a), dev_bf16(b), dev(offs), c)
    torch.cuda.synchronize()
    ref = O.grouped_gemm_dw(O.bf16_bits_to_f64(a), O.bf16_bits_to_f64(b), offs)
    check_bf16(host_vals(c), ref, "dw fp32", max_abs=1e-3)
    for g in range(G):
        if counts[g] == 0:
            assert not host_vals(c[g]).any()


@pytest.mark.parametrize("I,cap", [(128, 0), (576, 4)])
def test_grouped_gemm_swiglu_bwd(I, cap, grid_cap):
    # a capped grid makes the launcher pick the wide (320x256) tiles: few blocks, many tiles
    grid_cap(cap)
    counts = GROUP_CASES["ragged"]
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    H = 256
    rng = np.random.default_rng(8)
    d_out = W.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    wd = W.to_bf16_bits(rng.standard_normal((G, I, H)).astype(np.float32) * 0.05)
    gu = W.to_bf16_bits(rng.standard_normal((rows, 2 * I)).astype(np.float32))
    dgu = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_swiglu_bwd(dev_bf16(d_out), dev_bf16(wd), dev(offs), dev_bf16(gu), dgu)
    torch.cuda.synchronize()
    dh = O.grouped_gemm(O.bf16_bits_to_f64(d_out), np.swapaxes(wd, 1, 2), offs)
    g, u = O.bf16_bits_to_f64(gu[:, :I]), O.bf16_bits_to_f64(gu[:, I:])
    dg, du = O.swiglu_backward(dh, g, u)
    check_bf16(host_vals(dgu), np.concatenate([dg, du], 1), "dgu")


# ---- persistent grid: many tiles per block -------------------------------------------------
# With the grid capped, every block walks a long run of tiles: bf16 epilogues overlap the
# next tile's loads (their stores counted in the wait), fp32 / SwiGLU-backward / fp8
# epilogues drain between tiles, and weight-gradient tiles of empty experts have no stages.

STREAM_COUNTS = [300, 0, 257, 1, 511, 0, 0, 64, 700, 33, 0, 256, 255, 129, 0, 400]


@pytest.fixture
def grid_cap():
    yield M.moe_set_gemm_max_blocks
    M.moe_set_gemm_max_blocks(0)


@pytest.mark.parametrize("cap", [1, 3, 16])
def test_gemm_many_tiles_per_block(cap, grid_cap):
    grid_cap(cap)
    counts = STREAM_COUNTS
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    K, N, I = 192, 320, 192
    _say("stream", cap)
    rng = np.random.default_rng(20 + cap)
    a = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    av = O.bf16_bits_to_f64(a)
    b = W.to_bf16_bits(rng.standard_normal((G, K, N)).astype(np.float32) * 0.05)
    ref = O.grouped_gemm(av, b, offs)
    for mode in (M.MOE_GEMM_NN, M.MOE_GEMM_NT):
        bdev = dev_bf16(b) if mode == M.MOE_GEMM_NN else dev_bf16(np.ascontiguousarray(np.swapaxes(b, 1, 2)))
        for out_dt in (torch.bfloat16, torch.float32):
            c = torch.full((rows, N), float("nan"), dtype=out_dt, device="cuda")
            M.moe_grouped_gemm(mode, dev_bf16(a), bdev, dev(offs), c)
            torch.cuda.synchronize()
            r = O.to_bf16(ref) if out_dt == torch.bfloat16 else ref
            check_bf16(host_vals(c), r, f"stream cap={cap} mode={mode} {out_dt}",
                       max_abs=2e-2 if out_dt == torch.bfloat16 else 1e-3)

    # SwiGLU with and without the saved g,u (two epilogue store counts)
    wgu = W.to_bf16_bits(rng.standard_normal((G, K, 2 * I)).astype(np.float32) * 0.05)
    h1 = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    gu = torch.full((rows, 2 * I), float("nan"), dtype=torch.bfloat16, device="cuda")
    h2 = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_swiglu(dev_bf16(a), dev_bf16(wgu), dev(offs), h1, gu)
    M.moe_grouped_gemm_swiglu(dev_bf16(a), dev_bf16(wgu), dev(offs), h2, None)
    torch.cuda.synchronize()
    r = O.expert_mlp(av, wgu, np.zeros((G, I, 8)), offs, I)
    check_bf16(host_vals(h1), r["h"], f"stream cap={cap} swiglu h")
    check_bf16(host_vals(gu), np.concatenate([r["g"], r["u"]], 1), f"stream cap={cap} swiglu gu")
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))

    # SwiGLU backward: dh = d_out W_down^T, then the gate/up gradients
    d_out = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    wd = W.to_bf16_bits(rng.standard_normal((G, I, K)).astype(np.float32) * 0.05)
    gub = host_bits(gu)
    dgu = torch.full((rows, 2 * I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_swiglu_bwd(dev_bf16(d_out), dev_bf16(wd), dev(offs), dev_bf16(gub), dgu)
    torch.cuda.synchronize()
    dh = O.grouped_gemm(O.bf16_bits_to_f64(d_out), np.swapaxes(wd, 1, 2), offs)
    dg, du = O.swiglu_backward(dh, O.bf16_bits_to_f64(gub[:, :I]), O.bf16_bits_to_f64(gub[:, I:]))
    check_bf16(host_vals(dgu), np.concatenate([dg, du], 1), f"stream cap={cap} swiglu bwd")

    # weight gradient, bf16 and fp32 output; empty experts get zero tiles
    Md, Nd = 192, 256
    wa = W.to_bf16_bits(rng.standard_normal((rows, Md)).astype(np.float32))
    wb = W.to_bf16_bits(rng.standard_normal((rows, Nd)).astype(np.float32) * 0.1)
    dref = O.grouped_gemm_dw(O.bf16_bits_to_f64(wa), O.bf16_bits_to_f64(wb), offs)
    for out_dt in (torch.bfloat16, torch.float32):
        c = torch.full((G, Md, Nd), float("nan"), dtype=out_dt, device="cuda")
        M.moe_grouped_gemm(M.MOE_GEMM_TN_DW, dev_bf16(wa), dev_bf16(wb), dev(offs), c)
        torch.cuda.synchronize()
        r = O.to_bf16(dref) if out_dt == torch.bfloat16 else dref
        check_bf16(host_vals(c), r, f"stream cap={cap} dw {out_dt}",
                   max_abs=2e-2 if out_dt == torch.bfloat16 else 1e-3)
        for g in range(G):
            if counts[g] == 0:
                assert not host_vals(c[g]).any()


@pytest.mark.parametrize("cap", [1, 5])
def test_gemm_fp8_and_small_m_many_tiles(cap, grid_cap):
    grid_cap(cap)
    _say("stream fp8/small-M", cap)
    rng = np.random.default_rng(40 + cap)
    counts = STREAM_COUNTS
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    K, N = 256, 384
    a_bits = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    b_bits = W.to_bf16_bits(rng.standard_normal((G, K, N)).astype(np.float32) * 0.02)
    aq = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    as_ = torch.empty((rows,), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_rows(dev_bf16(a_bits), aq, as_)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_weights(dev_bf16(b_bits), bq, bs)
    c = torch.full((rows, N), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_grouped_gemm(M.MOE_GEMM_NT, aq, bq, dev(offs), c, M.MOE_FP8_E4M3, as_, bs)
    torch.cuda.synchronize()
    qa, sa = O.quantize_rows_e4m3(O.bf16_bits_to_f64(a_bits))
    ref = O.grouped_gemm(O.e4m3_decode(qa), b_bits, offs, False, sa, quantize_b=True)
    check_bf16(host_vals(c), ref, f"stream cap={cap} fp8", max_abs=1e-3, rel_l2=1e-4)

    # decode shape: a few rows per expert take the small-M tiles
    dcounts = [3, 0, 1, 8, 2, 0, 5, 1, 0, 4, 2, 6]
    doffs = _groups(dcounts)
    drows, dG = int(doffs[-1]), len(dcounts)
    Hd, Id = 256, 320
    x = W.to_bf16_bits(rng.standard_normal((drows, Hd)).astype(np.float32))
    wgu = W.to_bf16_bits(rng.standard_normal((dG, Hd, 2 * Id)).astype(np.float32) * 0.05)
    h = torch.full((drows, Id), float("nan"), dtype=torch.bfloat16, device="cuda")
    gu = torch.full((drows, 2 * Id), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_swiglu(dev_bf16(x), dev_bf16(wgu), dev(doffs), h, gu)
    torch.cuda.synchronize()
    r = O.expert_mlp(O.bf16_bits_to_f64(x), wgu, np.zeros((dG, Id, 8)), doffs, Id)
    check_bf16(host_vals(h), r["h"], f"stream cap={cap} small-M swiglu h")
    check_bf16(host_vals(gu), np.concatenate([r["g"], r["u"]], 1), f"stream cap={cap} small-M gu")


def test_quantize_weights_bit_exact():
    rng = np.random.default_rng(9)
    G, K, N = 3, 320, 192
    wv = rng.standard_normal((G, K, N)).astype(np.float32) * 0.02
    wv[1, :, 5] = 0.0
    w_bits = W.to_bf16_bits(wv)
    q = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((G, N), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_weights(dev_bf16(w_bits), q, s)
    torch.cuda.synchronize()
    rq, rs = O.quantize_cols_e4m3(O.bf16_bits_to_f64(w_bits))
    assert np.array_equal(q.cpu().numpy(), np.swapaxes(rq, 1, 2))
    assert np.array_equal(s.cpu().numpy(), rs)


def test_grouped_gemm_fp8():
    counts = [130, 0, 1, 255, 64]
    offs = _groups(counts)
    rows, G = int(offs[-1]), len(counts)
    K, N = 256, 384
    rng = np.random.default_rng(10)
    a_bits = W.to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    b_bits = W.to_bf16_bits(rng.standard_normal((G, K, N)).astype(np.float32) * 0.02)
    aq = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    as_ = torch.empty((rows,), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_rows(dev_bf16(a_bits), aq, as_)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_weights(dev_bf16(b_bits), bq, bs)
    c = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    M.moe_grouped_gemm(M.MOE_GEMM_NT, aq, bq, dev(offs), c, M.MOE_FP8_E4M3, as_, bs)
    torch.cuda.synchronize()
    qa, sa = O.quantize_rows_e4m3(O.bf16_bits_to_f64(a_bits))
    assert np.array_equal(aq.cpu().numpy(), qa) and np.array_equal(as_.cpu().numpy(), sa)
    ref = O.grouped_gemm(O.e4m3_decode(qa), b_bits, offs, False, sa, quantize_b=True)
    # same quantised operands; only the matrix-core accumulation order differs
    check_bf16(host_vals(c), ref, "fp8 gemm", max_abs=1e-3, rel_l2=1e-4)


# ---- whole layer -----------------------------------------------------------------------------

SMALL = {
    "tiny": W.WORKLOADS["tiny"],
    "small_post": W.custom("small_post", T=333, H=256, E=8, k=2, I=384, score=O.SOFTMAX_POST),
    "small_sig_shared": W.custom("small_sig_shared", T=8, H=320, E=16, k=1, I=256, score=O.SIGMOID,
                                 shared_I=192, hot_experts=(0, 1, 2), hot_bias=2.0),
    # shared expert as wide as the routed ones: it runs as one more group of the routed
    # launches (decode-sized tiles, then several 320-row tiles with a ragged last one)
    "small_shared_eq": W.custom("small_shared_eq", T=8, H=320, E=16, k=1, I=256, score=O.SIGMOID,
                                shared_I=256, hot_experts=(0, 1, 2), hot_bias=2.0),
    "mid_shared_eq": W.custom("mid_shared_eq", T=700, H=384, E=8, k=2, I=320, score=O.SOFTMAX_POST,
                              shared_I=320),
    "small_qwen": W.custom("small_qwen", T=257, H=256, E=32, k=8, I=192, training=True),
    "small_fp8": W.custom("small_fp8", T=300, H=256, E=32, k=8, I=256, fp8=True, zipf_s=1.2, n_empty=5),
    "t1": W.custom("t1", T=1, H=128, E=8, k=2, I=128, training=True),
    # decode-sized steps (at most 32 tokens and 256 choices, k <= 16) route, dispatch and
    # copy rows in one launch: its limits, E not a multiple of 16, each plain score
    "dec_256": W.custom("dec_256", T=32, H=128, E=256, k=8, I=128, score=O.SOFTMAX_POST),
    "dec_k16": W.custom("dec_k16", T=16, H=256, E=64, k=16, I=128, score=O.SOFTMAX_PRE),
    "dec_e100": W.custom("dec_e100", T=5, H=192, E=100, k=3, I=128, score=O.SIGMOID),
    "dec_renorm": W.custom("dec_renorm", T=31, H=128, E=40, k=6, I=128, training=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity_small(name):
    w = SMALL[name]
    _say("forward", name)
    d = W.make_inputs(w)
    g = GpuMoE(w, d)
    y = g.forward()
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I,
                        d.get("shared_gu"), d.get("shared_down"), fp8=w.fp8)
    ints = g.ints()
    for key in ("topk_idx", "counts", "offsets", "row_of", "src_of"):
        assert np.array_equal(ints[key], ref[key]), key
    assert np.allclose(ints["topk_prob"], ref["topk_prob"], rtol=1e-6, atol=0)
    if w.fp8:
        check_fp8(host_vals(y), ref["y"], f"{name} y")
    else:
        slack = combine_slack(ref["out"], ref["row_of"], ref["topk_prob"], ref["shared"])
        check_bf16(host_vals(y), ref["y"], f"{name} y", slack=slack)
        N = w.T * w.k
        check_bf16(host_vals(g.view("h", (N, w.I), torch.bfloat16)), ref["h"], f"{name} h")


@pytest.mark.parametrize("name", ["dec_256", "dec_k16", "dec_e100", "dec_renorm", "small_shared_eq"])
def test_decode_step_rows_copied(name):
    # the expert-contiguous rows of a decode-sized step: xp[r] = x[src_of[r]] bit for bit
    w = SMALL[name]
    _say("decode rows", name)
    d = W.make_inputs(w)
    g = GpuMoE(w, d)
    g.forward()
    src = g.ints()["src_of"]
    xp = g.view("xp", (w.T * w.k, w.H), torch.bfloat16).view(torch.int16).cpu().numpy()
    x = np.asarray(d["x"]).view(np.int16).reshape(w.T, w.H)
    assert np.array_equal(xp, x[src])


@pytest.mark.parametrize("name", ["small_qwen", "t1", "dec_renorm"])
def test_backward_parity_small(name):
    w = SMALL[name]
    _say("backward", name)
    d = W.make_inputs(w)
    g = GpuMoE(w, d)
    g.forward()
    g.backward(d["dy"])
    ref = O.moe_forward(d["x"], d["logits"], d["w_gu"], d["w_down"], w.k, w.score, w.I)
    rb = O.moe_backward(ref, d["dy"], d["w_gu"], d["w_down"], w.I)
    check_bf16(host_vals(g.dx), rb["dx"], f"{name} dx", slack=combine_slack(rb["dxp"], ref["row_of"]))
    check_bf16(host_vals(g.dw_gu), rb["dw_gu"], f"{name} dw_gu")
    check_bf16(host_vals(g.dw_down), rb["dw_down"], f"{name} dw_down")


def test_forward_row_permutation_invariance():
    # shuffling the tokens shuffles the outputs bit-exactly: a row's result does not
    # depend on which other rows share the call
    w = SMALL["small_post"]
    d = W.make_inputs(w)
    perm = np.random.default_rng(0).permutation(w.T)
    y0 = host_bits(GpuMoE(w, d).forward())
    d2 = dict(d)
    d2["x"], d2["logits"] = d["x"][perm], d["logits"][perm]
    y1 = host_bits(GpuMoE(w, d2).forward())
    assert np.array_equal(y0[perm], y1)


def test_invalid_arguments_return_status():
    lib = M.lib()
    x = torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")
    # k > E, H not a multiple of 64, null pointers: refused before any launch
    assert lib.moe_router_topk(x.data_ptr(), 64, 4, 5, 0, x.data_ptr(), x.data_ptr(), x.data_ptr(),
                               None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(x.data_ptr(), x.data_ptr(), None, None, 8, 100, 2,
                                     x.data_ptr(), None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute(None, None, 8, 128, 4, 2, 0, None, None, x.data_ptr(), None, None,
                           None, 0, None) == M.MOE_ERR_INVALID_ARG
    with pytest.raises(M.MoeError):
        M.moe_forward(M.problem(8, 128, 4, 2, 128, 0), M.tensors(x, None, x, x, x), x.view(torch.uint8))


def test_zero_tokens_is_a_no_op():
    # T = 0: the stand-alone calls write only what has a size (the router's counts, the
    # dispatch offsets: all zero), the layer forward does nothing, and the layer backward
    # writes zero weight gradients (every expert is empty)
    _say("zero tokens")
    H, E, k, I = 128, 8, 2, 128
    cuda = dict(device="cuda")
    logits = torch.empty((0, E), **cuda)
    idx = torch.empty((0, k), dtype=torch.int32, **cuda)
    prob = torch.empty((0, k), **cuda)
    counts = torch.full((E,), -1, dtype=torch.int32, **cuda)
    M.moe_router_topk(logits, k, O.SOFTMAX_PRE_RENORM, idx, prob, counts)
    x = torch.empty((0, H), dtype=torch.bfloat16, **cuda)
    xp = torch.empty((0, H), dtype=torch.bfloat16, **cuda)
    offs = torch.full((E + 1,), -1, dtype=torch.int32, **cuda)
    row_of = torch.empty((0, k), dtype=torch.int32, **cuda)
    src_of = torch.empty((0,), dtype=torch.int32, **cuda)
    ws = torch.empty(M.moe_permute_workspace_bytes(0, E, k), dtype=torch.uint8, **cuda)
    M.moe_permute(x, idx, E, xp, offs, row_of, src_of, ws)
    y = torch.empty((0, H), dtype=torch.bfloat16, **cuda)
    M.moe_unpermute_combine(xp, row_of, prob, y)
    torch.cuda.synchronize()
    assert (counts == 0).all() and (offs == 0).all()

    rng = np.random.default_rng(0)
    wgu = dev_bf16(O.f32_to_bf16_bits(0.02 * rng.standard_normal((E, H, 2 * I)).astype(np.float32)))
    wd = dev_bf16(O.f32_to_bf16_bits(0.02 * rng.standard_normal((E, I, H)).astype(np.float32)))
    prob_l = M.problem(0, H, E, k, I, O.SOFTMAX_PRE_RENORM, training=True)
    lws = torch.zeros(M.moe_workspace_bytes(prob_l), dtype=torch.uint8, **cuda)
    tens = M.tensors(x, logits, wgu, wd, y)
    M.moe_forward(prob_l, tens, lws)
    dwgu = torch.full_like(wgu, float("nan"))
    dwd = torch.full_like(wd, float("nan"))
    M.moe_backward(prob_l, tens, y, torch.empty_like(x), dwgu, dwd, lws)
    torch.cuda.synchronize()
    assert (dwgu == 0).all() and (dwd == 0).all()
