"""Helpers of the GPU parity tests: upload/download and the tolerance rules.

Float tolerances (bf16 outputs, fp32 accumulation): rel-L2 <= 1e-2 and max-abs <= 2e-2;
an element whose error exceeds 2e-2 is still accepted when it is within one bf16 ulp of
the reference plus one bf16 ulp of every rounded intermediate that feeds it (the
``slack`` argument): two correct fp32 accumulation orders can straddle a bf16 rounding
boundary, one bf16 ulp exceeds 2e-2 from magnitude 4 on, and a combine output sums k
expert rows that were each rounded to bf16. fp8 outputs: rel-L2 <= 5e-2 against the
quantised oracle. Integer outputs: bit-exact.
"""
import numpy as np
import torch

import mixture_experts_layer_amd as M
import oracle as O


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_vals(t):
    """bf16 / fp32 device tensor -> float64 numpy values."""
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(host_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_ulp(ref):
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def combine_slack(out_vals, row_of, prob=None, shared_vals=None):
    """One bf16 ulp of each rounded row a combine output sums: sum_j |p_j| ulp(out_j)
    (+ ulp(shared))."""
    out_vals = np.asarray(out_vals, np.float64)
    T, k = row_of.shape
    s = np.zeros((T, out_vals.shape[1]))
    for j in range(k):
        u = bf16_ulp(out_vals[np.asarray(row_of[:, j], np.int64)])
        s += u * (np.abs(np.asarray(prob, np.float64)[:, j:j + 1]) if prob is not None else 1.0)
    if shared_vals is not None:
        s += bf16_ulp(np.asarray(shared_vals, np.float64))
    return s


def check_bf16(got, ref, name, max_abs=2e-2, rel_l2=1e-2, slack=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / max(nref, 1e-30)
    diff = np.abs(got - ref)
    allow = bf16_ulp(ref) + (0.0 if slack is None else np.asarray(slack, np.float64))
    bad = (diff > max_abs) & (diff > allow * (1 + 1e-9))
    excused = int(((diff > max_abs) & ~bad).sum())
    info = f"{name}: rel_l2={rel:.3e} max_abs={diff.max() if diff.size else 0:.3e} excused={excused} bad={int(bad.sum())}"
    print(info)
    assert rel <= rel_l2, info
    assert not bad.any(), info
    return rel


def check_fp8(got, ref, name, rel_l2=5e-2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"{name}: rel_l2={rel:.3e}")
    assert rel <= rel_l2, f"{name}: rel_l2={rel:.3e}"
    return rel


class GpuMoE:
    """Uploads one workload's inputs and runs moe_forward / moe_backward through the C ABI."""

    def __init__(self, w, d, training=None, canary=True, router=False, mx=False,
                 placement=M.MOE_PLACE_COMBINE):
        self.w, self.d = w, d
        T = d["T"]
        self.T = T
        self.training = w.training if training is None else training
        self.router = router
        self.dtype = M.MOE_MXFP8 if mx else (M.MOE_FP8_E4M3 if w.fp8 else M.MOE_BF16)
        self.prob = M.problem(T, w.H, w.E, w.k, w.I, w.score, w.shared_I, self.dtype, self.training,
                              router, weight_placement=placement)
        self.w_router = dev_bf16(d["w_router"]) if router else None
        self.dw_router = torch.full((w.E, w.H), float("nan"), device="cuda") if router else None
        self.x = dev_bf16(d["x"])
        self.logits = dev(d["logits"])
        self.w_gu = dev_bf16(d["w_gu"])
        self.w_down = dev_bf16(d["w_down"])
        self.shared_gu = dev_bf16(d["shared_gu"]) if w.shared_I else None
        self.shared_down = dev_bf16(d["shared_down"]) if w.shared_I else None
        self.w_gu_scale = self.w_down_scale = None
        if mx:
            E, H, I = w.E, w.H, w.I
            self.w_gu_q = torch.empty((E, 2 * I, H), dtype=torch.uint8, device="cuda")
            self.w_gu_scale = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device="cuda")
            self.w_down_q = torch.empty((E, H, I), dtype=torch.uint8, device="cuda")
            self.w_down_scale = torch.empty((E, H, I // 32), dtype=torch.uint8, device="cuda")
            M.moe_quantize_mxfp8_weights(self.w_gu, self.w_gu_q, self.w_gu_scale)
            M.moe_quantize_mxfp8_weights(self.w_down, self.w_down_q, self.w_down_scale)
            if self.training:  # the second copy, blocked along the stored last axis
                self.w_gu_b = torch.empty((E, H, 2 * I), dtype=torch.uint8, device="cuda")
                self.w_gu_bs = torch.empty((E, H, 2 * I // 32), dtype=torch.uint8, device="cuda")
                self.w_down_b = torch.empty((E, I, H), dtype=torch.uint8, device="cuda")
                self.w_down_bs = torch.empty((E, I, H // 32), dtype=torch.uint8, device="cuda")
                M.moe_quantize_mxfp8_rows(self.w_gu.view(E * H, 2 * I), self.w_gu_b.view(E * H, 2 * I),
                                          self.w_gu_bs.view(E * H, 2 * I // 32))
                M.moe_quantize_mxfp8_rows(self.w_down.view(E * I, H), self.w_down_b.view(E * I, H),
                                          self.w_down_bs.view(E * I, H // 32))
        elif w.fp8:
            E, H, I = w.E, w.H, w.I
            self.w_gu_q = torch.empty((E, 2 * I, H), dtype=torch.uint8, device="cuda")
            self.w_gu_scale = torch.empty((E, 2 * I), dtype=torch.float32, device="cuda")
            self.w_down_q = torch.empty((E, H, I), dtype=torch.uint8, device="cuda")
            self.w_down_scale = torch.empty((E, H), dtype=torch.float32, device="cuda")
            M.moe_quantize_fp8_weights(self.w_gu, self.w_gu_q, self.w_gu_scale)
            M.moe_quantize_fp8_weights(self.w_down, self.w_down_q, self.w_down_scale)
        self.y = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
        nbytes = M.moe_workspace_bytes(self.prob)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        if canary:  # NaN bit patterns everywhere: an unwritten output shows up as NaN
            self.ws.fill_(0xFF)
            self.y.view(torch.int16).fill_(0x7FC0)
        self.views = M.moe_workspace_views(self.prob, self.ws)
        q = w.fp8 or mx
        self.tens = M.tensors(self.x, self.logits, self.w_gu_q if q else self.w_gu,
                              self.w_down_q if q else self.w_down, self.y,
                              self.w_gu_scale, self.w_down_scale, self.shared_gu, self.shared_down,
                              self.w_router, self.dw_router,
                              **({} if not (mx and self.training) else dict(
                                  w_gu_bwd=self.w_gu_b, w_gu_bwd_scale=self.w_gu_bs,
                                  w_down_bwd=self.w_down_b, w_down_bwd_scale=self.w_down_bs)))

    def forward(self):
        M.moe_forward(self.prob, self.tens, self.ws)
        torch.cuda.synchronize()
        return self.y

    def backward(self, dy_bits):
        w = self.w
        self.dy = dev_bf16(dy_bits)
        self.dx = torch.empty((self.T, w.H), dtype=torch.bfloat16, device="cuda")
        self.dw_gu = torch.empty((w.E, w.H, 2 * w.I), dtype=torch.bfloat16, device="cuda")
        self.dw_down = torch.empty((w.E, w.I, w.H), dtype=torch.bfloat16, device="cuda")
        for t in (self.dx, self.dw_gu, self.dw_down):
            t.view(torch.int16).fill_(0x7FC0)
        M.moe_backward(self.prob, self.tens, self.dy, self.dx, self.dw_gu, self.dw_down, self.ws)
        torch.cuda.synchronize()

    def view(self, name, shape, dtype):
        return M.view_tensor(getattr(self.views, name), shape, dtype, self.ws)

    def ints(self):
        w, T = self.w, self.T
        return dict(
            topk_idx=self.view("topk_idx", (T, w.k), torch.int32).cpu().numpy(),
            topk_prob=self.view("topk_prob", (T, w.k), torch.float32).cpu().numpy(),
            counts=self.view("counts", (w.E,), torch.int32).cpu().numpy(),
            offsets=self.view("offsets", (w.E + 1,), torch.int32).cpu().numpy(),
            row_of=self.view("row_of", (T, w.k), torch.int32).cpu().numpy(),
            src_of=self.view("src_of", (T * w.k,), torch.int32).cpu().numpy(),
        )


def mx_gemm_slack(a_abs, b_abs):
    """Accumulation slack of the block-scaled e4m3 GEMM for C = A B^T over K (a_abs [R, K],
    b_abs [N, K]: decoded magnitudes): K 2^-24 sum|ab| for the fp32 accumulation across
    K steps, plus, per 64-wide K step, 2^-10 of that step's largest product. The matrix
    instruction sums one step's 64 products with an error up to about 2^-12 of the largest
    of them (measured: at most 2^-11.9 over 4 M outputs at K = 64 .. 512 with random
    signs), not to fp32 precision; the 2^-10 keeps a 4x margin."""
    a_abs = np.asarray(a_abs, np.float64)
    b_abs = np.asarray(b_abs, np.float64)
    K = a_abs.shape[1]
    out = K * 2.0 ** -24 * (a_abs @ b_abs.T)
    rows = max(1, (1 << 22) // max(1, b_abs.shape[0] * 64))
    for r0 in range(0, a_abs.shape[0], rows):
        sl = slice(r0, r0 + rows)
        for k0 in range(0, K, 64):
            p = a_abs[sl, None, k0:k0 + 64] * b_abs[None, :, k0:k0 + 64]
            out[sl] += 2.0 ** -10 * p.max(axis=2)
    return out


def fp32_sum_bound(a_abs, b_abs_t, n):
    """Bound on the error of fp32 sums of n exact products: n * 2^-24 * sum |a b| per
    element (a_abs [R, n] @ b_abs_t [n, C]), the classic recursive-summation bound."""
    return n * 2.0 ** -24 * (np.asarray(a_abs, np.float64) @ np.asarray(b_abs_t, np.float64))


def check_close(got, ref, bound, name, floor=0.0):
    """Elementwise |got - ref| <= bound (+ floor); prints the worst ratio."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    lim = np.asarray(bound, np.float64) + floor
    ratio = (diff / np.maximum(lim, 1e-300)).max() if diff.size else 0.0
    print(f"{name}: max_abs={diff.max() if diff.size else 0:.3e} worst diff/bound={ratio:.3e}")
    assert (diff <= lim).all(), f"{name}: worst diff/bound {ratio:.3e}"


def topk_gap(logits, k):
    """Per token, the gap between the k-th and (k+1)-th largest logit (inf when k == E)."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]
