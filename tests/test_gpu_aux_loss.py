"""GPU parity (through the C ABI) of the auxiliary load-balancing loss (Transformer Engine
guide "Mixture of Experts", Load balancing): the dense scores and plain top-k map, the
loss from the counts, and its gradient to every logit, against the oracle.

Bounds: the scores are exp / sigmoid / sqrt of fp32 values divided by an fp32 sum of E
terms, within (E + 8) fp32 ulps relative; the loss sums positive terms (chunks of tokens,
then the chunks, then E experts), so its relative error is at most the number of
additions plus the scores' own; the gradient is a product and a difference of such
values."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
from gpu_helpers import check_close, dev, host_vals

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
SCORES = [O.SOFTMAX_PRE_RENORM, O.SOFTMAX_PRE, O.SIGMOID, O.SQRTSOFTPLUS]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("T,E,k", [(300, 16, 4), (4096, 128, 8), (777, 200, 6), (1, 8, 2),
                                   (0, 8, 2)])
@pytest.mark.parametrize("score", SCORES)
def test_aux_loss(T, E, k, score):
    _say("aux loss", T, E, k, score)
    rng = np.random.default_rng(T + E + 10 * score)
    lg = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    if T > 2:
        lg[2, : E // 2] = -np.inf           # masked experts
    total = max(T, 1)
    coeff = 1e-2
    ld = dev(lg) if T else torch.empty((0, E), device="cuda")
    scores = torch.full((T, E), float("nan"), device="cuda")
    rmap = torch.full((T, E), 7, dtype=torch.uint8, device="cuda")
    M.moe_aux_loss_scores(ld, k, score, scores, rmap)
    # counts from a real router (here: the plain one), as the guide does
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    if T:
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        q = torch.empty((T, k), device="cuda")
        M.moe_router_topk(ld, k, score, idx, q, counts)
    loss = torch.full((1,), float("nan"), device="cuda")
    ws = torch.empty(max(M.moe_aux_loss_workspace_bytes(T, E), 4), dtype=torch.uint8, device="cuda")
    M.moe_aux_loss(scores, counts, k, total, coeff, loss, ws)
    torch.cuda.synchronize()
    ref_s = O.aux_scores(lg, score) if T else np.zeros((0, E))
    got_s = host_vals(scores)
    check_close(got_s, ref_s, (E + 8) * U * np.abs(ref_s), "scores")
    if T:
        assert np.array_equal(rmap.cpu().numpy(), O.router_topk(lg, k, score)[3])
    c = counts.cpu().numpy()
    ref_loss = O.aux_loss(ref_s, c, total, k, coeff) if T else 0.0
    chunk = max(64, (T + 511) // 512)
    nb = (T + chunk - 1) // chunk
    got_loss = float(loss.cpu()[0])
    assert abs(got_loss - ref_loss) <= (chunk + nb + 2 * E + 16) * U * abs(ref_loss), (got_loss, ref_loss)
    _say(f"loss {got_loss:.9e} oracle {ref_loss:.9e}")
    if T == 0:
        return
    # gradient, written, then accumulated onto itself with an upstream gradient of 2
    d_logits = torch.full((T, E), float("nan"), device="cuda")
    M.moe_aux_loss_backward(ld, counts, k, total, coeff, score, d_logits)
    torch.cuda.synchronize()
    ref_dl = O.aux_loss_backward(lg, c, total, k, coeff, score)
    # the factor that multiplies (g_e - D) and the size of g, D
    l64 = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
    if score in O.SOFTMAX_KINDS:
        fac = O.aux_scores(lg, score, exact=True)
    else:
        r = O.score_values(l64, score)
        dr = r * (1 - r) if score == O.SIGMOID else 1 / (1 + np.exp(-l64)) / (2 * r)
        fac = np.nan_to_num(dr / r.sum(axis=1, keepdims=True))
    g = coeff * E / (k * total * total) * c[None, :].astype(np.float64)
    D = (O.aux_scores(lg, score, exact=True) * g).sum(axis=1, keepdims=True)
    bound = (2 * E + 64) * U * (np.abs(ref_dl) + fac * (g + D))
    got = host_vals(d_logits)
    fin = np.isfinite(ref_dl).all(axis=1)
    check_close(got[fin], ref_dl[fin], bound[fin], "d_logits")
    two = torch.full((1,), 2.0, device="cuda")
    M.moe_aux_loss_backward(ld, counts, k, total, coeff, score, d_logits, d_loss=two,
                            accumulate=True)
    torch.cuda.synchronize()
    check_close(host_vals(d_logits)[fin], 3 * ref_dl[fin], 4 * bound[fin], "d_logits accumulated")
