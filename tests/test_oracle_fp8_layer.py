"""Pins of the composed per-row / per-channel e4m3 layer of the oracle (Transformer Engine
guide "Mixture of Experts", Grouped GEMM, low precision: the expert GEMMs run in the
recipe's precision; pytorch/ao pull request 2600, Summary: dynamic fp8 activation
quantisation with scaled grouped GEMMs). Inputs are built so that every scale is a power of
two and every operand an exact e4m3 value, where the quantised layer must reproduce the
exact layer, plus a hand-worked token whose output changes if h is quantised before its
bf16 rounding or if W_down is scaled per input row instead of per output column; no GPU."""
import numpy as np

import oracle as O


def _e4m3_values(rng, shape):
    """Random finite e4m3 values (every code but the two NaNs)."""
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, codes & 0xF8, codes).astype(np.uint8)
    return O.e4m3_decode(codes)


def test_exact_operands_reproduce_the_unquantised_gemm1():
    # x rows: e4m3 values with one +-448 entry, times 2^p (row scale 2^p exactly);
    # weight columns: e4m3 values with one +-448 entry, times 2^r (column scale 2^r).
    # Every product is exact and so is every fp64 sum, so g and u (one fp32 rounding of the
    # same sum) and h must be bit-identical to the bf16 layer's.
    rng = np.random.default_rng(0)
    T, H, E, k, I = 24, 64, 3, 2, 32
    x = _e4m3_values(rng, (T, H))
    x[np.arange(T), rng.integers(0, H, T)] = 448.0 * rng.choice([-1.0, 1.0], T)
    x *= np.exp2(rng.integers(-6, 3, (T, 1)))
    w = _e4m3_values(rng, (E, H, 2 * I))
    for e in range(E):
        w[e, rng.integers(0, H, 2 * I), np.arange(2 * I)] = 448.0
    w *= np.exp2(rng.integers(-20, -16, (E, 1, 2 * I)))
    wd = O.to_bf16(rng.standard_normal((E, I, H)) * 0.02)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    a = O.moe_forward(x, logits, w, wd, k, O.SOFTMAX_PRE_RENORM, I)
    b = O.moe_forward(x, logits, w, wd, k, O.SOFTMAX_PRE_RENORM, I, fp8=True)
    qx, sx = O.quantize_rows_e4m3(a["xp"])
    assert np.array_equal(O.e4m3_decode(qx) * sx[:, None], a["xp"])   # lossless here
    for name in ("g", "u", "h"):
        assert np.array_equal(a[name], b[name]), name
    assert np.abs(a["g"]).max() > 0


def _worked_layer():
    """Two tokens, two experts, top-1 (softmax after the top-k: weight exactly 1), H = 8,
    I = 4. Both tokens: x = [448, 0, 1, 1, 1, 0, 0, 0] (row scale 1).
    gate columns: W[1] = 56 (column scale 2^-3), W[2] = 32, so g = 32 (silu(32) rounds to 32
    in fp32). up columns of h0, h1: u0 = 14 (W[2] = 14, scale 2^-5); u1 = 2^-5 + 2^-9 + 2^-15
    (W[2..4], with W[1] = 7 setting the column scale 2^-6; 2^-15 / 2^-6 is the smallest
    e4m3 subnormal). So h = [448, bf16(1.0634765625) = 1.0625, 0, 0]: the h row scale is 1,
    and 1.0625 is the midpoint of the e4m3 neighbours 1 and 1.125, so nearest-even gives 1;
    the fp32 value 1.0634765625 (before the bf16 rounding) would give 1.125.
    W_down: out0 = h1 * 1 (W_down[1, 0] = 1, W_down[2, 0] = 1.75 sets the column scale 2^-8),
    out1 = h1 * 3 (W_down[1, 1] = 3, W_down[3, 1] = 3.5 sets 2^-7). Scaled per input row
    instead, row 1 = [1, 3] has scale 3/448 and 1 becomes 144 * 3/448. Expert 1's W_down is
    twice expert 0's (scales 2^-7, 2^-6)."""
    T, H, E, I = 2, 8, 2, 4
    x = np.zeros((T, H))
    x[:, 0], x[:, 2:5] = 448.0, 1.0
    w = np.zeros((E, H, 2 * I))
    w[:, 1, 0:I], w[:, 2, 0:I] = 56.0, 32.0
    w[:, 2, I + 0] = 14.0
    w[:, 1, I + 1] = 7.0
    w[:, 2, I + 1], w[:, 3, I + 1], w[:, 4, I + 1] = 2.0 ** -5, 2.0 ** -9, 2.0 ** -15
    wd = np.zeros((E, I, H))
    wd[0, 1, 0], wd[0, 2, 0] = 1.0, 1.75
    wd[0, 1, 1], wd[0, 3, 1] = 3.0, 3.5
    wd[1] = 2.0 * wd[0]
    logits = np.array([[1.0, 0.0], [0.0, 1.0]], np.float32)
    return x, logits, w, wd, I


def test_worked_fp8_layer_quantises_bf16_h_per_row_and_w_down_per_column():
    x, logits, w, wd, I = _worked_layer()
    r = O.moe_forward(x, logits, w, wd, 1, O.SOFTMAX_POST, I, fp8=True)
    assert r["topk_idx"].tolist() == [[0], [1]] and r["topk_prob"].tolist() == [[1.0], [1.0]]
    assert r["g"].tolist() == [[32.0] * 4] * 2
    assert r["h"].tolist() == [[448.0, 1.0625, 0.0, 0.0]] * 2
    want = np.zeros((2, 8))
    want[0, :2] = [1.0, 3.0]     # e4m3(1.0625) = 1 (nearest-even), times 1 and 3
    want[1, :2] = [2.0, 6.0]     # expert 1: twice the weights
    assert np.array_equal(r["y"], want), r["y"][:, :2]
    # the same layer in bf16 keeps h1 = 1.0625
    rb = O.moe_forward(x, logits, w, wd, 1, O.SOFTMAX_POST, I)
    assert rb["y"][0, :2].tolist() == [1.0625, 3.1875]
