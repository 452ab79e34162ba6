"""CPU oracle for the single-device Mixture-of-Experts layer (test infrastructure).

Plain, slow, obviously correct: NumPy float64 arithmetic with an explicit
rounding to float32 (and then to bfloat16 or e4m3) at each point where the GPU
path holds float32 and stores a narrower type. Only tests, the smoke check and
the CPU-baseline leg of the benchmark use this module; the product path never
imports it, and it shares no code with the HIP library.

Every function cites the passage of the pages it follows:
  [TE-MoE]   Transformer Engine user guide, "Mixture of Experts"
  [TE-MIX]   Transformer Engine example te_mixtral.py (TEMixtralSparseMoeBlock)
  [TT-1269]  torchtitan pull request 1269 (Llama4 MoE: GroupedExperts, MoE.forward)
  [AO-2600]  pytorch/ao pull request 2600, "MoE refactor to use grouped_mm and
             scaled_grouped_mm"
  [HF-48201] transformers pull request 48201 (Qwen3MoeSparseMoeBlock benchmark)

Readings taken where the pages are silent are marked READING in the docstrings.

Pinned by tests/test_oracle_*.py against brute force, closed forms, library
routines and finite differences; no function here is "parity unpinned".

``exact=True`` switches every rounding off (pure float64), which the
finite-difference and dense-reference pins use.
"""
from __future__ import annotations

import numpy as np

SOFTMAX_PRE_RENORM, SOFTMAX_POST, SIGMOID, SQRTSOFTPLUS, SOFTMAX_PRE = 0, 1, 2, 3, 4
SOFTMAX_KINDS = (SOFTMAX_PRE_RENORM, SOFTMAX_POST, SOFTMAX_PRE)
E4M3_MAX = 448.0

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 values (exact: bf16 is the top half of fp32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (NaN -> quiet NaN).

    Adds 0x7FFF plus the lowest kept bit to the fp32 pattern and keeps the top half;
    for every non-NaN input the sum fits in 32 bits.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) & 0x8000) | 0x7FC0
    return r


def as_values(a) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values; any float array -> float64."""
    a = np.asarray(a)
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def to_f32(x, exact=False):
    """One rounding of a float64 result to float32 (the GPU's accumulator type)."""
    x = np.asarray(x, dtype=np.float64)
    return x if exact else x.astype(np.float32).astype(np.float64)


def to_bf16(x, exact=False):
    """float64 -> float32 -> bfloat16, returned as float64 values.

    The GPU path holds float32 and stores bfloat16, so the oracle rounds twice,
    in that order, at the same points.
    """
    x = np.asarray(x, dtype=np.float64)
    if exact:
        return x
    return bf16_bits_to_f64(f32_to_bf16_bits(x.astype(np.float32)))


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (the 'fn' variant: no infinities, S.1111.111 is NaN) -> float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits. Exponent field 0
    holds subnormals m/8 * 2^-6. Largest finite value 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3 codes, round to nearest-even, saturating to +-448.

    Exact for every float32 input: the scaling by powers of two is exact in float64
    and ``np.rint`` rounds half to even.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    assert not np.isnan(v).any(), "NaN input to e4m3_encode"
    sign = np.where(np.signbit(v), 0x80, 0x00)
    a = np.minimum(np.abs(v), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal grid: multiples of 2^-9; q == 8 lands exactly on the smallest normal (code 8)
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    mant, ex = np.frexp(np.where(sub, 1.0, a))          # a = mant * 2^ex, mant in [0.5, 1)
    e_unb = ex - 1                                        # a = (2*mant) * 2^e_unb
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)  # 3-bit mantissa, may round up to 8
    e_unb = np.where(q == 8, e_unb + 1, e_unb)
    q = np.where(q == 8, 0, q)
    normal_code = ((e_unb + 7) << 3) | q
    code = np.where(sub, code, normal_code)
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# router  [TE-MoE "Router"; TE-MIX TEMixtralSparseMoeBlock.forward]
# ---------------------------------------------------------------------------


def _logit_values(logits) -> np.ndarray:
    """Logits as float64 values: float32 logits (the layer's input type) widen exactly;
    float64 logits (the exact-arithmetic pins) are kept as they are.
    READING (the pages do not treat non-finite logits): -inf marks an expert that can only
    be chosen when too few others are left, and a NaN logit counts as -inf everywhere
    (selection and weights), so every token always gets k distinct valid expert ids."""
    l = np.asarray(logits)
    if l.dtype != np.float64:
        l = l.astype(np.float32)
    l = l.astype(np.float64)
    return np.where(np.isnan(l), -np.inf, l)


def _best_available(key: np.ndarray, avail: np.ndarray) -> np.ndarray:
    """Per row, the lowest index among the available entries holding the largest key
    (-inf keys included: an available -inf entry still beats every unavailable one)."""
    top = np.where(avail, key, -np.inf).max(axis=1, keepdims=True)
    return np.argmax(avail & (key == top), axis=1)


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert ids per token, in descending order of the logit.

    [TE-MoE "Router"]: the router picks the top-k experts per token.
    READING: selection is on the logits themselves (softmax and sigmoid are strictly
    increasing, so the chosen set is the same real-number choice), ties go to the
    lower expert index, and the ids are listed best first.
    Built as k rounds of arg-max, each round removing the chosen expert.
    """
    l = _logit_values(logits)
    T, E = l.shape
    assert 1 <= k <= E
    avail = np.ones((T, E), dtype=bool)
    idx = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        e = _best_available(l, avail)
        idx[:, j] = e
        avail[rows, e] = False
    return idx


def softplus(l):
    """log(1 + e^l) in float64, as max(l, 0) + log1p(e^-|l|) (no overflow)."""
    l = np.asarray(l, dtype=np.float64)
    return np.maximum(l, 0.0) + np.log1p(np.exp(-np.abs(l)))


def score_values(l, score):
    """Per-expert score of the sigmoid and sqrtsoftplus functions, float64
    [TE-MoE "Router": score functions softmax, sigmoid or sqrtsoftplus].
    SQRTSOFTPLUS: sqrt(softplus(l)) = sqrt(log(1 + e^l))."""
    l = np.asarray(l, dtype=np.float64)
    if score == SIGMOID:
        return 1.0 / (1.0 + np.exp(-l))
    if score == SQRTSOFTPLUS:
        return np.sqrt(softplus(l))
    raise ValueError(f"no per-expert score for score function {score}")


def topk_probs(logits: np.ndarray, idx: np.ndarray, score: int, exact=False,
               scaling_factor=1.0) -> np.ndarray:
    """Routing weights of the selected experts, computed in float64, rounded once to fp32.

    SOFTMAX_PRE_RENORM [TE-MIX forward: softmax in fp32 over all experts, topk, then
      divide by the row sum of the kept weights; AO-2600 mixtral model does the same]:
      p_e = exp(l_e - m) / sum_e' exp(l_e' - m),  q_j = p_idx_j / sum_j' p_idx_j'.
    SOFTMAX_POST [TE-MoE "Router": use_pre_softmax=False applies the softmax after
      the top-k]: q_j = exp(l_idx_j) / sum_j' exp(l_idx_j').
    SIGMOID [TE-MoE "Router" score functions; "Token combine": sigmoid top-1 weights
      are not one and must be applied]: q_j = 1 / (1 + exp(-l_idx_j)).
      READING: no renormalisation of sigmoid weights.
    SQRTSOFTPLUS [TE-MoE "Router" score functions; "Token combine": its weights are not
      one either]: q_j = sqrt(log(1 + exp(l_idx_j))). READING: not renormalised, as
      sigmoid.
    SOFTMAX_PRE [TE-MoE "Router": use_pre_softmax=True applies the softmax before the
      top-k; "Token combine": pre-softmax top-1 weights are not one]: q_j = p_idx_j, the
      softmax over all experts, not renormalised over the kept ones.
    scaling_factor [TE-MoE "Router": scaling rescales the returned weights]: multiplied
      into q after the score function (and after the softmax renormalisation).
    """
    l = _logit_values(logits)
    T = l.shape[0]
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    if score in (SOFTMAX_PRE_RENORM, SOFTMAX_PRE):
        m = l.max(axis=1, keepdims=True)
        p = np.exp(l - m)
        p = p / p.sum(axis=1, keepdims=True)
        ps = np.take_along_axis(p, idx.astype(np.int64), axis=1)
        q = ps / ps.sum(axis=1, keepdims=True) if score == SOFTMAX_PRE_RENORM else ps
    elif score == SOFTMAX_POST:
        m = sel.max(axis=1, keepdims=True)
        z = np.exp(sel - m)
        q = z / z.sum(axis=1, keepdims=True)
    elif score in (SIGMOID, SQRTSOFTPLUS):
        q = score_values(sel, score)
    else:
        raise ValueError(f"unknown score function {score}")
    assert q.shape == (T, idx.shape[1])
    return to_f32(q * float(scaling_factor), exact)


def selection_keys(logits, score, expert_bias=None):
    """The values the top-k ranks (key) and the values grouped routing sums (gval), as
    float32 numbers (the router's math is fp32 [TE-MoE "Router"]; these values decide
    integers, so both sides take the decision in fp32).
      softmax (any order): key = the logit (softmax is increasing); gval = the softmax
        probability over all experts, fp32 (before the top-k, renormalised or not) or the
        logit (after the top-k: the kept logits are the scores the top-k sees).
      sigmoid, sqrtsoftplus: s = fp32(score); without a bias key = the logit and
        gval = s; with expert_bias [TE-MoE "Router" expert bias; "Load balancing": added
        to the scores for the selection only] key = gval = fp32(s + bias).
    """
    l = _logit_values(logits)
    if score in (SIGMOID, SQRTSOFTPLUS):
        sv = to_f32(score_values(l, score))
        if expert_bias is None:
            return l, sv
        kb = to_f32(sv + np.asarray(expert_bias, np.float32).astype(np.float64)[None, :])
        return kb, kb
    if expert_bias is not None:
        raise ValueError("expert_bias applies to the sigmoid and sqrtsoftplus scores")
    if score in (SOFTMAX_PRE_RENORM, SOFTMAX_PRE):
        m = l.max(axis=1, keepdims=True)
        p = np.exp(l - m)
        return l, to_f32(p / p.sum(axis=1, keepdims=True))
    return l, l


def topk_select_ext(logits, k, score, expert_bias=None, num_groups=0, group_topk=0):
    """Top-k with the router's options [TE-MoE "Router": expert bias, grouped routing].

    Grouped routing: the E experts form num_groups equal groups of consecutive ids; a
    group's score is the fp32 sum, best first, of the gvals of its m best experts
    (ranked by key, lower id first on a tie), READING m = k // group_topk (the pages say
    "the sum of its best expert scores" without the count; with the top-k spread over
    group_topk groups, each kept group contributes about k / group_topk experts); the
    group_topk best groups are kept (lower group id first on a tie) and the top-k is
    taken among their experts only. Without groups this is topk_select on the keys.
    """
    key, gval = selection_keys(logits, score, expert_bias)
    T, E = key.shape
    allowed = np.ones((T, E), dtype=bool)
    if num_groups and num_groups > 1:
        assert E % num_groups == 0 and 1 <= group_topk <= num_groups
        gs = E // num_groups
        m = k // group_topk
        assert m >= 1 and k <= group_topk * gs
        gscore = np.zeros((T, num_groups), dtype=np.float64)
        for g in range(num_groups):
            kg = key[:, g * gs:(g + 1) * gs]
            vg = gval[:, g * gs:(g + 1) * gs]
            best = topk_select(kg, m)          # best m by key, lower id first on a tie
            acc = np.zeros(T, dtype=np.float64)
            for j in range(m):                 # fp32 sum, best first
                acc = to_f32(acc + np.take_along_axis(vg, best[:, j:j + 1].astype(np.int64), 1)[:, 0])
            gscore[:, g] = acc
        kept = topk_select(gscore, group_topk)
        allowed[:] = False
        for j in range(group_topk):
            for g in range(num_groups):
                sel = kept[:, j] == g
                allowed[sel, g * gs:(g + 1) * gs] = True
    idx = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    avail = allowed.copy()
    for j in range(k):
        e = _best_available(key, avail)
        idx[:, j] = e
        avail[rows, e] = False
    return idx


def pack_routing_map(rmap):
    """Bit-packed routing map [TE-MoE "Router": routing_map_format bitmap_u8]: bit e%8 of
    byte e//8 of a token's row is routing_map[t,e] (least significant bit first).
    READING: the bit order within a byte, which the pages do not state."""
    return np.packbits(np.asarray(rmap, dtype=np.uint8), axis=1, bitorder="little")


def expert_bias_update(bias, tokens_per_expert, coeff):
    """Auxiliary-loss-free load balancing step [TT-1269 MoE._update_expert_bias; TE-MoE
    "Load balancing": lower the bias of overloaded experts, raise it for under-used
    ones]: delta = coeff * sign(mean(tokens) - tokens), minus its mean; bias + delta.
    Computed in float64 from fp32 inputs, rounded once to fp32."""
    c = np.asarray(tokens_per_expert, dtype=np.float64)
    d = coeff * np.sign(c.mean() - c)
    d = d - d.mean()
    return to_f32(np.asarray(bias, np.float32).astype(np.float64) + d)


def aux_scores(logits, score, exact=False):
    """Dense routing scores for the auxiliary load-balancing loss [TE-MoE "Load balancing":
    fused_compute_score_for_moe_aux_loss returns one score per expert, not only the kept
    top-k, and ignores expert bias and grouped routing].
    READING (the pages give no formula): every token's scores form a distribution over
    the experts, as the router probabilities of the Switch Transformer balance loss (Fedus,
    Zoph and Shazeer 2021, section 2.2) do: softmax (any order) -> the softmax over all
    experts; sigmoid and sqrtsoftplus -> the per-expert scores divided by their sum.
    float64, one rounding to fp32. Returns [T, E]."""
    l = _logit_values(logits)
    if score in SOFTMAX_KINDS:
        z = np.exp(l - l.max(axis=1, keepdims=True))
    else:
        z = score_values(l, score)
    return to_f32(z / z.sum(axis=1, keepdims=True), exact)


def aux_loss(scores, tokens_per_expert, total_num_tokens, topk, coeff, exact=False):
    """Auxiliary load-balancing loss [TE-MoE "Load balancing": fused_moe_aux_loss(scores,
    tokens_per_expert, total_num_tokens, num_experts, topk, coeff) penalises uneven token
    counts and has a gradient with respect to every expert's logit].
    READING: the Switch Transformer balance loss, coeff * E * sum_e f_e P_e, with f_e the
    fraction of the routed (token, choice) pairs that went to expert e, c_e / (k T), and
    P_e the mean score of expert e over the tokens, sum_t s_te / T:
        loss = coeff * E / (k T^2) * sum_e c_e sum_t s_te,
    T = total_num_tokens, E the number of score columns; k = 1 is the published form.
    float64 from the fp32 scores and the integer counts, one rounding to fp32."""
    s = np.asarray(scores, dtype=np.float64)
    c = np.asarray(tokens_per_expert, dtype=np.float64)
    E = s.shape[1]
    T = float(total_num_tokens)
    val = coeff * E / (topk * T * T) * float((c * s.sum(axis=0)).sum())
    return float(to_f32(val, exact))


def aux_loss_backward(logits, tokens_per_expert, total_num_tokens, topk, coeff, score,
                      d_loss=1.0, exact=False):
    """Gradient of aux_loss(aux_scores(logits)) with respect to the logits, for an upstream
    gradient d_loss. With C = d_loss * coeff * E / (k T^2), the loss gradient with respect to
    s_te is g_e = C c_e for every token, then through the normalised scores:
      softmax: dl_te = s_te (g_e - sum_i s_ti g_i);
      sigmoid / sqrtsoftplus, s_te = r_te / sum_i r_ti:
        dl_te = r'(l_te) (g_e - sum_i s_ti g_i) / sum_i r_ti,
        r' = r (1 - r) (sigmoid) or sigmoid(l) / (2 r) (sqrtsoftplus).
    float64, one rounding to fp32. Returns [T, E]."""
    l = _logit_values(logits)
    T_, E = l.shape
    c = np.asarray(tokens_per_expert, dtype=np.float64)
    T = float(total_num_tokens)
    g = d_loss * coeff * E / (topk * T * T) * c[None, :]
    if score in SOFTMAX_KINDS:
        z = np.exp(l - l.max(axis=1, keepdims=True))
        s = z / z.sum(axis=1, keepdims=True)
        dl = s * (g - (s * g).sum(axis=1, keepdims=True))
    else:
        r = score_values(l, score)
        tot = r.sum(axis=1, keepdims=True)
        s = r / tot
        dr = r * (1.0 - r) if score == SIGMOID else (1.0 / (1.0 + np.exp(-l))) / (2.0 * r)
        dl = dr * (g - (s * g).sum(axis=1, keepdims=True)) / tot
    return to_f32(dl, exact)


def router_topk(logits: np.ndarray, k: int, score: int, exact=False, expert_bias=None,
                num_groups=0, group_topk=0, scaling_factor=1.0):
    """Fused score function + top-k [TE-MoE "Router"], with its options (expert bias,
    grouped routing, scaling; see topk_select_ext and topk_probs).

    Returns topk_idx [T,k] int32, topk_prob [T,k], counts [E] int32,
    routing_map [T,E] uint8 (1 at the selected experts), probs_dense [T,E] (the
    weights at the selected experts, 0 elsewhere).
    counts = tokens routed to each expert [TE-MoE "Load balancing": routing_map.sum(0)].
    """
    T, E = logits.shape
    if expert_bias is None and not (num_groups and num_groups > 1):
        idx = topk_select(logits, k)
    else:
        idx = topk_select_ext(logits, k, score, expert_bias, num_groups, group_topk)
    q = topk_probs(logits, idx, score, exact, scaling_factor)
    rmap = np.zeros((T, E), dtype=np.uint8)
    dense = np.zeros((T, E), dtype=np.float64)
    rows = np.arange(T)[:, None]
    rmap[rows, idx] = 1
    dense[rows, idx] = q
    counts = rmap.sum(axis=0).astype(np.int32)
    return idx, q, counts, rmap, dense


def gate_logits(x_vals, w_router_vals, exact=False):
    """Router projection logits[t,e] = sum_h x[t,h] * W_r[e,h], summed in float64, one
    rounding to fp32 [TE-MoE "Example: MoE layer on a single device": a bias-free linear
    layer from the hidden size to the expert count produces the logits the router
    scores; TE-MIX TEMixtralSparseMoeBlock: the gate is a bias-free Linear of shape
    (experts, hidden) applied to the hidden states].
    READING: W_r is [E, H] (the linear layer's weight layout); the logits keep the fp32
    accumulator with no bf16 rounding, since the router's math runs in fp32 whatever
    the logits' type [TE-MoE "Router"].
    """
    x = as_values(x_vals)
    w = as_values(w_router_vals)
    return to_f32(x @ w.T, exact)


def router_backward(logits, idx, d_prob, score, exact=False, scaling_factor=1.0):
    """Gradient of the routing weights with respect to the logits [TE-MoE "Router": the
    score function and the top-k run in one differentiable kernel with fp32 math].

    The top-k choice is piecewise constant, so only the weights' dependence on the logits
    through the score function carries a gradient. Each score function is differentiated
    as it is defined in topk_probs, in float64, then rounded once to fp32:
      SOFTMAX_PRE_RENORM: p = softmax(l) over all experts, s = sum of the kept p,
        q_j = p_idx_j / s. Through the renormalisation dp_i = (dq_i - sum_j q_j dq_j)/s
        for a kept expert i (0 for the others), then through the softmax
        dl_e = p_e (dp_e - sum_i p_i dp_i) for every expert e.
      SOFTMAX_PRE: q_j = p_idx_j with p = softmax(l) over all experts; dp = dq at the
        kept experts (0 elsewhere), dl_e = p_e (dp_e - sum_i p_i dp_i) for every expert e
        (the experts not kept get -p_e sum_j q_j dq_j).
      SOFTMAX_POST: q = softmax of the kept logits, dl_idx_j = q_j (dq_j - sum q dq);
        0 elsewhere.
      SIGMOID: q_j = sigmoid(l_idx_j), dl_idx_j = dq_j q_j (1 - q_j); 0 elsewhere.
      SQRTSOFTPLUS: q_j = sqrt(softplus(l_idx_j)),
        dl_idx_j = dq_j sigmoid(l_idx_j) / (2 q_j); 0 elsewhere.
    A scaling factor c multiplies the weights, so the score function sees c * d_prob.
    Returns d_logits [T, E] (float64 values of fp32 results).
    """
    l = _logit_values(logits)
    T, E = l.shape
    ii = np.asarray(idx, dtype=np.int64)
    dq = np.asarray(d_prob, dtype=np.float64) * float(scaling_factor)
    rows = np.arange(T)[:, None]
    dl = np.zeros((T, E), dtype=np.float64)
    sel = np.take_along_axis(l, ii, axis=1)
    if score == SOFTMAX_PRE_RENORM:
        m = l.max(axis=1, keepdims=True)
        p = np.exp(l - m)
        p = p / p.sum(axis=1, keepdims=True)
        ps = np.take_along_axis(p, ii, axis=1)
        s_ = ps.sum(axis=1, keepdims=True)
        q = ps / s_
        dp = np.zeros((T, E), dtype=np.float64)
        dp[rows, ii] = (dq - (q * dq).sum(axis=1, keepdims=True)) / s_
        dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    elif score == SOFTMAX_PRE:
        m = l.max(axis=1, keepdims=True)
        p = np.exp(l - m)
        p = p / p.sum(axis=1, keepdims=True)
        dp = np.zeros((T, E), dtype=np.float64)
        dp[rows, ii] = dq
        dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    elif score == SOFTMAX_POST:
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        q = z / z.sum(axis=1, keepdims=True)
        dl[rows, ii] = q * (dq - (q * dq).sum(axis=1, keepdims=True))
    elif score == SIGMOID:
        q = 1.0 / (1.0 + np.exp(-sel))
        dl[rows, ii] = dq * q * (1.0 - q)
    elif score == SQRTSOFTPLUS:
        dl[rows, ii] = dq * (1.0 / (1.0 + np.exp(-sel))) / (2.0 * np.sqrt(softplus(sel)))
    else:
        raise ValueError(f"unknown score function {score}")
    return to_f32(dl, exact)


# ---------------------------------------------------------------------------
# dispatch  [TE-MoE "Token dispatch"]
# ---------------------------------------------------------------------------


def dispatch_meta(idx: np.ndarray, E: int):
    """Expert-contiguous row layout for dropless routing [TE-MoE "Token dispatch";
    "Example: MoE layer on a single device": num_out_tokens = num_tokens * top_k].

    offsets[e] = number of routed rows of experts < e (cumulative per-expert counts);
    block e holds the (token, slot) pairs routed to e.
    READING: inside a block, rows follow ascending token index (a token never picks
    an expert twice). row_of[t, j] is the row of token t's j-th choice; src_of[r] is
    the token that fills row r.
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.array([(flat == e).sum() for e in range(E)], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_of = np.full(T * k, -1, dtype=np.int64)
    src_of = np.full(T * k, -1, dtype=np.int64)
    for e in range(E):
        entries = np.nonzero(flat == e)[0]               # ascending flat index = ascending token
        rows = offsets[e] + np.arange(entries.size)
        row_of[entries] = rows
        src_of[rows] = entries // k
    return offsets.astype(np.int32), row_of.reshape(T, k).astype(np.int32), src_of.astype(np.int32)


def dispatch_meta_padded(idx: np.ndarray, E: int, align: int):
    """Padded dispatch layout [TE-MoE "Padding and alignment": each expert's block is
    rounded up to a multiple of align_size rows, and the per-expert padding offsets let
    combine drop the padding; "Receive buffer": counts 129 and 127 need 384 rows at
    alignment 128].

    Block e starts at offsets[e] = sum over e' < e of ceil(count_e' / align) * align; its
    tokens keep the unpadded order (dispatch_meta) and are followed by its padding rows.
    pad_offsets[e] = offsets[e] - (unpadded start of e). src_of is -1 on padding rows.
    Returns offsets [E+1], pad_offsets [E], row_of [T,k], src_of [offsets[E]].
    """
    off_u, row_u, src_u = dispatch_meta(idx, E)
    counts = np.diff(off_u)
    padded = -(-counts // align) * align
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    pad_offsets = (offsets[:E] - off_u[:E]).astype(np.int32)
    e_of = np.asarray(idx, dtype=np.int64)
    row_of = (row_u + pad_offsets[e_of]).astype(np.int32)
    src_of = np.full(int(offsets[E]), -1, dtype=np.int32)
    src_of[row_of.reshape(-1)] = np.repeat(np.arange(idx.shape[0]), idx.shape[1])
    return offsets, pad_offsets, row_of, src_of


def permute(x_bits: np.ndarray, src_of: np.ndarray) -> np.ndarray:
    """Token dispatch gather: row r of the permuted buffer is token src_of[r]
    [TE-MoE "Token dispatch"]. A bit copy."""
    return np.asarray(x_bits)[np.asarray(src_of, dtype=np.int64)]


def quantize_rows_e4m3(vals: np.ndarray):
    """Dynamic per-row e4m3 quantisation [TE-MoE "Grouped GEMM": inputs are quantised
    and the expert GEMMs run in the recipe's precision; AO-2600: fp8 dynamic
    activation quantisation with scaled_grouped_mm].

    READING: s_r = amax_r / 448 (float32 divide), s_r = 1 when the row is all zero;
    q = e4m3(x / s_r) with a float32 divide, nearest-even, saturating.
    vals: float64 array holding float32-representable values (bf16 here), [R, C].
    """
    v = np.asarray(vals, dtype=np.float64).astype(np.float32)
    amax = np.abs(v).max(axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = e4m3_encode((v / s[:, None]).astype(np.float32))
    return q, s


MX_BLOCK = 32


def quantize_mx_e4m3(vals: np.ndarray):
    """MXFP8 quantisation along the last axis: e4m3 elements with one E8M0 (power-of-two)
    scale per block of 32 consecutive values [TE-MIX: the mxfp8 recipe, te_mixtral_mxfp8
    and FP8GlobalStateManager.get_fp8_recipe().mxfp8(); the pages name the recipe only].

    READING, from the OCP Microscaling (MX) v1.0 conversion of a block: X = 2^(floor(
    log2(amax)) - 8), 8 being the largest e4m3 exponent, clamped to [2^-127, 2^127]; the
    codes are e4m3_encode(v / X) (an exact division by a power of two; nearest-even,
    saturating to +-448, which values in [448, 512) * X reach); an all-zero block takes
    X = 2^-127. Returns codes [.., C] uint8 and scale bytes [.., C/32] uint8 (the
    exponent of X plus 127).
    """
    v = np.asarray(vals, dtype=np.float64).astype(np.float32).astype(np.float64)
    C = v.shape[-1]
    assert C % MX_BLOCK == 0
    blk = v.reshape(v.shape[:-1] + (C // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = m * 2^ex, m in [0.5, 1)
    se = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), -127)
    codes = e4m3_encode((blk / np.exp2(se)[..., None]).astype(np.float32))
    return codes.reshape(v.shape), (se + 127).astype(np.uint8)


def mx_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values of MXFP8 codes with their block scale bytes (2^(byte - 127))."""
    c = np.asarray(codes)
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    vals = vals * np.exp2(np.asarray(scales, np.float64) - 127.0)[..., None]
    return vals.reshape(c.shape)


def grouped_gemm_mx(qa, sa, qb, sb, offsets, exact=False):
    """MXFP8 grouped GEMM, C = A_e B_e^T per expert block with the block scales of both
    operands along K: C[r, n] = fp32( sum over blocks b of X_a[r,b] X_b[n,b] *
    sum_{k in b} P_a[r,k] P_b[n,k] ), summed in float64 (every product is exact).
    qa [N, K] codes, sa [N, K/32]; qb [E, Ncol, K] codes, sb [E, Ncol, K/32]."""
    a = mx_decode(qa, sa)
    E = qb.shape[0]
    out = np.zeros((a.shape[0], qb.shape[1]), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = to_f32(a[r0:r1] @ mx_decode(qb[e], sb[e]).T, exact)
    return out


MX_COL_ALIGN = 64


def mx_col_offsets(offsets, align=MX_COL_ALIGN):
    """Starts of the expert blocks along the token axis of the weight-gradient operands:
    expert e takes its rows rounded up to a multiple of `align` (two MX blocks), so its
    blocks start at its own first row and never hold another expert's rows [TE-MIX: the
    mxfp8 recipe with pad_to_multiple=128, every expert's rows padded so that blocks never
    straddle experts]. READING: the padding exists only in these operands (zero values),
    not in the routed rows. Returns int64 [E+1]."""
    n = np.diff(np.asarray(offsets, np.int64))
    return np.concatenate([[0], np.cumsum((n + align - 1) // align * align)]).astype(np.int64)


def quantize_mx_cols(vals: np.ndarray, offsets, align=MX_COL_ALIGN):
    """MXFP8 quantisation along the token axis of expert-contiguous rows [R, C] (the
    reduction axis of the weight-gradient GEMMs): per expert, blocks of 32 consecutive rows
    starting at its first row, its last block completed with zero rows, the same block
    conversion as ``quantize_mx_e4m3``. Returns the transposed codes [C, Kp], scale bytes
    [C, Kp/32] and the expert starts along Kp (``mx_col_offsets``)."""
    v = np.asarray(vals, dtype=np.float64)
    co = mx_col_offsets(offsets, align)
    padded = np.zeros((int(co[-1]), v.shape[1]), dtype=np.float64)
    for e in range(len(co) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        padded[co[e]:co[e] + r1 - r0] = v[r0:r1]
    q, s = quantize_mx_e4m3(padded.T)
    return q, s, co


def grouped_gemm_mx_wgrad(qa_t, sa_t, qb_t, sb_t, col_offsets, exact=False):
    """MXFP8 weight-gradient GEMM: dW_e[m, n] = fp32( sum over expert e's token positions
    k of A_t[m, k] B_t[n, k] ) with both operands' block scales along the token axis,
    summed in float64 (every product is exact). qa_t [M, Kp], qb_t [N, Kp] codes with their
    scale bytes; an expert with no rows gets zeros. Returns float32 values [E, M, N]."""
    a = mx_decode(qa_t, sa_t)
    b = mx_decode(qb_t, sb_t)
    E = len(col_offsets) - 1
    out = np.zeros((E, a.shape[0], b.shape[0]), dtype=np.float64)
    for e in range(E):
        c0, c1 = int(col_offsets[e]), int(col_offsets[e + 1])
        if c1 > c0:
            out[e] = to_f32(a[:, c0:c1] @ b[:, c0:c1].T, exact)
    return out


def quantize_cols_e4m3(w_vals: np.ndarray):
    """Per-output-channel e4m3 quantisation of expert weights [.., K, N]: one scale per
    (expert, column) over the K (reduction) dimension. Same rounding rule as
    ``quantize_rows_e4m3`` applied to the transposed matrix."""
    w = np.asarray(w_vals, dtype=np.float64)
    lead = w.shape[:-2]
    K, N = w.shape[-2:]
    wt = np.swapaxes(w.reshape(-1, K, N), 1, 2).reshape(-1, K)     # rows = (batch, column)
    q, s = quantize_rows_e4m3(wt)
    q = np.swapaxes(q.reshape(-1, N, K), 1, 2).reshape(*lead, K, N)
    return q, s.reshape(*lead, N)


# ---------------------------------------------------------------------------
# grouped expert MLP  [TE-MoE "Grouped GEMM", "Grouped MLP"; TE-MIX _expert_ffn;
#                      TT-1269 GroupedExperts]
# ---------------------------------------------------------------------------


def silu(g):
    """SiLU, x * sigmoid(x) = x / (1 + e^-x), float64."""
    return g / (1.0 + np.exp(-g))


def grouped_gemm(a_vals, b, offsets, exact=False, a_scale=None, b_scale=None, quantize_b=False):
    """Y_e = A_e B_e for every expert block e of the rows of A [TE-MoE "Grouped GEMM":
    Y_i = X_i W_i (the pages write the weight transposed), one result block per expert,
    identical to a loop of one product per expert].

    a_vals [N, K] (expert-contiguous rows); b [E, K, Ncol] as values or bf16 bits
    (converted one expert at a time); offsets [E+1]. Accumulation in float64, then one
    rounding to fp32. Scaled (fp8 recipe): Y = fp32((sum_k qa qb) * s_a[row] * s_b[e, col]),
    with b holding decoded codes and b_scale the column scales, or with quantize_b=True
    each expert's weight is quantised per output column here.
    Returns float64 values of the fp32 results, [N, Ncol].
    """
    a = np.asarray(a_vals, dtype=np.float64)
    E = b.shape[0]
    out = np.zeros((a.shape[0], b.shape[2]), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        be = as_values(b[e])
        col_scale = None if b_scale is None else np.asarray(b_scale, np.float64)[e]
        if quantize_b:
            qb, sb = quantize_cols_e4m3(be)
            be, col_scale = e4m3_decode(qb), sb.astype(np.float64)
        y = a[r0:r1] @ be
        if a_scale is not None:
            y = y * np.asarray(a_scale, np.float64)[r0:r1, None] * col_scale[None, :]
        out[r0:r1] = to_f32(y, exact)
    return out


def swiglu_from_gu(g, u, exact=False):
    """h = silu(g) * u from float32 g, u, then fp32 -> bf16 [TT-1269 GroupedExperts:
    silu(x w1) * (x w3); TE-MIX _expert_ffn: silu(gate) * up]."""
    return to_bf16(silu(g) * u, exact)


def expert_mlp_mx(xp_vals, w_gu_vals, w_down_vals, offsets, I, exact=False):
    """The grouped SwiGLU MLP in the MXFP8 recipe [TE-MIX mxfp8; TE-MoE "Grouped GEMM":
    the expert GEMMs run in the recipe's precision]: x rows and (bf16) h rows are
    quantised per 32-element block along K; each expert's weights per output channel and
    32-element block along K (the GEMM's reduction axis), offline. g, u fp32, h bf16,
    out bf16 as in the other recipes."""
    qx, sx = quantize_mx_e4m3(xp_vals)
    E = len(w_gu_vals)
    qw = [quantize_mx_e4m3(as_values(w_gu_vals[e]).T) for e in range(E)]
    gu = grouped_gemm_mx(qx, sx, np.stack([q for q, _ in qw]), np.stack([s_ for _, s_ in qw]),
                         offsets, exact)
    g, u = gu[:, :I], gu[:, I:]
    h = swiglu_from_gu(g, u, exact)
    qh, sh = quantize_mx_e4m3(h)
    qd = [quantize_mx_e4m3(as_values(w_down_vals[e]).T) for e in range(E)]
    out = grouped_gemm_mx(qh, sh, np.stack([q for q, _ in qd]), np.stack([s_ for _, s_ in qd]),
                          offsets, exact)
    return {"g": g, "u": u, "h": h, "out": to_bf16(out, exact)}


def expert_mlp_mx_backward(mlp, xp_vals, d_out, w_gu_vals, w_down_vals, offsets, I,
                           exact=False):
    """Backward of the grouped SwiGLU MLP in the MXFP8 recipe [TE-MIX mxfp8: the recipe
    covers the training step; TE-MoE "Grouped GEMM": every expert GEMM runs in the
    recipe's precision]. READING (the pages give no per-tensor detail): e4m3 codes for
    every operand, blocks of 32 along each GEMM's own reduction axis, so a tensor used by
    two GEMMs along different axes is quantised twice:
      dh   = fp32(MX_K(d_out) . MX_K(W_down[e])^T)      (blocks along H: d_out rows and
                                                          W_down [I, H] as stored)
      dGU  = SwiGLU'(dh; saved bf16 g, u)               (bf16)
      dxp  = bf16(MX_K(dGU) . MX_K(W_gu[e])^T)          (blocks along 2I: dGU rows and
                                                          W_gu [H, 2I] as stored)
      dW_down[e] = bf16(MX_T(h_e)^T . MX_T(d_out_e))    (blocks along the expert's tokens,
      dW_gu[e]   = bf16(MX_T(xp_e)^T . MX_T(dGU_e))      quantize_mx_cols)
    `mlp` is the forward's dict (g, u fp32 values, h bf16 values); d_out bf16 values."""
    E = len(w_gu_vals)
    qd, sd = quantize_mx_e4m3(d_out)
    wd = [quantize_mx_e4m3(as_values(w_down_vals[e])) for e in range(E)]
    dh = grouped_gemm_mx(qd, sd, np.stack([q for q, _ in wd]), np.stack([s_ for _, s_ in wd]),
                         offsets, exact)
    dg, du = swiglu_backward(dh, to_bf16(mlp["g"], exact), to_bf16(mlp["u"], exact), exact)
    dgu = np.concatenate([dg, du], axis=1)
    qg, sg = quantize_mx_e4m3(dgu)
    wg = [quantize_mx_e4m3(as_values(w_gu_vals[e])) for e in range(E)]
    dxp = to_bf16(grouped_gemm_mx(qg, sg, np.stack([q for q, _ in wg]),
                                  np.stack([s_ for _, s_ in wg]), offsets, exact), exact)
    qh, sh, co = quantize_mx_cols(mlp["h"], offsets)
    qo, so, _ = quantize_mx_cols(d_out, offsets)
    dw_down = to_bf16(grouped_gemm_mx_wgrad(qh, sh, qo, so, co, exact), exact)
    qx, sx, _ = quantize_mx_cols(xp_vals, offsets)
    qt, st, _ = quantize_mx_cols(dgu, offsets)
    dw_gu = to_bf16(grouped_gemm_mx_wgrad(qx, sx, qt, st, co, exact), exact)
    return dict(dh=dh, dgu=dgu, dxp=dxp, dw_down=dw_down, dw_gu=dw_gu)


def expert_mlp(xp_vals, w_gu_vals, w_down_vals, offsets, I, exact=False, fp8=False,
               row_scale=None):
    """Grouped expert SwiGLU MLP on expert-contiguous rows.

    [TE-MIX __init__ / _expert_ffn]: fused gate/up weight with 2I outputs split in
    two halves, gate first. READING: w_gu [E, H, 2I] in the x @ W orientation with
    gate = columns [0, I), up = columns [I, 2I); no biases.
    [TE-MoE "Grouped MLP"]: FC1 with the activation, then FC2 reading the bf16
    intermediate h.
    fp8 [TE-MoE "Grouped GEMM" low precision; AO-2600 fp8dq]: x rows quantised per
    row, weights per output column; h is re-quantised per row from its bf16 value.
    row_scale [N] (ScaledSwiGLU, [TE-MoE "Grouped MLP"]: the activation output is
    multiplied by the routing weight of its row before FC2): h = bf16(silu(g) u p_r),
    READING: the product taken on the fp32 g, u with one rounding, as the unscaled h.
    Returns dict with g, u (fp32 values), h (bf16 values), out (bf16 values).
    """
    if fp8:
        qx, sx = quantize_rows_e4m3(xp_vals)
        gu = grouped_gemm(e4m3_decode(qx), w_gu_vals, offsets, exact, sx, quantize_b=True)
    else:
        gu = grouped_gemm(xp_vals, w_gu_vals, offsets, exact)
    g, u = gu[:, :I], gu[:, I:]
    if row_scale is None:
        h = swiglu_from_gu(g, u, exact)
    else:
        h = to_bf16(silu(g) * u * np.asarray(row_scale, np.float64)[:, None], exact)
    if fp8:
        qh, sh = quantize_rows_e4m3(h)
        out = grouped_gemm(e4m3_decode(qh), w_down_vals, offsets, exact, sh, quantize_b=True)
    else:
        out = grouped_gemm(h, w_down_vals, offsets, exact)
    return {"g": g, "u": u, "h": h, "out": to_bf16(out, exact)}


def dense_mlp(x_vals, w_gu_vals, w_down_vals, I, exact=False):
    """Shared expert: the same SwiGLU MLP on every token, unweighted
    [TT-1269 MoE.forward: shared_expert(x) is the base the routed outputs are added to;
    TE-MoE "Expert parallelism": shared experts are a regular dense MLP]."""
    T = x_vals.shape[0]
    offs = np.array([0, T])
    r = expert_mlp(x_vals, np.asarray(w_gu_vals)[None], np.asarray(w_down_vals)[None], offs, I, exact)
    return r["out"]


# ---------------------------------------------------------------------------
# combine  [TE-MoE "Token combine", "Token probabilities"]
# ---------------------------------------------------------------------------


def combine(out_vals, row_of, prob=None, shared_vals=None, exact=False):
    """y[t] = sum_j q[t,j] * out[row_of[t,j]] (+ shared[t]), summed in float64, one
    rounding to fp32 then bf16 [TE-MoE "Token combine": weighted sum of the per-expert
    contributions in the same pass; "Token probabilities": weights applied once].
    prob=None: unweighted sum (the dispatch backward uses this form). shared_vals is any
    [T, H] term added before the rounding (the shared expert's output; in the backward,
    the router's contribution to dx).
    """
    o = np.asarray(out_vals, dtype=np.float64)
    T, k = row_of.shape
    acc = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = o[np.asarray(row_of[:, j], dtype=np.int64)]
        if prob is not None:
            rows = rows * np.asarray(prob, np.float64)[:, j:j + 1]
        acc += rows
    if shared_vals is not None:
        acc += np.asarray(shared_vals, dtype=np.float64)
    return to_bf16(acc, exact)


def prob_grad(dy_vals, out_vals, row_of, exact=False, rows_first=False):
    """Gradient of y[t] = sum_j q[t,j] out[row_of[t,j]] (+ shared[t]) with respect to
    the routing weights: d_prob[t,j] = sum_h dy[t,h] * out[row_of[t,j],h], summed in
    float64, one rounding to fp32 [TE-MoE "Token combine": the merging weights are an
    input of the differentiable combine]. out holds the stored (bf16) expert outputs.
    rows_first: the first argument holds the routed rows and the second the token rows
    (weights applied to the expert inputs: d_prob[t,j] = <dxp[row_of[t,j]], x[t]>)."""
    a = np.asarray(as_values(dy_vals), dtype=np.float64)
    b = np.asarray(as_values(out_vals), dtype=np.float64)
    if rows_first:
        a, b = b, a
    T, k = row_of.shape
    dq = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        dq[:, j] = (a * b[np.asarray(row_of[:, j], dtype=np.int64)]).sum(axis=1)
    return to_f32(dq, exact)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------


PLACE_COMBINE, PLACE_INPUT, PLACE_ACTIVATION = 0, 1, 2


def row_weights(q, row_of, n_rows):
    """The routing weight of every routed row: w[row_of[t, j]] = q[t, j]."""
    w = np.zeros(n_rows)
    for j in range(row_of.shape[1]):
        w[np.asarray(row_of[:, j], np.int64)] = np.asarray(q, np.float64)[:, j]
    return w


def moe_forward(x_bits, logits, w_gu_bits, w_down_bits, k, score, I,
                shared_gu_bits=None, shared_down_bits=None, fp8=False, exact=False,
                placement=PLACE_COMBINE, mx=False):
    """Route -> dispatch -> grouped MLP -> combine [TE-MoE "Introduction", the four
    stages; "Example: MoE layer on a single device"]. x and the weights are bf16 bit
    patterns (or float64 values, for the exact-arithmetic pins); logits are float32.
    placement PLACE_INPUT applies the routing weights to the expert inputs instead of
    the outputs [TT-1269 MoE.forward, scoring_before_experts: the routed rows are
    multiplied by their scores in fp32 and cast back to the activation type, and the
    outputs are summed unweighted]: xp[r] = bf16(q[t,j] * x[t]), y = sum_j out[row_of].
    placement PLACE_ACTIVATION applies them to the SwiGLU output before FC2 [TE-MoE
    "Grouped MLP": ScaledSwiGLU; with a bias-free FC2 the expert output is then already
    weighted and the combine must not weight it again]: h = bf16(silu(g) u q), y = sum_j
    out[row_of].
    Returns a dict of every intermediate."""
    x = as_values(x_bits)
    E = logits.shape[1]
    idx, q, counts, rmap, dense = router_topk(logits, k, score, exact)
    offsets, row_of, src_of = dispatch_meta(idx, E)
    xp = x[src_of.astype(np.int64)]
    if placement == PLACE_INPUT:
        qr = np.zeros(len(src_of))
        for j in range(k):
            qr[row_of[:, j].astype(np.int64)] = q[:, j]
        xp = to_bf16(xp * qr[:, None], exact)
    rscale = row_weights(q, row_of, len(src_of)) if placement == PLACE_ACTIVATION else None
    mlp = (expert_mlp_mx(xp, w_gu_bits, w_down_bits, offsets, I, exact) if mx else
           expert_mlp(xp, w_gu_bits, w_down_bits, offsets, I, exact, fp8, rscale))
    shared = None
    if shared_gu_bits is not None:
        Is = shared_down_bits.shape[0]
        shared = dense_mlp(x, shared_gu_bits, shared_down_bits, Is, exact)
    y = combine(mlp["out"], row_of, q if placement == PLACE_COMBINE else None, shared, exact)
    res = dict(topk_idx=idx, topk_prob=q, counts=counts, routing_map=rmap, probs_dense=dense,
               offsets=offsets, row_of=row_of, src_of=src_of, xp=xp, shared=shared, y=y,
               x=x, logits=logits, score=score, placement=placement)
    res.update(mlp)
    return res


def swiglu_backward(dh, g, u, exact=False):
    """Gradient of h = silu(g) * u: with s = sigmoid(g),
    dg = dh * u * s * (1 + g (1 - s)),  du = dh * g * s.  Returns bf16 values."""
    s = 1.0 / (1.0 + np.exp(-g))
    dg = dh * u * s * (1.0 + g * (1.0 - s))
    du = dh * g * s
    return to_bf16(dg, exact), to_bf16(du, exact)


def grouped_gemm_dw(a_vals, b_vals, offsets, exact=False, out_bf16=False):
    """dW_e = A_e^T B_e over the rows of each expert block (reduction over that expert's
    routed rows) [TE-MoE "Example": every stage is differentiable]. An expert with no
    rows gets a zero gradient. Returns fp32 values [E, Ka, Kb] (bf16 values when
    out_bf16: fp32 then bf16, one expert at a time)."""
    a = np.asarray(a_vals, dtype=np.float64)
    b = np.asarray(b_vals, dtype=np.float64)
    E = len(offsets) - 1
    out = np.zeros((E, a.shape[1], b.shape[1]), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            y = to_f32(a[r0:r1].T @ b[r0:r1], exact)
            out[e] = to_bf16(y, exact) if out_bf16 else y
    return out


def moe_backward(fwd, dy_bits, w_gu_bits, w_down_bits, I, exact=False, w_router_bits=None,
                 mx=False):
    """Backward of the expert path for an upstream gradient dy [T, H]
    [TE-MoE "Example: MoE layer on a single device": all stages differentiable;
    HF-48201 "Numbers": the block is timed forward + backward].

    READING: without a router weight the logits are an input, so no gradient flows to
    the router and dx goes through the expert path only. dW are rounded to bf16.
    With w_router_bits [E, H] (the logits were gate_logits(x, W_r)) the router is
    differentiated too [TE-MoE "Router": one differentiable kernel]:
      d_prob    = prob_grad(dy, out, row_of);  d_logits = router_backward(...)
      dW_router = fp32(d_logits^T @ x)   (float64 sum of the fp32 d_logits values)
      dx[t]     = bf16(sum_j dxp[row_of[t,j]] + sum_e d_logits[t,e] W_r[e])   (one
                  rounding of the float64 sum of both paths)
      d_out[row_of[t,j]] = bf16(q[t,j] * dy[t])                 (combine backward)
      dh    = fp32(d_out_e @ W_down[e]^T);  dGU = SwiGLU'(dh; saved bf16 g, u)
      dW_down[e] = bf16(h_e^T @ d_out_e)
      dxp   = bf16(dGU_e @ W_gu[e]^T);      dW_gu[e] = bf16(xp_e^T @ dGU_e)
      dx[t] = bf16(sum_j dxp[row_of[t,j]])                      (dispatch backward)
    mx: the four expert GEMMs in the MXFP8 recipe (``expert_mlp_mx_backward``; the forward
    ran with mx too).
    Weights on the SwiGLU output (PLACE_ACTIVATION, ScaledSwiGLU): the combine was
    unweighted, so d_out[row_of[t,j]] = dy[t]; dh = fp32(d_out W_down^T) is the gradient
    of the scaled h, the SwiGLU backward takes p dh, and
      d_prob[t, j] = sum_i dh[r, i] silu(g[r, i]) u[r, i],  r = row_of[t, j]
    (fp32, from the saved bf16 g, u); dx = bf16(sum_j dxp[row_of[t,j]] (+ router term)).
    """
    dy = as_values(dy_bits)
    row_of, q, offsets = fwd["row_of"], fwd["topk_prob"], fwd["offsets"]
    place = fwd.get("placement", PLACE_COMBINE)
    T, k = row_of.shape
    N = T * k
    H = dy.shape[1]
    w_gu = np.asarray(w_gu_bits)     # converted one expert at a time inside the GEMMs
    w_d = np.asarray(w_down_bits)
    d_out = np.zeros((N, H), dtype=np.float64)
    for j in range(k):
        d_out[row_of[:, j].astype(np.int64)] = (to_bf16(dy * q[:, j:j + 1], exact)
                                                if place == PLACE_COMBINE else dy)
    if mx:
        m = expert_mlp_mx_backward(fwd, fwd["xp"], d_out, w_gu, w_d, offsets, I, exact)
        dh, dgu, dxp, dw_gu, dw_down = m["dh"], m["dgu"], m["dxp"], m["dw_gu"], m["dw_down"]
    else:
        # GEMM2 backward: dh = d_out W_d^T (per expert), then the SwiGLU backward
        dh = grouped_gemm(d_out, np.swapaxes(w_d, 1, 2), offsets, exact)
        g_saved, u_saved = to_bf16(fwd["g"], exact), to_bf16(fwd["u"], exact)
        if place == PLACE_ACTIVATION:
            rw = row_weights(q, row_of, N)
            dg, du = swiglu_backward(dh * rw[:, None], g_saved, u_saved, exact)
        else:
            dg, du = swiglu_backward(dh, g_saved, u_saved, exact)
        dgu = np.concatenate([dg, du], axis=1)
        dw_down = grouped_gemm_dw(fwd["h"], d_out, offsets, exact, out_bf16=True)
        # GEMM1 backward
        dxp = to_bf16(grouped_gemm(dgu, np.swapaxes(w_gu, 1, 2), offsets, exact), exact)
        dw_gu = grouped_gemm_dw(fwd["xp"], dgu, offsets, exact, out_bf16=True)
    res = dict(d_out=d_out, dh=dh, dgu=dgu, dxp=dxp, dw_gu=dw_gu, dw_down=dw_down)
    dx_router = None
    if w_router_bits is not None:
        # the weights met the expert outputs (combine) or the expert inputs (input)
        if place == PLACE_INPUT:
            d_prob = prob_grad(dxp, fwd["x"], row_of, exact, rows_first=True)
        elif place == PLACE_ACTIVATION:
            hu = silu(to_bf16(fwd["g"], exact)) * to_bf16(fwd["u"], exact)
            per_row = (dh * hu).sum(axis=1)
            d_prob = to_f32(np.stack([per_row[np.asarray(row_of[:, j], np.int64)]
                                      for j in range(k)], axis=1), exact)
        else:
            d_prob = prob_grad(dy, fwd["out"], row_of, exact)
        d_logits = router_backward(fwd["logits"], fwd["topk_idx"], d_prob, fwd["score"], exact,
                                   fwd.get("scaling_factor", 1.0))
        dx_router = d_logits @ as_values(w_router_bits)
        res.update(d_prob=d_prob, d_logits=d_logits, dx_router=dx_router,
                   dw_router=to_f32(d_logits.T @ fwd["x"], exact))
    # input placement: xp = q x, so dx gets q * dxp
    res["dx"] = combine(dxp, row_of, q if place == PLACE_INPUT else None, dx_router, exact)
    return res
