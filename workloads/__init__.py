"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and lays them out; it holds none of the
MoE layer's arithmetic (no routing, no permutation, no GEMM, no quantisation).
Both the HIP path and the CPU oracle are fed from it.

Recipe (per tensor): ``numpy.random.default_rng(SeedSequence([seed, tensor_id]))``,
values drawn in float32; bfloat16 tensors are rounded to nearest-even by
``torch.Tensor.to(torch.bfloat16)`` and handed over as uint16 bit patterns.

Shapes follow the model families named on the pages (Mixtral-8x7B, Qwen3-30B-A3B,
Llama4-17Bx16E); the sizes the pages leave open are fixed here.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids of the seed sequence
TID_X, TID_LOGITS, TID_WGATE, TID_WUP, TID_WDOWN = 0, 1, 2, 3, 4
TID_SGATE, TID_SUP, TID_SDOWN, TID_DY, TID_PERM, TID_GUMBEL = 5, 6, 7, 8, 9, 10
TID_WROUTER = 11

SOFTMAX_PRE_RENORM, SOFTMAX_POST, SIGMOID = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    score: int
    shared_I: int = 0          # 0: no shared expert
    fp8: bool = False          # e4m3 grouped GEMMs
    training: bool = False     # forward + backward
    hot_experts: tuple = ()    # logits += hot_bias on these experts
    hot_bias: float = 0.0
    zipf_s: float = 0.0        # >0: Gumbel-top-k logits with Zipf weights
    n_empty: int = 0           # experts that never receive a token (zipf only)
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=128, E=4, k=2, I=256, score=SOFTMAX_PRE_RENORM),
    "mixtral": Workload("mixtral", T=4096, H=4096, E=8, k=2, I=14336, score=SOFTMAX_POST),
    "llama4": Workload("llama4", T=8, H=5120, E=16, k=1, I=8192, score=SIGMOID,
                       shared_I=8192, hot_experts=(0, 1, 2), hot_bias=2.0),
    "qwen3": Workload("qwen3", T=4096, H=2048, E=128, k=8, I=768, score=SOFTMAX_PRE_RENORM,
                      training=True),
    "skewed_fp8": Workload("skewed_fp8", T=8192, H=2048, E=128, k=8, I=768,
                           score=SOFTMAX_PRE_RENORM, fp8=True, zipf_s=1.2, n_empty=10),
}


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tid]))


def _normal_f32(seed, tid, shape, std=1.0) -> np.ndarray:
    a = _rng(seed, tid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), nearest-even, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16(seed, tid, shape, std=1.0) -> np.ndarray:
    return to_bf16_bits(_normal_f32(seed, tid, shape, std))


def make_logits(w: Workload, seed: int = 0, T: int | None = None) -> np.ndarray:
    T = w.T if T is None else T
    if w.zipf_s > 0:
        # Gumbel-top-k: l = log(weight_e) + Gumbel(0,1) samples k experts per token
        # without replacement with probability proportional to weight_e.
        perm = _rng(seed, TID_PERM).permutation(w.E)
        live, dead = perm[: w.E - w.n_empty], perm[w.E - w.n_empty:]
        logw = np.zeros(w.E, dtype=np.float64)
        ranks = np.arange(1, live.size + 1, dtype=np.float64)
        logw[live] = -w.zipf_s * np.log(ranks)
        g = _rng(seed, TID_GUMBEL).gumbel(size=(T, w.E))
        l = (logw[None, :] + g).astype(np.float32)
        l[:, dead] = np.float32(-1.0e4)
        return l
    l = _normal_f32(seed, TID_LOGITS, (T, w.E))
    for e in w.hot_experts:
        l[:, e] += np.float32(w.hot_bias)
    return l


def make_inputs(name, seed: int = 0, T: int | None = None, with_weights: bool = True):
    """Return a dict of host arrays for workload ``name`` (a key of WORKLOADS or a Workload).

    bf16 tensors are uint16 bit patterns: x [T,H], w_gu [E,H,2I] (gate columns
    [0,I), up columns [I,2I)), w_down [E,I,H], optional shared_gu [H,2Is],
    shared_down [Is,H], optional dy [T,H], w_router [E,H] (the router projection's
    weight, N(0, 0.02) like the expert weights). logits [T,E] float32.
    ``T`` overrides the token count (same recipe, fewer or more rows).
    """
    w = WORKLOADS[name] if isinstance(name, str) else name
    T = w.T if T is None else T
    out = {"workload": w, "T": T}
    out["x"] = _bf16(seed, TID_X, (T, w.H))
    out["logits"] = make_logits(w, seed, T)
    if w.training:
        out["dy"] = _bf16(seed, TID_DY, (T, w.H))
    if with_weights:
        g = _normal_f32(seed, TID_WGATE, (w.E, w.H, w.I), 0.02)
        u = _normal_f32(seed, TID_WUP, (w.E, w.H, w.I), 0.02)
        out["w_gu"] = to_bf16_bits(np.concatenate([g, u], axis=2))
        del g, u
        out["w_down"] = _bf16(seed, TID_WDOWN, (w.E, w.I, w.H), 0.02)
        out["w_router"] = _bf16(seed, TID_WROUTER, (w.E, w.H), 0.02)
        if w.shared_I:
            sg = _normal_f32(seed, TID_SGATE, (w.H, w.shared_I), 0.02)
            su = _normal_f32(seed, TID_SUP, (w.H, w.shared_I), 0.02)
            out["shared_gu"] = to_bf16_bits(np.concatenate([sg, su], axis=1))
            del sg, su
            out["shared_down"] = _bf16(seed, TID_SDOWN, (w.shared_I, w.H), 0.02)
    return out


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit sizes, for parity cases between the named ones."""
    base = dict(T=64, H=128, E=4, k=2, I=256, score=SOFTMAX_PRE_RENORM)
    base.update(kw)
    return Workload(name, **base)
