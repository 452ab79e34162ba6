"""Python binding of libmoe_amd.so, the MI355X (gfx950) MoE layer hot path.

Argument marshalling only: every function here checks tensor dtypes, shapes and
devices, then calls the C entry point of the same name declared in
include/moe_amd.h. All arithmetic runs in the HIP kernels. PyTorch supplies device
memory and the current stream. The library must have been built
(``python -m mixture_experts_layer_amd._build``); importing without it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library then shares)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_amd.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_BF16, MOE_FP8_E4M3, MOE_FP32, MOE_MXFP8 = 0, 1, 2, 3
MOE_SOFTMAX_PRE_RENORM, MOE_SOFTMAX_POST, MOE_SIGMOID, MOE_SQRTSOFTPLUS, MOE_SOFTMAX_PRE = range(5)
MOE_GEMM_NN, MOE_GEMM_NT, MOE_GEMM_TN_DW = 0, 1, 2
MOE_PLACE_COMBINE, MOE_PLACE_INPUT, MOE_PLACE_ACTIVATION = 0, 1, 2

EXPORTS = [
    "moe_status_str", "moe_router_topk", "moe_permute_workspace_bytes", "moe_permute",
    "moe_grouped_gemm_swiglu", "moe_grouped_gemm", "moe_grouped_gemm_swiglu_bwd",
    "moe_set_gemm_max_blocks", "moe_unpermute_combine", "moe_combine_backward", "moe_quantize_fp8_rows",
    "moe_quantize_fp8_weights", "moe_workspace_bytes", "moe_workspace_views", "moe_forward",
    "moe_backward", "moe_router_logits", "moe_combine_backward_router",
    "moe_router_weight_grad_workspace_bytes", "moe_router_weight_grad",
    "moe_dispatch_backward_router", "moe_router_topk_ex", "moe_expert_bias_update",
    "moe_dispatch_backward_router_input", "moe_padded_rows", "moe_permute_padded",
    "moe_quantize_mxfp8_rows", "moe_quantize_mxfp8_weights", "moe_grouped_gemm_mxfp8",
    "moe_mxfp8_cols_capacity", "moe_mxfp8_col_offsets", "moe_quantize_mxfp8_cols",
    "moe_grouped_gemm_mxfp8_wgrad", "moe_grouped_gemm_mxfp8_swiglu_bwd",
    "moe_aux_loss_scores", "moe_aux_loss_workspace_bytes", "moe_aux_loss",
    "moe_aux_loss_backward", "moe_grouped_gemm_swiglu_scaled",
    "moe_grouped_gemm_swiglu_scaled_bwd", "moe_permute_probs", "moe_dispatch_backward_router_scaled",
    "moe_permute_noalloc", "moe_permute_noalloc_limit", "moe_grouped_gemm_splitk_workspace_bytes",
]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} returned {_status_name(status)} ({status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("H", ctypes.c_int), ("E", ctypes.c_int),
                ("k", ctypes.c_int), ("I", ctypes.c_int), ("shared_I", ctypes.c_int),
                ("score", ctypes.c_int), ("dtype", ctypes.c_int), ("training", ctypes.c_int),
                ("router", ctypes.c_int), ("num_groups", ctypes.c_int), ("group_topk", ctypes.c_int),
                ("scaling_factor", ctypes.c_float), ("weight_placement", ctypes.c_int),
                ("align_size", ctypes.c_int)]


class Tensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("x", "logits", "w_gu", "w_gu_scale", "w_down", "w_down_scale",
                 "shared_gu", "shared_down", "y", "w_router", "dw_router", "expert_bias",
                 "w_gu_bwd", "w_gu_bwd_scale", "w_down_bwd", "w_down_bwd_scale")]


class RouterOpts(ctypes.Structure):
    _fields_ = [("expert_bias", ctypes.c_void_p), ("num_groups", ctypes.c_int),
                ("group_topk", ctypes.c_int), ("scaling_factor", ctypes.c_float),
                ("map_format", ctypes.c_int)]


class Views(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_prob", "counts", "offsets", "row_of", "src_of", "xp",
                 "xp_scale", "gu", "h", "hq", "h_scale", "out", "xq", "xq_scale", "hq_scale",
                 "shared_h", "shared_out",
                 "shared_offsets", "d_out", "dgu", "dxp", "scratch")] + \
               [("scratch_bytes", ctypes.c_size_t), ("pad_offsets", ctypes.c_void_p),
                ("rows", ctypes.c_int)] + \
               [(n, ctypes.c_void_p) for n in ("logits", "d_logits", "router_ws")] + \
               [("router_ws_bytes", ctypes.c_size_t)] + \
               [(n, ctypes.c_void_p) for n in ("mx_col_offsets", "dgq", "dgq_scale", "mx_ta",
                                               "mx_ta_scale", "mx_tb", "mx_tb_scale")] + \
               [("mx_kp", ctypes.c_int)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m mixture_experts_layer_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "moe_status_str": ([i], ctypes.c_char_p),
        "moe_router_topk": ([vp, i, i, i, i, vp, vp, vp, vp, vp, vp], i),
        "moe_permute_workspace_bytes": ([i, i, i], sz),
        "moe_permute": ([vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp, sz, vp], i),
        "moe_grouped_gemm_swiglu": ([vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, sz, vp], i),
        "moe_grouped_gemm": ([i, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, vp, sz, vp], i),
        "moe_grouped_gemm_splitk_workspace_bytes": ([i, i, i], sz),
        "moe_grouped_gemm_swiglu_bwd": ([vp, vp, vp, vp, i, i, i, i, vp, vp], i),
        "moe_set_gemm_max_blocks": ([i], i),
        "moe_unpermute_combine": ([vp, vp, vp, vp, i, i, i, vp, vp], i),
        "moe_combine_backward": ([vp, vp, vp, i, i, i, vp, vp], i),
        "moe_quantize_fp8_rows": ([vp, i, i, vp, vp, vp], i),
        "moe_quantize_fp8_weights": ([vp, i, i, i, vp, vp, vp], i),
        "moe_workspace_bytes": ([ctypes.POINTER(Problem)], sz),
        "moe_workspace_views": ([ctypes.POINTER(Problem), vp, sz, ctypes.POINTER(Views)], i),
        "moe_forward": ([ctypes.POINTER(Problem), ctypes.POINTER(Tensors), vp, sz, vp], i),
        "moe_backward": ([ctypes.POINTER(Problem), ctypes.POINTER(Tensors), vp, vp, vp, vp, vp,
                          sz, vp], i),
        "moe_router_logits": ([vp, vp, i, i, i, vp, vp], i),
        "moe_combine_backward_router": ([vp, vp, vp, vp, vp, vp, i, i, i, i, i, ctypes.c_float, vp,
                                         vp, vp, vp], i),
        "moe_router_topk_ex": ([vp, i, i, i, i, ctypes.POINTER(RouterOpts), vp, vp, vp, vp, vp, vp], i),
        "moe_expert_bias_update": ([vp, vp, i, ctypes.c_float, vp], i),
        "moe_dispatch_backward_router_input": ([vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                                ctypes.c_float, vp, vp, vp], i),
        "moe_padded_rows": ([i, i, i, i], sz),
        "moe_quantize_mxfp8_rows": ([vp, i, i, vp, vp, vp], i),
        "moe_quantize_mxfp8_weights": ([vp, i, i, i, vp, vp, vp], i),
        "moe_grouped_gemm_mxfp8": ([vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp], i),
        "moe_mxfp8_cols_capacity": ([i, i], ctypes.c_longlong),
        "moe_mxfp8_col_offsets": ([vp, i, vp, vp], i),
        "moe_quantize_mxfp8_cols": ([vp, i, i, vp, vp, i, i, vp, vp, vp], i),
        "moe_grouped_gemm_mxfp8_wgrad": ([vp, vp, vp, vp, vp, i, i, i, i, vp, vp], i),
        "moe_grouped_gemm_mxfp8_swiglu_bwd": ([vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp], i),
        "moe_permute_padded": ([vp, vp, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, sz, vp], i),
        "moe_router_weight_grad_workspace_bytes": ([i, i, i], sz),
        "moe_router_weight_grad": ([vp, vp, i, i, i, vp, vp, sz, vp], i),
        "moe_dispatch_backward_router": ([vp, vp, vp, vp, vp, i, i, i, i, vp, vp], i),
        "moe_aux_loss_scores": ([vp, i, i, i, i, vp, vp, vp], i),
        "moe_aux_loss_workspace_bytes": ([i, i], sz),
        "moe_aux_loss": ([vp, vp, i, i, i, i, ctypes.c_float, vp, vp, sz, vp], i),
        "moe_aux_loss_backward": ([vp, vp, i, i, i, i, ctypes.c_float, i, vp, vp, i, vp], i),
        "moe_grouped_gemm_swiglu_scaled": ([vp, vp, vp, vp, i, i, i, i, vp, vp, vp], i),
        "moe_grouped_gemm_swiglu_scaled_bwd": ([vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp], i),
        "moe_permute_probs": ([vp, vp, i, i, vp, vp], i),
        "moe_permute_noalloc": ([vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp], i),
        "moe_permute_noalloc_limit": ([], sz),
        "moe_dispatch_backward_router_scaled": ([vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                                 ctypes.c_float, vp, vp, vp], i),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    return lib


_lib = _load()


def lib():
    return _lib


def _status_name(st):
    return _lib.moe_status_str(st).decode()


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


def _p(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _want(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _want_rows(t, dtype, min_rows, cols, name):
    """A routed-row buffer: at least min_rows rows (a padded dispatch has more) of cols."""
    if t.dtype != dtype or t.dim() != 2 or t.shape[0] < min_rows or t.shape[1] != cols:
        raise ValueError(f"{name}: expected {dtype} [>= {min_rows}, {cols}], got {t.dtype} "
                         f"{tuple(t.shape)}")


_SCORE = {"softmax_pre_renorm": MOE_SOFTMAX_PRE_RENORM, "softmax_post": MOE_SOFTMAX_POST,
          "sigmoid": MOE_SIGMOID, "sqrtsoftplus": MOE_SQRTSOFTPLUS,
          "softmax_pre": MOE_SOFTMAX_PRE}


def _score(s):
    return _SCORE[s] if isinstance(s, str) else int(s)


# ---- stage calls ---------------------------------------------------------------------

def moe_status_str(status):
    """Name of a moe_status_t value."""
    return _lib.moe_status_str(int(status)).decode()


def moe_router_topk(logits, k, score, topk_idx, topk_prob, counts, routing_map=None,
                    probs_dense=None, stream=None):
    T, E = logits.shape
    _want(logits, torch.float32, (T, E), "logits")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(topk_prob, torch.float32, (T, k), "topk_prob")
    _want(counts, torch.int32, (E,), "counts")
    if routing_map is not None:
        _want(routing_map, torch.uint8, (T, E), "routing_map")
    if probs_dense is not None:
        _want(probs_dense, torch.float32, (T, E), "probs_dense")
    _check("moe_router_topk", _lib.moe_router_topk(
        _p(logits), T, E, k, _score(score), _p(topk_idx), _p(topk_prob), _p(counts),
        _p(routing_map), _p(probs_dense), _stream(stream)))


def router_opts(expert_bias=None, num_groups=0, group_topk=0, scaling_factor=1.0, bitmap=False):
    if expert_bias is not None:
        _want(expert_bias, torch.float32, (expert_bias.numel(),), "expert_bias")
    return RouterOpts(_p(expert_bias), int(num_groups), int(group_topk), float(scaling_factor),
                      int(bool(bitmap)))


def moe_router_topk_ex(logits, k, score, opts, topk_idx, topk_prob, counts, routing_map=None,
                       probs_dense=None, stream=None):
    T, E = logits.shape
    _want(logits, torch.float32, (T, E), "logits")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(topk_prob, torch.float32, (T, k), "topk_prob")
    _want(counts, torch.int32, (E,), "counts")
    if routing_map is not None:
        cols = (E + 7) // 8 if opts is not None and opts.map_format else E
        _want(routing_map, torch.uint8, (T, cols), "routing_map")
    if probs_dense is not None:
        _want(probs_dense, torch.float32, (T, E), "probs_dense")
    _check("moe_router_topk_ex", _lib.moe_router_topk_ex(
        _p(logits), T, E, k, _score(score), None if opts is None else ctypes.byref(opts),
        _p(topk_idx), _p(topk_prob), _p(counts), _p(routing_map), _p(probs_dense),
        _stream(stream)))


def moe_expert_bias_update(expert_bias, tokens_per_expert, coeff, stream=None):
    E = expert_bias.numel()
    _want(expert_bias, torch.float32, (E,), "expert_bias")
    _want(tokens_per_expert, torch.int32, (E,), "tokens_per_expert")
    _check("moe_expert_bias_update", _lib.moe_expert_bias_update(
        _p(expert_bias), _p(tokens_per_expert), E, float(coeff), _stream(stream)))


def moe_permute_workspace_bytes(T, E, k):
    return int(_lib.moe_permute_workspace_bytes(T, E, k))


def moe_permute(x, topk_idx, E, xp, offsets, row_of, src_of, ws, out_dtype=MOE_BF16,
                xp_scale=None, stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    _want(x, torch.bfloat16, (T, H), "x")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(xp, torch.bfloat16 if out_dtype == MOE_BF16 else torch.uint8, (T * k, H), "xp")
    _want(offsets, torch.int32, (E + 1,), "offsets")
    _want(row_of, torch.int32, (T, k), "row_of")
    _want(src_of, torch.int32, (T * k,), "src_of")
    _check("moe_permute", _lib.moe_permute(
        _p(x), _p(topk_idx), T, H, E, k, out_dtype, _p(xp), _p(xp_scale), _p(offsets),
        _p(row_of), _p(src_of), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute_noalloc(x, topk_idx, E, xp, offsets, row_of, src_of, out_dtype=MOE_BF16,
                        xp_scale=None, stream=None):
    """moe_permute without a workspace: the scratch is the library's own device array."""
    T, H = x.shape
    k = topk_idx.shape[1]
    _want(x, torch.bfloat16, (T, H), "x")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(xp, torch.bfloat16 if out_dtype == MOE_BF16 else torch.uint8, (T * k, H), "xp")
    _want(offsets, torch.int32, (E + 1,), "offsets")
    _want(row_of, torch.int32, (T, k), "row_of")
    _want(src_of, torch.int32, (T * k,), "src_of")
    _check("moe_permute_noalloc", _lib.moe_permute_noalloc(
        _p(x), _p(topk_idx), T, H, E, k, out_dtype, _p(xp), _p(xp_scale), _p(offsets),
        _p(row_of), _p(src_of), _stream(stream)))


def moe_permute_noalloc_limit():
    return int(_lib.moe_permute_noalloc_limit())


def moe_padded_rows(T, E, k, align):
    return int(_lib.moe_padded_rows(T, E, k, align))


def moe_permute_padded(x, topk_idx, E, align, xp, offsets, pad_offsets, row_of, src_of, ws,
                       out_dtype=MOE_BF16, xp_scale=None, stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    R = moe_padded_rows(T, E, k, align)
    _want(x, torch.bfloat16, (T, H), "x")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(xp, torch.bfloat16 if out_dtype == MOE_BF16 else torch.uint8, (R, H), "xp")
    _want(offsets, torch.int32, (E + 1,), "offsets")
    _want(pad_offsets, torch.int32, (E,), "pad_offsets")
    _want(row_of, torch.int32, (T, k), "row_of")
    _want(src_of, torch.int32, (R,), "src_of")
    _check("moe_permute_padded", _lib.moe_permute_padded(
        _p(x), _p(topk_idx), T, H, E, k, align, out_dtype, _p(xp), _p(xp_scale), _p(offsets),
        _p(pad_offsets), _p(row_of), _p(src_of), _p(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_grouped_gemm_splitk_workspace_bytes(rows, G, ncols):
    return int(_lib.moe_grouped_gemm_splitk_workspace_bytes(rows, G, ncols))


def _ws(ws):
    """(pointer, bytes) of an optional uint8 device workspace."""
    if ws is None:
        return None, 0
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("ws: a contiguous uint8 tensor")
    return ws.data_ptr(), ws.numel()


def moe_grouped_gemm_swiglu(xp, w_gu, offsets, h, gu_saved=None, dtype=MOE_BF16, xp_scale=None,
                            w_scale=None, stream=None, ws=None):
    rows, H = xp.shape
    G = offsets.numel() - 1
    I = h.shape[1]
    _want(h, torch.bfloat16, (rows, I), "h")
    if dtype == MOE_BF16:
        _want(w_gu, torch.bfloat16, (G, H, 2 * I), "w_gu")
    else:
        _want(w_gu, torch.uint8, (G, 2 * I, H), "w_gu")
    if gu_saved is not None:
        _want(gu_saved, torch.bfloat16, (rows, 2 * I), "gu_saved")
    wp, wb = _ws(ws)
    _check("moe_grouped_gemm_swiglu", _lib.moe_grouped_gemm_swiglu(
        _p(xp), _p(xp_scale), _p(w_gu), _p(w_scale), _p(offsets), G, rows, H, I, dtype, _p(h),
        _p(gu_saved), wp, wb, _stream(stream)))


def moe_grouped_gemm(mode, A, B, offsets, C, dtype=MOE_BF16, a_scale=None, b_scale=None,
                     stream=None, ws=None):
    G = offsets.numel() - 1
    rows = A.shape[0]
    c_dtype = MOE_FP32 if C.dtype == torch.float32 else MOE_BF16
    if mode == MOE_GEMM_TN_DW:
        M, N, K = A.shape[1], B.shape[1], 0
        _want(C, C.dtype, (G, M, N), "C")
    else:
        K = A.shape[1]
        N = B.shape[2] if mode == MOE_GEMM_NN else B.shape[1]
        M = 0
        _want(C, C.dtype, (rows, N), "C")
    wp, wb = _ws(ws)
    _check("moe_grouped_gemm", _lib.moe_grouped_gemm(
        mode, _p(A), _p(a_scale), _p(B), _p(b_scale), _p(offsets), G, rows, M, N, K, dtype,
        _p(C), c_dtype, wp, wb, _stream(stream)))


def moe_grouped_gemm_swiglu_bwd(d_out, w_down, offsets, gu_saved, dgu, stream=None):
    rows, H = d_out.shape
    G, I, _ = w_down.shape
    _want(gu_saved, torch.bfloat16, (rows, 2 * I), "gu_saved")
    _want(dgu, torch.bfloat16, (rows, 2 * I), "dgu")
    _check("moe_grouped_gemm_swiglu_bwd", _lib.moe_grouped_gemm_swiglu_bwd(
        _p(d_out), _p(w_down), _p(offsets), _p(gu_saved), G, rows, H, I, _p(dgu),
        _stream(stream)))


def moe_set_gemm_max_blocks(max_blocks):
    """Cap the persistent grid of the grouped-GEMM launches (0: every resident block)."""
    _check("moe_set_gemm_max_blocks", _lib.moe_set_gemm_max_blocks(int(max_blocks)))


def moe_unpermute_combine(y_perm, row_of, topk_prob, y, shared_out=None, stream=None):
    T, k = row_of.shape
    H = y.shape[1]
    _want_rows(y_perm, torch.bfloat16, T * k, H, "y_perm")
    _want(y, torch.bfloat16, (T, H), "y")
    _check("moe_unpermute_combine", _lib.moe_unpermute_combine(
        _p(y_perm), _p(row_of), _p(topk_prob), _p(shared_out), T, H, k, _p(y), _stream(stream)))


def moe_combine_backward(dy, row_of, topk_prob, d_out, stream=None):
    T, k = row_of.shape
    H = dy.shape[1]
    _want_rows(d_out, torch.bfloat16, T * k, H, "d_out")
    _check("moe_combine_backward", _lib.moe_combine_backward(
        _p(dy), _p(row_of), _p(topk_prob), T, H, k, _p(d_out), _stream(stream)))


def moe_quantize_mxfp8_rows(x, q, scale, stream=None):
    R, C = x.shape
    _want(x, torch.bfloat16, (R, C), "x")
    _want(q, torch.uint8, (R, C), "q")
    _want(scale, torch.uint8, (R, C // 32), "scale")
    _check("moe_quantize_mxfp8_rows", _lib.moe_quantize_mxfp8_rows(
        _p(x), R, C, _p(q), _p(scale), _stream(stream)))


def moe_quantize_mxfp8_weights(w, q, scale, stream=None):
    G, K, N = w.shape
    _want(w, torch.bfloat16, (G, K, N), "w")
    _want(q, torch.uint8, (G, N, K), "q")
    _want(scale, torch.uint8, (G, N, K // 32), "scale")
    _check("moe_quantize_mxfp8_weights", _lib.moe_quantize_mxfp8_weights(
        _p(w), G, K, N, _p(q), _p(scale), _stream(stream)))


def moe_grouped_gemm_mxfp8(A, a_scale, B, b_scale, offsets, C, swiglu=False, stream=None):
    rows, K = A.shape
    G, N, _ = B.shape
    _want(A, torch.uint8, (rows, K), "A")
    _want(a_scale, torch.uint8, (rows, K // 32), "a_scale")
    _want(B, torch.uint8, (G, N, K), "B")
    _want(b_scale, torch.uint8, (G, N, K // 32), "b_scale")
    _want(offsets, torch.int32, (G + 1,), "offsets")
    _want(C, torch.bfloat16, (rows, N // 2 if swiglu else N), "C")
    _check("moe_grouped_gemm_mxfp8", _lib.moe_grouped_gemm_mxfp8(
        _p(A), _p(a_scale), _p(B), _p(b_scale), _p(offsets), G, rows, N, K, int(bool(swiglu)),
        _p(C), _stream(stream)))


def moe_mxfp8_cols_capacity(R, G):
    n = _lib.moe_mxfp8_cols_capacity(int(R), int(G))
    if n < 0:
        raise MoeError("moe_mxfp8_cols_capacity", 1)
    return n


def moe_mxfp8_col_offsets(offsets, col_offsets, stream=None):
    G = offsets.numel() - 1
    _want(offsets, torch.int32, (G + 1,), "offsets")
    _want(col_offsets, torch.int32, (G + 1,), "col_offsets")
    _check("moe_mxfp8_col_offsets", _lib.moe_mxfp8_col_offsets(
        _p(offsets), G, _p(col_offsets), _stream(stream)))


def moe_quantize_mxfp8_cols(x, offsets, col_offsets, qt, scale_t, stream=None):
    R, C = x.shape
    G = offsets.numel() - 1
    Kp = qt.shape[1]
    _want(x, torch.bfloat16, (R, C), "x")
    _want(offsets, torch.int32, (G + 1,), "offsets")
    _want(col_offsets, torch.int32, (G + 1,), "col_offsets")
    _want(qt, torch.uint8, (C, Kp), "qt")
    _want(scale_t, torch.uint8, (C, Kp // 32), "scale_t")
    _check("moe_quantize_mxfp8_cols", _lib.moe_quantize_mxfp8_cols(
        _p(x), R, C, _p(offsets), _p(col_offsets), G, Kp, _p(qt), _p(scale_t), _stream(stream)))


def moe_grouped_gemm_mxfp8_wgrad(At, a_scale, Bt, b_scale, col_offsets, C, stream=None):
    M, Kp = At.shape
    N = Bt.shape[0]
    G = col_offsets.numel() - 1
    _want(At, torch.uint8, (M, Kp), "At")
    _want(a_scale, torch.uint8, (M, Kp // 32), "a_scale")
    _want(Bt, torch.uint8, (N, Kp), "Bt")
    _want(b_scale, torch.uint8, (N, Kp // 32), "b_scale")
    _want(col_offsets, torch.int32, (G + 1,), "col_offsets")
    _want(C, torch.bfloat16, (G, M, N), "C")
    _check("moe_grouped_gemm_mxfp8_wgrad", _lib.moe_grouped_gemm_mxfp8_wgrad(
        _p(At), _p(a_scale), _p(Bt), _p(b_scale), _p(col_offsets), G, M, N, Kp, _p(C),
        _stream(stream)))


def moe_grouped_gemm_mxfp8_swiglu_bwd(A, a_scale, B, b_scale, offsets, gu, dgu, stream=None):
    rows, K = A.shape
    G, I, _ = B.shape
    _want(A, torch.uint8, (rows, K), "A")
    _want(a_scale, torch.uint8, (rows, K // 32), "a_scale")
    _want(B, torch.uint8, (G, I, K), "B")
    _want(b_scale, torch.uint8, (G, I, K // 32), "b_scale")
    _want(offsets, torch.int32, (G + 1,), "offsets")
    _want(gu, torch.bfloat16, (rows, 2 * I), "gu")
    _want(dgu, torch.bfloat16, (rows, 2 * I), "dgu")
    _check("moe_grouped_gemm_mxfp8_swiglu_bwd", _lib.moe_grouped_gemm_mxfp8_swiglu_bwd(
        _p(A), _p(a_scale), _p(B), _p(b_scale), _p(offsets), G, rows, I, K, _p(gu), _p(dgu),
        _stream(stream)))


def moe_quantize_fp8_rows(x, q, scale, stream=None):
    R, C = x.shape
    _want(q, torch.uint8, (R, C), "q")
    _want(scale, torch.float32, (R,), "scale")
    _check("moe_quantize_fp8_rows", _lib.moe_quantize_fp8_rows(
        _p(x), R, C, _p(q), _p(scale), _stream(stream)))


def moe_quantize_fp8_weights(w, q, scale, stream=None):
    G, K, N = w.shape
    _want(q, torch.uint8, (G, N, K), "q")
    _want(scale, torch.float32, (G, N), "scale")
    _check("moe_quantize_fp8_weights", _lib.moe_quantize_fp8_weights(
        _p(w), G, K, N, _p(q), _p(scale), _stream(stream)))


def moe_router_logits(x, w_router, logits, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    _want(x, torch.bfloat16, (T, H), "x")
    _want(w_router, torch.bfloat16, (E, H), "w_router")
    _want(logits, torch.float32, (T, E), "logits")
    _check("moe_router_logits", _lib.moe_router_logits(
        _p(x), _p(w_router), T, H, E, _p(logits), _stream(stream)))


def moe_combine_backward_router(dy, expert_out, row_of, topk_idx, topk_prob, score, d_out,
                                d_logits, d_prob=None, scaling_factor=1.0, logits=None,
                                stream=None):
    T, k = row_of.shape
    H = dy.shape[1]
    E = d_logits.shape[1]
    _want(dy, torch.bfloat16, (T, H), "dy")
    _want_rows(expert_out, torch.bfloat16, T * k, H, "expert_out")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(topk_prob, torch.float32, (T, k), "topk_prob")
    _want_rows(d_out, torch.bfloat16, T * k, H, "d_out")
    _want(d_logits, torch.float32, (T, E), "d_logits")
    if d_prob is not None:
        _want(d_prob, torch.float32, (T, k), "d_prob")
    if logits is not None:
        _want(logits, torch.float32, (T, E), "logits")
    _check("moe_combine_backward_router", _lib.moe_combine_backward_router(
        _p(dy), _p(expert_out), _p(row_of), _p(topk_idx), _p(topk_prob), _p(logits), T, H, E, k,
        _score(score), float(scaling_factor), _p(d_out), _p(d_prob), _p(d_logits),
        _stream(stream)))


def moe_router_weight_grad_workspace_bytes(T, H, E):
    return int(_lib.moe_router_weight_grad_workspace_bytes(T, H, E))


def moe_router_weight_grad(x, d_logits, dw_router, ws, stream=None):
    T, H = x.shape
    E = d_logits.shape[1]
    _want(x, torch.bfloat16, (T, H), "x")
    _want(d_logits, torch.float32, (T, E), "d_logits")
    _want(dw_router, torch.float32, (E, H), "dw_router")
    _check("moe_router_weight_grad", _lib.moe_router_weight_grad(
        _p(x), _p(d_logits), T, H, E, _p(dw_router), _p(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_dispatch_backward_router(dxp, row_of, topk_idx, d_logits, w_router, dx, stream=None):
    T, k = row_of.shape
    E, H = w_router.shape
    _want_rows(dxp, torch.bfloat16, T * k, H, "dxp")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(d_logits, torch.float32, (T, E), "d_logits")
    _want(dx, torch.bfloat16, (T, H), "dx")
    _check("moe_dispatch_backward_router", _lib.moe_dispatch_backward_router(
        _p(dxp), _p(row_of), _p(topk_idx), _p(d_logits), _p(w_router), T, H, E, k, _p(dx),
        _stream(stream)))


def moe_dispatch_backward_router_input(dxp, x, row_of, topk_idx, topk_prob, w_router, score, dx,
                                       d_logits, scaling_factor=1.0, logits=None, stream=None):
    T, k = row_of.shape
    E, H = w_router.shape
    _want_rows(dxp, torch.bfloat16, T * k, H, "dxp")
    _want(x, torch.bfloat16, (T, H), "x")
    _want(topk_prob, torch.float32, (T, k), "topk_prob")
    _want(dx, torch.bfloat16, (T, H), "dx")
    _want(d_logits, torch.float32, (T, E), "d_logits")
    if logits is not None:
        _want(logits, torch.float32, (T, E), "logits")
    _check("moe_dispatch_backward_router_input", _lib.moe_dispatch_backward_router_input(
        _p(dxp), _p(x), _p(row_of), _p(topk_idx), _p(topk_prob), _p(logits), _p(w_router), T, H,
        E, k,
        _score(score), float(scaling_factor), _p(dx), _p(d_logits), _stream(stream)))


# ---- ScaledSwiGLU ------------------------------------------------------------------------------

def moe_permute_probs(row_of, topk_prob, row_prob, stream=None):
    T, k = row_of.shape
    _want(topk_prob, torch.float32, (T, k), "topk_prob")
    if row_prob.dtype != torch.float32 or row_prob.dim() != 1 or row_prob.shape[0] < T * k:
        raise ValueError("row_prob: expected float32 [>= T*k]")
    _check("moe_permute_probs", _lib.moe_permute_probs(
        _p(row_of), _p(topk_prob), T, k, _p(row_prob), _stream(stream)))


def moe_grouped_gemm_swiglu_scaled(xp, w_gu, offsets, row_scale, h, gu_saved=None, stream=None):
    rows, H = xp.shape
    G, _, I2 = w_gu.shape
    I = I2 // 2
    _want(xp, torch.bfloat16, (rows, H), "xp")
    _want(w_gu, torch.bfloat16, (G, H, 2 * I), "w_gu")
    _want(offsets, torch.int32, (G + 1,), "offsets")
    _want(row_scale, torch.float32, (rows,), "row_scale")
    _want(h, torch.bfloat16, (rows, I), "h")
    if gu_saved is not None:
        _want(gu_saved, torch.bfloat16, (rows, 2 * I), "gu_saved")
    _check("moe_grouped_gemm_swiglu_scaled", _lib.moe_grouped_gemm_swiglu_scaled(
        _p(xp), _p(w_gu), _p(offsets), _p(row_scale), G, rows, H, I, _p(h), _p(gu_saved),
        _stream(stream)))


def moe_grouped_gemm_swiglu_scaled_bwd(d_out, w_down, offsets, gu_saved, row_scale, dgu,
                                       d_scale_part=None, stream=None):
    rows, H = d_out.shape
    G, I, _ = w_down.shape
    _want(d_out, torch.bfloat16, (rows, H), "d_out")
    _want(w_down, torch.bfloat16, (G, I, H), "w_down")
    _want(offsets, torch.int32, (G + 1,), "offsets")
    _want(gu_saved, torch.bfloat16, (rows, 2 * I), "gu_saved")
    _want(row_scale, torch.float32, (rows,), "row_scale")
    _want(dgu, torch.bfloat16, (rows, 2 * I), "dgu")
    if d_scale_part is not None:
        _want(d_scale_part, torch.float32, (rows, I // 64), "d_scale_part")
    _check("moe_grouped_gemm_swiglu_scaled_bwd", _lib.moe_grouped_gemm_swiglu_scaled_bwd(
        _p(d_out), _p(w_down), _p(offsets), _p(gu_saved), _p(row_scale), G, rows, H, I, _p(dgu),
        _p(d_scale_part), _stream(stream)))


def moe_dispatch_backward_router_scaled(dxp, d_scale_part, row_of, topk_idx, topk_prob, w_router,
                                        I, score, dx, d_logits, scaling_factor=1.0, logits=None,
                                        stream=None):
    T, k = row_of.shape
    E, H = w_router.shape
    _want_rows(dxp, torch.bfloat16, T * k, H, "dxp")
    _want_rows(d_scale_part, torch.float32, T * k, I // 64, "d_scale_part")
    _want(topk_idx, torch.int32, (T, k), "topk_idx")
    _want(topk_prob, torch.float32, (T, k), "topk_prob")
    _want(dx, torch.bfloat16, (T, H), "dx")
    _want(d_logits, torch.float32, (T, E), "d_logits")
    _check("moe_dispatch_backward_router_scaled", _lib.moe_dispatch_backward_router_scaled(
        _p(dxp), _p(d_scale_part), _p(row_of), _p(topk_idx), _p(topk_prob), _p(logits),
        _p(w_router), T, H, E, k, I, _score(score), float(scaling_factor), _p(dx), _p(d_logits),
        _stream(stream)))


# ---- auxiliary load-balancing loss ----------------------------------------------------------

def moe_aux_loss_scores(logits, k, score, scores, routing_map=None, stream=None):
    T, E = logits.shape
    _want(logits, torch.float32, (T, E), "logits")
    _want(scores, torch.float32, (T, E), "scores")
    if routing_map is not None:
        _want(routing_map, torch.uint8, (T, E), "routing_map")
    _check("moe_aux_loss_scores", _lib.moe_aux_loss_scores(
        _p(logits), T, E, k, _score(score), _p(scores), _p(routing_map), _stream(stream)))


def moe_aux_loss_workspace_bytes(T, E):
    return int(_lib.moe_aux_loss_workspace_bytes(T, E))


def moe_aux_loss(scores, tokens_per_expert, k, total_num_tokens, coeff, loss, ws, stream=None):
    T, E = scores.shape
    _want(scores, torch.float32, (T, E), "scores")
    _want(tokens_per_expert, torch.int32, (E,), "tokens_per_expert")
    _want(loss, torch.float32, (1,), "loss")
    _check("moe_aux_loss", _lib.moe_aux_loss(
        _p(scores) if T else None, _p(tokens_per_expert), T, E, k, int(total_num_tokens),
        float(coeff), _p(loss), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_aux_loss_backward(logits, tokens_per_expert, k, total_num_tokens, coeff, score, d_logits,
                          d_loss=None, accumulate=False, stream=None):
    T, E = logits.shape
    _want(logits, torch.float32, (T, E), "logits")
    _want(tokens_per_expert, torch.int32, (E,), "tokens_per_expert")
    _want(d_logits, torch.float32, (T, E), "d_logits")
    if d_loss is not None:
        _want(d_loss, torch.float32, (1,), "d_loss")
    _check("moe_aux_loss_backward", _lib.moe_aux_loss_backward(
        _p(logits), _p(tokens_per_expert), T, E, k, int(total_num_tokens), float(coeff),
        _score(score), _p(d_loss), _p(d_logits), int(bool(accumulate)), _stream(stream)))


# ---- whole layer -----------------------------------------------------------------------

def problem(T, H, E, k, I, score, shared_I=0, dtype=MOE_BF16, training=False, router=False,
            num_groups=0, group_topk=0, scaling_factor=1.0, weight_placement=MOE_PLACE_COMBINE,
            align_size=0):
    return Problem(T, H, E, k, I, shared_I, _score(score), dtype, int(bool(training)),
                   int(bool(router)), int(num_groups), int(group_topk), float(scaling_factor),
                   int(weight_placement), int(align_size))


def moe_workspace_bytes(prob: Problem):
    n = int(_lib.moe_workspace_bytes(ctypes.byref(prob)))
    if n == 0:
        raise MoeError("moe_workspace_bytes", MOE_ERR_INVALID_ARG)
    return n


def moe_workspace_views(prob: Problem, ws):
    v = Views()
    _check("moe_workspace_views", _lib.moe_workspace_views(
        ctypes.byref(prob), _p(ws), ws.numel() * ws.element_size(), ctypes.byref(v)))
    return v


def tensors(x, logits, w_gu, w_down, y, w_gu_scale=None, w_down_scale=None, shared_gu=None,
            shared_down=None, w_router=None, dw_router=None, expert_bias=None, w_gu_bwd=None,
            w_gu_bwd_scale=None, w_down_bwd=None, w_down_bwd_scale=None):
    return Tensors(_p(x), _p(logits), _p(w_gu), _p(w_gu_scale), _p(w_down), _p(w_down_scale),
                   _p(shared_gu), _p(shared_down), _p(y), _p(w_router), _p(dw_router),
                   _p(expert_bias), _p(w_gu_bwd), _p(w_gu_bwd_scale), _p(w_down_bwd),
                   _p(w_down_bwd_scale))


def moe_forward(prob: Problem, tens: Tensors, ws, stream=None):
    _check("moe_forward", _lib.moe_forward(
        ctypes.byref(prob), ctypes.byref(tens), _p(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_backward(prob: Problem, tens: Tensors, dy, dx, dw_gu, dw_down, ws, stream=None):
    _check("moe_backward", _lib.moe_backward(
        ctypes.byref(prob), ctypes.byref(tens), _p(dy), _p(dx), _p(dw_gu), _p(dw_down), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def view_tensor(ptr, shape, dtype, like):
    """A torch tensor aliasing device memory at ``ptr`` inside a workspace tensor ``like``."""
    base = like.data_ptr()
    nbytes = int(torch.tensor([], dtype=dtype).element_size())
    off = int(ptr) - base
    count = 1
    for s in shape:
        count *= s
    if off < 0 or off + count * nbytes > like.numel() * like.element_size():
        raise ValueError("view outside the workspace")
    flat = like.view(torch.uint8)[off: off + count * nbytes]
    return flat.view(dtype).view(*shape)
