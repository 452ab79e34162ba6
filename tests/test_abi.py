"""The C-ABI library loads on a machine without a GPU and exports every entry point
that include/moe_amd.h declares; host-only entry points answer without touching a GPU."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_amd.h")
LIB = os.path.join(ROOT, "mixture_experts_layer_amd", "libmoe_amd.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:long\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (loads the HIP runtime the library links against)
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, "mixture_experts_layer_amd", "_build.py")],
                       cwd=ROOT, check=True)
    return ctypes.CDLL(LIB)


def test_header_declares_entry_points():
    names = declared()
    for must in ("moe_router_topk", "moe_permute", "moe_grouped_gemm_swiglu", "moe_grouped_gemm",
                 "moe_grouped_gemm_swiglu_bwd", "moe_unpermute_combine", "moe_combine_backward",
                 "moe_forward", "moe_backward", "moe_workspace_bytes"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_the_header(lib):
    import mixture_experts_layer_amd as M
    assert sorted(M.EXPORTS) == declared()
    for n in M.EXPORTS:
        assert callable(getattr(M, n))


def test_host_only_entry_points(lib):
    lib.moe_status_str.restype = ctypes.c_char_p
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(1) == b"MOE_ERR_INVALID_ARG"
    lib.moe_permute_workspace_bytes.restype = ctypes.c_size_t
    assert lib.moe_permute_workspace_bytes(4096, 128, 8) > 0
    assert lib.moe_set_gemm_max_blocks(-1) == 1
    assert lib.moe_set_gemm_max_blocks(0) == 0
    # argument validation answers before any device work
    assert lib.moe_router_topk(None, 4, 8, 2, 0, None, None, None, None, None, None) == 1


def test_gemm_size_limits_answer_before_device_work(lib):
    # one expert's weight matrix of 4 GiB or more is refused (the kernels address it with
    # 32-bit offsets); sizes just under the limit pass the size checks and stop at the
    # pointer checks
    gg = lib.moe_grouped_gemm
    gg.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    NN, NT, BF16 = 0, 1, 0
    for mode in (NN, NT):
        assert gg(mode, None, None, None, None, None, 8, 16, 0, 65536, 32768, BF16, None, BF16, None) == 2
        assert gg(mode, None, None, None, None, None, 8, 16, 0, 65536, 32704, BF16, None, BF16, None) == 1
    sw = lib.moe_grouped_gemm_swiglu
    sw.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    assert sw(None, None, None, None, None, 8, 16, 32768, 32768, BF16, None, None, None) == 2
    assert sw(None, None, None, None, None, 8, 16, 32704, 32768, BF16, None, None, None) == 1


def test_router_entry_points_validate_on_the_host(lib):
    lib.moe_router_weight_grad_workspace_bytes.restype = ctypes.c_size_t
    # split operand [T, 2E padded to 64] bf16 plus 16 K splits of [2E.., H] fp32 partials
    assert lib.moe_router_weight_grad_workspace_bytes(4096, 2048, 128) == 4096 * 256 * 2 + 16 * 256 * 2048 * 4
    assert lib.moe_router_weight_grad_workspace_bytes(4096, 100, 128) == 0   # H % 64
    assert lib.moe_router_weight_grad_workspace_bytes(64, 128, 300) == 0     # E > 256
    # null pointers and unsupported sizes answer before any device work
    assert lib.moe_router_logits(None, None, 8, 128, 4, None, None) == 1
    assert lib.moe_router_logits(None, None, 8, 100, 4, None, None) == 2
    assert lib.moe_dispatch_backward_router(None, None, None, None, None, 8, 128, 4, 2, None, None) == 1


def test_mxfp8_backward_entry_points_validate_on_the_host(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    cap = lib.moe_mxfp8_cols_capacity
    cap.argtypes, cap.restype = [i, i], ctypes.c_longlong
    # every expert's range rounded up to 64 columns: at most R + 63 G, rounded to 64
    assert cap(0, 1) == 64 and cap(1, 1) == 64 and cap(64, 1) == 128 and cap(32768, 128) == 40832
    assert cap(-1, 4) == -1 and cap(10, 0) == -1
    fake = vp(0x1000)
    co = lib.moe_mxfp8_col_offsets
    co.argtypes = [vp, i, vp, vp]
    assert co(None, 4, fake, None) == 1 and co(fake, 0, fake, None) == 1
    qc = lib.moe_quantize_mxfp8_cols
    qc.argtypes = [vp, i, i, vp, vp, i, i, vp, vp, vp]
    assert qc(fake, 100, 64, fake, fake, 4, 64, fake, fake, None) == 1     # Kp below capacity
    assert qc(fake, 100, 64, fake, fake, 4, 448 + 32, fake, fake, None) == 2  # Kp % 64
    assert qc(fake, 100, 60, fake, fake, 4, 448, fake, fake, None) == 2    # C % 8
    assert qc(fake, 100, 64, None, fake, 4, 448, fake, fake, None) == 1    # no offsets
    wg = lib.moe_grouped_gemm_mxfp8_wgrad
    wg.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, vp]
    assert wg(fake, fake, fake, fake, fake, 4, 96, 64, 448, fake, None) == 2   # M % 64
    assert wg(fake, fake, fake, fake, fake, 4, 64, 64, 480, fake, None) == 2   # Kp % 64
    assert wg(fake, None, fake, fake, fake, 4, 64, 64, 448, fake, None) == 1   # no scales
    sb = lib.moe_grouped_gemm_mxfp8_swiglu_bwd
    sb.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp]
    assert sb(fake, fake, fake, fake, fake, 4, 100, 96, 256, fake, fake, None) == 2  # I % 64
    assert sb(fake, fake, fake, fake, fake, 4, 100, 64, 200, fake, fake, None) == 2  # K % 64
    assert sb(fake, fake, fake, fake, fake, 4, 100, 64, 256, None, fake, None) == 1  # no g,u
    assert sb(fake, fake, fake, fake, fake, 4, 0, 64, 256, fake, fake, None) == 0    # no rows
