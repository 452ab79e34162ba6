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
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_void_p]
    NN, NT, BF16 = 0, 1, 0
    for mode in (NN, NT):
        assert gg(mode, None, None, None, None, None, 8, 16, 0, 65536, 32768, BF16, None, BF16, None, 0, None) == 2
        assert gg(mode, None, None, None, None, None, 8, 16, 0, 65536, 32704, BF16, None, BF16, None, 0, None) == 1
    sw = lib.moe_grouped_gemm_swiglu
    sw.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    assert sw(None, None, None, None, None, 8, 16, 32768, 32768, BF16, None, None, None, 0, None) == 2
    assert sw(None, None, None, None, None, 8, 16, 32704, 32768, BF16, None, None, None, 0, None) == 1


def test_splitk_space_only_for_decode_shapes(lib):
    # split-K space: part count at offset 0, then 8 parts of [rows, ncols] fp32; only shapes
    # of at most 256 rows and 32 rows per group on average split
    f = lib.moe_grouped_gemm_splitk_workspace_bytes
    f.argtypes, f.restype = [ctypes.c_int] * 3, ctypes.c_size_t
    assert f(48, 16, 640) == 256 + 8 * 48 * 640 * 4
    assert f(256, 8, 128) == 256 + 8 * 256 * 128 * 4
    assert f(257, 16, 640) == 0 and f(200, 4, 640) == 0 and f(0, 4, 640) == 0 and f(8, 0, 64) == 0


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


_SIZE_SWEEP = r"""
import itertools, sys
import mixture_experts_layer_amd as M
Ts = (0, 1, 2, 31, 32, 33, 257, 4096, 8193, 65536)
variants = []
for training, router, placement, align, dtype, shared in itertools.product(
        (False, True), (False, True), (M.MOE_PLACE_COMBINE, M.MOE_PLACE_INPUT, M.MOE_PLACE_ACTIVATION),
        (0, 128), (M.MOE_BF16, M.MOE_FP8_E4M3, M.MOE_MXFP8), (0, 192)):
    if dtype == M.MOE_FP8_E4M3 and training:
        continue
    variants.append(dict(training=training, router=router, weight_placement=placement,
                         align_size=align, dtype=dtype, shared_I=shared))
for v in variants:
    sizes = []
    for T in Ts:
        print(T, v, flush=True)
        sizes.append(int(M.lib().moe_workspace_bytes(M.ctypes.byref(M.problem(T, 256, 16, 4, 192, 0, **v)))))
    # a combination the layer does not take gets 0 for every T; any other, a size for every T
    assert all(n == 0 for n in sizes) or all(n > 0 for n in sizes), (v, sizes)
for T in Ts:
    for E, k in ((8, 2), (128, 8), (256, 32)):
        assert M.moe_permute_workspace_bytes(T, E, k) > 0
        assert M.moe_aux_loss_workspace_bytes(T, E) > 0
        assert M.moe_grouped_gemm_splitk_workspace_bytes(T, E, 256) >= 0
print("sizes ok", flush=True)
"""


def test_workspace_sizes_for_every_token_count():
    # host-only size queries answer for every token count, T = 0 included (no division by
    # a zero chunk size)
    r = subprocess.run([sys.executable, "-c", _SIZE_SWEEP], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-5:])
    assert r.returncode == 0 and "sizes ok" in r.stdout, tail


def test_routed_rows_beyond_int32_are_refused(lib):
    # row ids and offsets are int32: with a narrow hidden size the routed rows T*k can pass
    # the T*k*H bound and still overflow them; every shape check refuses such a T before
    # touching a pointer (MOE_ERR_UNSUPPORTED = 2)
    import mixture_experts_layer_amd as M
    T, H, E, k = 1 << 26, 64, 256, 32          # T*k = 2^31 rows, T*k*H = 2^37
    assert lib.moe_router_topk(None, T, E, k, 0, None, None, None, None, None, None) == 2
    assert lib.moe_permute(None, None, T, H, E, k, 0, None, None, None, None, None, None, 0,
                           None) == 2
    assert lib.moe_unpermute_combine(None, None, None, None, T, H, k, None, None) == 2
    assert lib.moe_combine_backward(None, None, None, T, H, k, None, None) == 2
    assert lib.moe_permute_probs(None, None, T, k, None, None) == 2
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    assert lib.moe_workspace_bytes(ctypes.byref(M.problem(T, H, E, k, 64, 0))) == 0
    # just inside the bound the size query answers
    T_ok = (0x7fffffff - 256 * 4095) // (k + 1)
    assert lib.moe_workspace_bytes(ctypes.byref(M.problem(T_ok, H, E, k, 64, 0))) > 0
    assert lib.moe_workspace_bytes(ctypes.byref(M.problem(T_ok + 1, H, E, k, 64, 0))) == 0


def test_workspace_views_inside_an_exact_size(lib):
    # random mostly-valid layer problems (host-only calls): the workspace size is exact (one
    # byte less is MOE_ERR_WORKSPACE = 3) and every view the layer uses lies inside it
    import random
    import mixture_experts_layer_amd as M
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    rng = random.Random(7)
    base, accepted = 1 << 40, 0
    for _ in range(3000):
        E = rng.choice([1, 2, 4, 8, 16, 40, 64, 128, 256])
        k = rng.randint(1, min(E, 32))
        dtype = rng.choice([0, 0, 1, 3])
        ng = rng.choice([0, 0, 1, 2, 4, 8])
        p = M.Problem(rng.choice([0, 1, 2, 7, 31, 32, 33, 256, 257, 4096, 8193, 65536]),
                      64 * rng.randint(1, 80), E, k, 64 * rng.randint(1, 40),
                      rng.choice([0, 0, 64, 128]), rng.choice([0, 1, 2, 3, 4]), dtype,
                      0 if dtype == 1 else rng.choice([0, 1]), rng.choice([0, 1]), ng,
                      rng.randint(1, ng) if ng > 1 else 0, rng.choice([0.0, 1.0, 2.5]),
                      rng.choice([0, 1, 2]), rng.choice([0, 0, 1, 8, 64, 128]))
        b = lib.moe_workspace_bytes(ctypes.byref(p))
        if not b:
            continue
        accepted += 1
        v = M.Views()
        assert lib.moe_workspace_views(ctypes.byref(p), ctypes.c_void_p(base), ctypes.c_size_t(b),
                                       ctypes.byref(v)) == 0
        assert lib.moe_workspace_views(ctypes.byref(p), ctypes.c_void_p(base),
                                       ctypes.c_size_t(b - 1), ctypes.byref(v)) == 3
        for name, ftype in M.Views._fields_:
            ptr = getattr(v, name)
            if ftype is ctypes.c_void_p and ptr:
                assert base <= ptr < base + b, (name, hex(ptr), b)
    assert accepted > 500
