"""GPU test of moe_permute_noalloc (through the C ABI): the dispatch with its scratch in the
library's device array must give the results of moe_permute with a caller workspace, bit
for bit, on two calls in a row (the second smaller, so stale scratch from the first call
is present), in bf16 and in e4m3; sizes past the array are refused before any launch."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import oracle as O
from gpu_helpers import dev, dev_bf16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(rng, T, H, E, k):
    x = O.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = O.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
    return x, idx


def _both(x, idx, E, out_dtype):
    T, H = x.shape
    k = idx.shape[1]
    xd, idd = dev_bf16(x), dev(idx)
    res = []
    for noalloc in (False, True):
        act = torch.uint8 if out_dtype == M.MOE_FP8_E4M3 else torch.bfloat16
        xp = torch.full((T * k, H), 0x55, dtype=torch.uint8, device="cuda").view(act) \
            if act == torch.uint8 else torch.full((T * k, H), float("nan"), dtype=act, device="cuda")
        xs = torch.full((T * k,), float("nan"), device="cuda") if out_dtype == M.MOE_FP8_E4M3 else None
        offs = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
        row_of = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
        src_of = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            M.moe_permute_noalloc(xd, idd, E, xp, offs, row_of, src_of, out_dtype, xs)
        else:
            ws = torch.empty(M.moe_permute_workspace_bytes(T, E, k), dtype=torch.uint8,
                             device="cuda")
            M.moe_permute(xd, idd, E, xp, offs, row_of, src_of, ws, out_dtype, xs)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (xp.view(torch.uint8), offs, row_of, src_of)] +
                   ([xs.cpu()] if xs is not None else []))
    return res


@pytest.mark.parametrize("out_dtype", [M.MOE_BF16, M.MOE_FP8_E4M3])
def test_permute_noalloc_matches_permute(out_dtype):
    rng = np.random.default_rng(0)
    # a large dispatch, then a smaller one over the stale scratch
    for T, H, E, k in ((4096, 256, 128, 8), (300, 128, 16, 4)):
        _say("noalloc permute", T, H, E, k, out_dtype)
        x, idx = _inputs(rng, T, H, E, k)
        ref, got = _both(x, idx, E, out_dtype)
        for a, b, name in zip(ref, got, ("xp", "offsets", "row_of", "src_of", "xp_scale")):
            assert torch.equal(a, b), (T, name)
        # and the layout is the oracle's
        offs, row_of, src_of = O.dispatch_meta(idx, E)
        assert np.array_equal(got[1].numpy(), offs) and np.array_equal(got[2].numpy(), row_of)


def test_permute_noalloc_refuses_oversized_scratch():
    lim = M.moe_permute_noalloc_limit()
    assert lim == 4 << 20
    T, H, E, k = 65536, 64, 256, 16      # 1 M routed rows: scratch above the limit
    assert M.moe_permute_workspace_bytes(T, E, k) > lim
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    xp = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    with pytest.raises((M.MoeError, ValueError)):
        M.moe_permute_noalloc(x, idx, E, xp, offs, torch.empty((T, k), dtype=torch.int32,
                                                               device="cuda"),
                              torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    # the C entry point itself reports MOE_ERR_UNSUPPORTED before any launch
    st = M._lib.moe_permute_noalloc(M._p(x), M._p(idx), T, H, E, k, M.MOE_BF16, M._p(x), None,
                                    M._p(offs), M._p(idx), M._p(idx), None)
    assert st == M.MOE_ERR_UNSUPPORTED
