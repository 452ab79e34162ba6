"""The layer's forward + backward captured in one HIP graph and replayed.

Every launch takes its sizes from arguments and its expert row counts from device
memory, with no host synchronisation, allocation or memset inside, so the whole step can
be recorded once and replayed. Each replay must reproduce the eager run bit for bit:
no value depends on the order in which blocks run (the grouped GEMM's dynamic tile
tickets only decide which block computes a tile, never how). Between replays the outputs
are overwritten by eager kernels, so a replay that skipped or reused work shows up.
"""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from gpu_helpers import GpuMoE

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().copy()


@pytest.mark.parametrize("name", ["qwen3", "llama4"])
def test_graph_replay_matches_eager(name):
    w = W.WORKLOADS[name]
    _say("graph", name)
    d = W.make_inputs(name)
    g = GpuMoE(w, d)
    g.forward()
    outs = [g.y]
    if g.training:
        g.backward(d["dy"])
        outs += [g.dx, g.dw_gu, g.dw_down]
    eager = [_bits(t) for t in outs]

    def step():
        M.moe_forward(g.prob, g.tens, g.ws)
        if g.training:
            M.moe_backward(g.prob, g.tens, g.dy, g.dx, g.dw_gu, g.dw_down, g.ws)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs:  # eager work between replays: NaN patterns over every output
            t.view(torch.int16).fill_(0x7FC0 + r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, ref, label in zip(outs, eager, ["y", "dx", "dw_gu", "dw_down"]):
            assert np.array_equal(_bits(t), ref), f"{name} replay {r}: {label} differs from the eager run"
    del graph
