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


# decode steps of one or two tokens, whose expert GEMMs split over K (partial sums in the
# workspace, then a second launch): inference with a shared expert, and a training step
SPLIT = {
    "dec_split_shared": W.custom("dec_split_shared", T=2, H=1024, E=16, k=1, I=512, score=W.SIGMOID,
                                 shared_I=512),
    "dec_split_train": W.custom("dec_split_train", T=2, H=768, E=16, k=2, I=256, training=True),
}


@pytest.mark.parametrize("name", ["qwen3", "llama4", "dec_split_shared", "dec_split_train"])
def test_graph_replay_matches_eager(name):
    w = SPLIT[name] if name in SPLIT else W.WORKLOADS[name]
    _say("graph", name)
    d = W.make_inputs(w)
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


def test_two_layers_on_two_streams_and_a_replay():
    """Two layers with their own workspaces step at the same time on two streams, then one
    of them as a graph replay beside eager steps of the other. Each keeps its grouped-GEMM
    tile counters in its own workspace (the workspaces start filled with 0xFF: the forward's
    dispatch zeroes the counters), so every output must still equal the single-stream run
    bit for bit."""
    w = W.WORKLOADS["qwen3"]
    _say("two streams", w.name)
    d = W.make_inputs("qwen3")
    layers = [GpuMoE(w, d), GpuMoE(w, d)]

    def step(g):
        M.moe_forward(g.prob, g.tens, g.ws)
        M.moe_backward(g.prob, g.tens, g.dy, g.dx, g.dw_gu, g.dw_down, g.ws)

    def outs(g):
        return [g.y, g.dx, g.dw_gu, g.dw_down]

    for g in layers:  # allocates each layer's gradient buffers
        g.forward()
        g.backward(d["dy"])
    ref = [_bits(t) for t in outs(layers[0])]
    torch.cuda.synchronize()

    def check(label):
        for g in layers:
            for t, r, name in zip(outs(g), ref, ["y", "dx", "dw_gu", "dw_down"]):
                assert np.array_equal(_bits(t), r), f"{label}: {name} differs from the single-stream run"

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(6):
        for g, s in zip(layers, streams):
            with torch.cuda.stream(s):
                step(g)
    torch.cuda.synchronize()
    check("two streams")

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(layers[0])  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(layers[0])
    torch.cuda.synchronize()
    for r in range(3):
        for g in layers:
            for t in outs(g):
                t.view(torch.int16).fill_(0x7FC0 + r)
        torch.cuda.synchronize()
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(streams[0]):
            graph.replay()
        with torch.cuda.stream(streams[1]):
            for _ in range(2):
                step(layers[1])
        torch.cuda.synchronize()
        check(f"replay {r} beside eager steps")
    del graph
