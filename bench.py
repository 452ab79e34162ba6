#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path on one MI355X.

Default workload: the Qwen3-30B-A3B-shaped MoE block, forward + backward
(T=4096 tokens, hidden 2048, 128 experts, top-8, expert width 768, bf16), synthetic
seeded inputs resident in HBM. One step = moe_forward + moe_backward through the C ABI
(router, dispatch, grouped SwiGLU MLP, combine, and the expert-path backward).

Prints one JSON line: whole-layer tokens/s, grouped-GEMM TFLOP/s, a roofline entry for
the dominant kernel (timed with HIP events on the launch stream), and the CPU oracle
timed on a bounded token sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense matrix-core peaks


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_costs(w, training, active=None, mx=False):
    """Algorithmic FLOPs and HBM bytes of each GEMM launch (read every input once,
    write every output once). Weights are counted for the `active` experts (those that
    received rows; all E by default): an expert with no rows has no tiles. mx: every GEMM
    operand is e4m3 (the scale bytes, 1/32 more, are not counted); outputs stay bf16."""
    N, H, I = w.T * w.k, w.H, w.I
    E = w.E if active is None else active
    act = 1 if (w.fp8 or mx) else 2
    q = 1 if mx else 2  # backward GEMM operands
    c = {
        "gemm1_swiglu": (2.0 * N * H * 2 * I,
                         N * H * act + E * H * 2 * I * act + N * I * 2 + (N * 2 * I * 2 if training else 0)),
        "gemm2": (2.0 * N * I * H, N * I * act + E * I * H * act + N * H * 2),
    }
    if training:
        c.update({
            "gemm2_bwd_swiglu": (2.0 * N * H * I, N * H * q + E * I * H * q + 2 * N * 2 * I * 2),
            "dw_down": (2.0 * N * I * H, N * I * q + N * H * q + E * I * H * 2),
            "gemm1_bwd_dx": (2.0 * N * 2 * I * H, N * 2 * I * q + E * H * 2 * I * q + N * H * 2),
            "dw_gu": (2.0 * N * H * 2 * I, N * H * q + N * 2 * I * q + E * H * 2 * I * 2),
        })
    return c


def row_costs(w, training, router=False):
    """Algorithmic bytes of the row-movement launches (with the router projection, the
    combine backward also reads the expert outputs and writes d_logits, and the dispatch
    backward also reads d_logits and the router weight)."""
    T, N, H, k, E = w.T, w.T * w.k, w.H, w.k, w.E
    act = 1 if w.fp8 else 2
    c = {
        "permute_scatter": T * H * 2 + N * H * act + T * k * 4,
        "combine": N * H * 2 + T * k * 8 + T * H * 2,
    }
    if training and not router:
        c["combine_bwd"] = T * H * 2 + T * k * 8 + N * H * 2
        c["dispatch_bwd"] = N * H * 2 + T * k * 4 + T * H * 2
    if training and router:
        c["combine_bwd_router"] = T * H * 2 + 2 * N * H * 2 + T * k * 12 + T * E * 4
        c["dispatch_bwd_router"] = N * H * 2 + T * k * 8 + E * H * 2 + T * H * 2
    return c


def router_costs(w, training):
    """Algorithmic FLOPs and bytes of the router projection and its weight gradient."""
    T, H, E = w.T, w.H, w.E
    c = {"router_logits": (2.0 * T * H * E, T * H * 2 + E * H * 2 + T * E * 4)}
    if training:
        c["router_wgrad"] = (2.0 * T * H * E, T * E * 4 + T * H * 2 + E * H * 4)
    return c


GEMM_STAGES = ["gemm1_swiglu", "gemm2", "gemm2_bwd_swiglu", "dw_down", "gemm1_bwd_dx", "dw_gu"]
TITLES = {"qwen3": "Qwen3-30B-A3B-shaped block, forward + backward",
          "mixtral": "Mixtral-shaped block, forward",
          "llama4": "Llama4-shaped decode step, forward",
          "skewed_fp8": "skewed-routing block in e4m3, forward"}


def traffic_file(workload):
    """The committed HBM-traffic summary of one workload's grouped-GEMM launches."""
    return os.path.join(ROOT, "profiles", f"grouped_gemm_hbm_traffic_{workload}.md")


def gemm_stages(workload):
    """GEMM stages a --pmc-pass run launches, in order: the forward pair, plus the four
    backward launches when the workload trains."""
    import workloads as W
    return GEMM_STAGES if W.WORKLOADS[workload].training else GEMM_STAGES[:2]
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_amd", "csrc", "gemm.hip")
CALIB_BYTES = 256 << 20


def _source_hash():
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _pmc_rows(folder, counter):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def pmc_summary(fetch_dir, write_dir, workload):
    """HBM bytes per launch of each GEMM stage of one --pmc-pass run: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what each counter reads for a plain copy of
    CALIB_BYTES (read CALIB_BYTES, write CALIB_BYTES)."""
    out = {}
    stages = gemm_stages(workload)
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(folder, counter)
        gemm = [r for r in rows if "grouped_gemm_kernel" in r[1]]
        assert len(gemm) >= len(stages), f"{counter}: {len(gemm)} GEMM dispatches"
        # the calibration copy (an fp32 negation, CALIB_BYTES in and out) is the last dispatch
        assert "elementwise" in rows[-1][1], rows[-1][1]
        factor = CALIB_BYTES / (rows[-1][2] * 1024.0)
        # the pass launches each stage once, in GEMM_STAGES order, after one warm step
        stage_rows = gemm[-len(stages):]
        out[counter] = {"factor": factor, "stages": {n: r[2] * 1024.0 * factor
                                                     for n, r in zip(stages, stage_rows)},
                        "kernels": {n: r[1] for n, r in zip(stages, stage_rows)}}
    data = {"workload": workload, "gemm_source_sha256_16": _source_hash(),
            "fetch_factor": round(out["FETCH_SIZE"]["factor"], 4),
            "write_factor": round(out["WRITE_SIZE"]["factor"], 4),
            "bytes_per_launch": {n: round(out["FETCH_SIZE"]["stages"][n] + out["WRITE_SIZE"]["stages"][n])
                                 for n in stages},
            "fetch_bytes_per_launch": {n: round(out["FETCH_SIZE"]["stages"][n]) for n in stages},
            "write_bytes_per_launch": {n: round(out["WRITE_SIZE"]["stages"][n]) for n in stages}}
    wl = f" --workload {workload}"
    lines = [f"# HBM traffic of the grouped-GEMM launches: {TITLES.get(workload, workload)}", "",
             "Commands (repository root; rocprofv3 run from /tmp):", "", "```",
             f"rocprofv3 --pmc FETCH_SIZE -f csv -d out/pmc_fetch -o run -- python3 bench.py{wl} --pmc-pass --no-cpu-baseline",
             f"rocprofv3 --pmc WRITE_SIZE -f csv -d out/pmc_write -o run -- python3 bench.py{wl} --pmc-pass --no-cpu-baseline",
             f"python3 bench.py{wl} --pmc-summary out/pmc_fetch out/pmc_write", "```", "",
             f"Calibration: a plain copy of {CALIB_BYTES >> 20} MiB reads FETCH_SIZE x {data['fetch_factor']} "
             f"and WRITE_SIZE x {data['write_factor']} of its true byte counts; the factors scale the "
             "GEMM readings below. The data block is read by bench.py while the GEMM source hash matches.", "",
             "| stage | kernel | HBM read MB | HBM write MB | total MB |", "|---|---|---:|---:|---:|"]
    for n in stages:
        k = out["FETCH_SIZE"]["kernels"][n]
        k = k[k.find("grouped_gemm_kernel"):][:60]
        lines.append(f"| {n} | `{k}` | {data['fetch_bytes_per_launch'][n] / 1e6:.1f} | "
                     f"{data['write_bytes_per_launch'][n] / 1e6:.1f} | {data['bytes_per_launch'][n] / 1e6:.1f} |")
    lines += ["", "```json", json.dumps(data), "```", ""]
    return "\n".join(lines)


def trace_summary(folder, steps):
    """Markdown tables from a rocprofv3 --kernel-trace run of this script with --steps
    `steps`: every kernel (calls and durations); the layer steps' launches in order (the
    first, cold step left out; the steps end where the per-stage region begins, at the
    first launch of the plain router entry point, since the layer's own router launch also
    writes chunk histograms); and the stages timed inside steps, the region whose HIP events
    give the bench line's per-launch times and roofline: `steps` passes over the entry
    points, each opened by one plain router launch (and the fill of its counts), up to the
    closing layer step."""
    import csv
    import glob
    import re

    def short(name):
        name = name.replace("moe::", "").replace("(anonymous namespace)::", "").replace("void ", "")
        m = re.match(r"(grouped_gemm_kernel<[^>]*>|mx_gemm_kernel<[^>]*>)", name)
        return m.group(1) if m else re.sub(r"\(.*$", "", name)[:70]

    ev = []
    for path in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if "spin_kernel" in r["Kernel_Name"]:  # the untimed stream hold before each pass
                continue
            ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short(r["Kernel_Name"])))
    ev.sort()
    lines = ["| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    per = {}
    for t0, t1, n in ev:
        per.setdefault(n, []).append((t1 - t0) / 1e3)
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{n}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")

    def plain_router(n):
        return n.startswith(("router_row_kernel<", "router_topk_kernel<")) and n.endswith(", false>")

    def layer_router(n):
        return (n.startswith(("router_row_kernel<", "router_topk_kernel<")) and n.endswith(", true>")) \
            or n.startswith(("router_logits", "router_ext", "route_dispatch_small_kernel"))

    end = next((i for i, e in enumerate(ev) if plain_router(e[2])), len(ev))
    start = next((i for i, e in enumerate(ev[:end]) if layer_router(e[2])), 0)
    layer = ev[start:end]
    names = [n for _, _, n in layer]
    firsts = [i for i, n in enumerate(names) if n == names[0]] if names else []
    period = firsts[1] - firsts[0] if len(firsts) > 1 else len(names)
    nstep = len(names) // period if period else 0
    if nstep > 1:
        lines += ["", f"Layer steps: {nstep} steps of {period} launches; per launch over steps 2..{nstep}:", "",
                  "| # | kernel | avg us | min us | max us |", "|---:|---|---:|---:|---:|"]
        for j in range(period):
            v = [(layer[s * period + j][1] - layer[s * period + j][0]) / 1e3 for s in range(1, nstep)]
            lines.append(f"| {j} | `{names[j]}` | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        spans = [(layer[s * period + period - 1][1] - layer[s * period][0]) / 1e3 for s in range(1, nstep)]
        lines += ["", f"Step span (first launch start to last launch end), steps 2..{nstep}: "
                      f"avg {sum(spans) / len(spans):.1f} us, min {min(spans):.1f} us"]
    plain = [i for i, e in enumerate(ev) if plain_router(e[2])]
    closing = [i for i, e in enumerate(ev) if layer_router(e[2])]
    if len(plain) >= steps and closing and closing[-1] > plain[-1]:
        s0 = plain[-steps]
        if s0 > 0 and ev[s0 - 1][2] == "fill_i32_kernel":
            s0 -= 1
        region = ev[s0:closing[-1]]
        per_step = len(region) // steps
        if per_step and per_step * steps == len(region):
            lines += ["", f"Stages timed inside steps by the bench (its HIP events): {steps} passes of "
                          f"{per_step} launches; per launch over all passes:", "",
                      "| # | kernel | avg us | min us | max us |", "|---:|---|---:|---:|---:|"]
            for j in range(per_step):
                v = [(region[s * per_step + j][1] - region[s * per_step + j][0]) / 1e3 for s in range(steps)]
                lines.append(f"| {j} | `{region[j][2]}` | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines) + "\n"


def measured_traffic(stage, workload):
    """HBM bytes per launch of `stage` from the committed counter summary, or None when the
    summary is missing, was taken on another workload, or the GEMM source changed since the
    counters were taken."""
    try:
        text = open(traffic_file(workload)).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if data.get("gemm_source_sha256_16") != _source_hash() or data.get("workload") != workload:
        return None
    return data["bytes_per_launch"].get(stage)


def step_order(training, mx, fp8, router):
    """Stage names in the order moe_forward / moe_backward enqueue their kernels."""
    fwd = (["router_logits"] if router else []) + ["router", "permute"]
    if mx:
        fwd += ["quantize_x", "gemm1_swiglu", "quantize_h", "gemm2", "combine"]
    else:
        fwd += ["gemm1_swiglu"] + (["quantize_h"] if fp8 else []) + ["gemm2", "combine"]
    if not training:
        return fwd
    bwd = ["combine_bwd_router", "router_wgrad"] if router else ["combine_bwd"]
    if mx:
        bwd += ["quantize_dout", "gemm2_bwd_swiglu", "quantize_dgu", "gemm1_bwd_dx", "col_offsets",
                "quantize_cols_h", "quantize_cols_dout", "dw_down", "quantize_cols_x",
                "quantize_cols_dgu", "dw_gu"]
    else:
        bwd += ["gemm2_bwd_swiglu", "dw_down", "gemm1_bwd_dx", "dw_gu"]
    bwd += ["dispatch_bwd_router"] if router else ["dispatch_bwd"]
    return fwd + bwd


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3",
                    help="qwen3 (default, forward+backward) | mixtral | llama4 | skewed_fp8 | tiny")
    ap.add_argument("--kernel-reps", type=int, default=20)
    # the oracle's cost has a large fixed part (every expert's weights in float64), so a small
    # token sample understates its rate; the default is the whole Qwen3-shaped workload
    # (about 10 s on 16 host cores)
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=False,
                    help="time replays of the step captured in a HIP graph instead of eager "
                         "launches (measured no faster: the host stays ahead of the GPU)")
    ap.add_argument("--router", action="store_true",
                    help="the layer owns its router projection: logits = x . W_r^T in the "
                         "forward, d_logits, dW_r and the router's dx term in the backward")
    ap.add_argument("--groups", type=int, nargs=2, metavar=("NUM_GROUPS", "GROUP_TOPK"),
                    help="grouped routing: experts in NUM_GROUPS groups, top-k from GROUP_TOPK")
    ap.add_argument("--expert-bias", action="store_true",
                    help="an expert selection bias (sigmoid / sqrtsoftplus scores only)")
    ap.add_argument("--score", choices=["softmax_pre_renorm", "softmax_post", "sigmoid",
                                        "sqrtsoftplus", "softmax_pre"],
                    help="override the workload's score function")
    ap.add_argument("--scaling", type=float, default=1.0, help="routing-weight scaling factor")
    ap.add_argument("--placement", choices=["combine", "input", "activation"], default="combine",
                    help="apply the routing weights to the expert outputs (combine) or inputs")
    ap.add_argument("--align", type=int, default=0, help="padded dispatch alignment (rows)")
    ap.add_argument("--mx", action="store_true",
                    help="the MXFP8 recipe (e4m3 with a power-of-two scale per 32 along K) in "
                         "every expert GEMM, forward and (training workloads) backward")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="launch each stage once plus a 256 MiB calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM-traffic summary from two rocprofv3 --pmc output folders")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="print kernel tables from a rocprofv3 --kernel-trace output folder")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary, args.workload))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.steps), end="")
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the MoE path here is single-device "
              f"(no expert parallelism); got --gpus {args.gpus}, WORLD_SIZE={world}.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_amd as M
    import workloads as W

    w = W.WORKLOADS[args.workload]
    training = w.training
    _log(f"bench: workload {w.name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} "
         f"fp8={w.fp8} training={training}")
    d = W.make_inputs(w.name)
    dev = torch.device("cuda:0")
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    x, w_gu, w_down = bf(d["x"]), bf(d["w_gu"]), bf(d["w_down"])
    logits = torch.from_numpy(d["logits"]).to(dev)
    shared_gu = bf(d["shared_gu"]) if w.shared_I else None
    shared_down = bf(d["shared_down"]) if w.shared_I else None
    if args.mx:  # the per-row fp8 recipe is replaced, not combined
        import dataclasses
        w = dataclasses.replace(w, fp8=False)
    dtype = M.MOE_MXFP8 if args.mx else (M.MOE_FP8_E4M3 if w.fp8 else M.MOE_BF16)
    w_gu_s = w_down_s = None
    if w.fp8:  # offline weight preparation, outside the timed region
        wq = torch.empty((w.E, 2 * w.I, w.H), dtype=torch.uint8, device=dev)
        w_gu_s = torch.empty((w.E, 2 * w.I), dtype=torch.float32, device=dev)
        M.moe_quantize_fp8_weights(w_gu, wq, w_gu_s)
        dq = torch.empty((w.E, w.H, w.I), dtype=torch.uint8, device=dev)
        w_down_s = torch.empty((w.E, w.H), dtype=torch.float32, device=dev)
        M.moe_quantize_fp8_weights(w_down, dq, w_down_s)
        w_gu, w_down = wq, dq
    mx_bwd = {}
    if args.mx:
        # weight preparation, once per optimizer update (outside the timed region; timed
        # below as its own launches): codes blocked along the forward K, and for training a
        # second copy blocked along the stored last axis for the data gradients
        E_, H_, I_ = w.E, w.H, w.I
        w_gu_bf, w_down_bf = w_gu, w_down
        wq = torch.empty((E_, 2 * I_, H_), dtype=torch.uint8, device=dev)
        w_gu_s = torch.empty((E_, 2 * I_, H_ // 32), dtype=torch.uint8, device=dev)
        dq = torch.empty((E_, H_, I_), dtype=torch.uint8, device=dev)
        w_down_s = torch.empty((E_, H_, I_ // 32), dtype=torch.uint8, device=dev)
        mx_prep = {"quantize_w_fwd": lambda: (M.moe_quantize_mxfp8_weights(w_gu_bf, wq, w_gu_s),
                                              M.moe_quantize_mxfp8_weights(w_down_bf, dq, w_down_s))}
        if training:
            gb = torch.empty((E_, H_, 2 * I_), dtype=torch.uint8, device=dev)
            gbs = torch.empty((E_, H_, 2 * I_ // 32), dtype=torch.uint8, device=dev)
            db = torch.empty((E_, I_, H_), dtype=torch.uint8, device=dev)
            dbs = torch.empty((E_, I_, H_ // 32), dtype=torch.uint8, device=dev)
            mx_prep["quantize_w_bwd"] = lambda: (
                M.moe_quantize_mxfp8_rows(w_gu_bf.view(E_ * H_, 2 * I_), gb.view(E_ * H_, 2 * I_),
                                          gbs.view(E_ * H_, 2 * I_ // 32)),
                M.moe_quantize_mxfp8_rows(w_down_bf.view(E_ * I_, H_), db.view(E_ * I_, H_),
                                          dbs.view(E_ * I_, H_ // 32)))
            mx_bwd = dict(w_gu_bwd=gb, w_gu_bwd_scale=gbs, w_down_bwd=db, w_down_bwd_scale=dbs)
        for fn in mx_prep.values():
            fn()
        w_gu, w_down = wq, dq
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    router = args.router
    w_router = bf(d["w_router"]) if router else None
    dw_router = torch.empty((w.E, w.H), dtype=torch.float32, device=dev) if router else None
    score = M._score(args.score) if args.score else w.score
    if score != w.score:
        import dataclasses
        w = dataclasses.replace(w, score=score)
    groups = args.groups or (0, 0)
    e_bias = (torch.randn(w.E, generator=torch.Generator().manual_seed(0)) * 0.1).to(dev) \
        if args.expert_bias else None
    placement = {"combine": M.MOE_PLACE_COMBINE, "input": M.MOE_PLACE_INPUT,
                 "activation": M.MOE_PLACE_ACTIVATION}[args.placement]
    prob = M.problem(w.T, w.H, w.E, w.k, w.I, w.score, w.shared_I, dtype, training, router,
                     groups[0], groups[1], args.scaling, placement, args.align)
    ws = torch.zeros(M.moe_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    tens = M.tensors(x, None if router else logits, w_gu, w_down, y, w_gu_s, w_down_s, shared_gu,
                     shared_down, w_router, dw_router, e_bias, **mx_bwd)
    router_opts = M.router_opts(e_bias, groups[0], groups[1], args.scaling)
    if training:
        dy = bf(d["dy"])
        dx = torch.empty_like(x)
        dw_gu = torch.empty((w.E, w.H, 2 * w.I), dtype=torch.bfloat16, device=dev)
        dw_down = torch.empty((w.E, w.I, w.H), dtype=torch.bfloat16, device=dev)

    if args.pmc_pass:  # counters: one warm step, then each GEMM stage once
        args.warmup, args.steps = 1, 1

    def step():
        M.moe_forward(prob, tens, ws)
        if training:
            M.moe_backward(prob, tens, dy, dx, dw_gu, dw_down, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _log(f"bench: warmup done ({args.warmup} steps)")

    # With --graph the whole step (every launch reads its sizes from arguments and its row
    # counts from device memory) is recorded once in a HIP graph and replayed.
    run = step
    graph = None
    if args.graph and not args.pmc_pass:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
        _log("bench: step captured in a HIP graph")

    # ---- timed region: whole layer --------------------------------------------------
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = w.T / (ms / 1e3)
    _log(f"bench: {args.steps} steps, {ms:.3f} ms/step, {tokens_per_s:,.0f} tokens/s")

    # ---- per-kernel durations with HIP events on the launch stream -----------------
    stream = torch.cuda.current_stream()
    v = M.moe_workspace_views(prob, ws)
    N, H, I, E, k, T = v.rows, w.H, w.I, w.E, w.k, w.T  # rows: T*k (+ padding capacity)
    vt = lambda name, shape, dt: M.view_tensor(getattr(v, name), shape, dt, ws)
    offs = vt("offsets", (E + 1,), torch.int32)
    row_of = vt("row_of", (T, k), torch.int32)
    topk_prob = vt("topk_prob", (T, k), torch.float32)
    act_dt = torch.uint8 if w.fp8 else torch.bfloat16
    xp = vt("xp", (N, H), act_dt)
    h = vt("h", (N, I), torch.bfloat16)
    out = vt("out", (N, H), torch.bfloat16)
    gu = vt("gu", (N, 2 * I), torch.bfloat16) if training else None
    xp_scale = vt("xp_scale", (N,), torch.float32) if w.fp8 else None
    hq = vt("hq", (N, I), torch.uint8) if w.fp8 else None
    h_scale = vt("h_scale", (N,), torch.float32) if w.fp8 else None
    shared_out = vt("shared_out", (T, H), torch.bfloat16) if w.shared_I else None
    scratch = M.view_tensor(v.scratch, (max(v.scratch_bytes, 16),), torch.uint8, ws)
    idx_t = vt("topk_idx", (T, k), torch.int32)
    src_of = vt("src_of", (N,), torch.int32)
    counts = vt("counts", (E,), torch.int32)

    pdtype = M.MOE_BF16 if args.mx else dtype  # MXFP8 quantises after the bf16 dispatch
    # split-K space of the decode-sized bf16 GEMMs (the layer keeps its own in ws)
    sk_bytes = max(M.moe_grouped_gemm_splitk_workspace_bytes(N, E, 2 * I),
                   M.moe_grouped_gemm_splitk_workspace_bytes(N, E, H)) if dtype == M.MOE_BF16 else 0
    skws = torch.empty(sk_bytes, dtype=torch.uint8, device=dev) if sk_bytes else None
    launches = {
        "router": lambda: M.moe_router_topk_ex(logits, k, w.score, router_opts, idx_t, topk_prob,
                                               counts),
        "permute": (lambda: M.moe_permute_padded(
            x, idx_t, E, args.align, xp, offs, vt("pad_offsets", (E,), torch.int32), row_of,
            src_of, scratch, pdtype, xp_scale)) if args.align > 1 else
                   (lambda: M.moe_permute(x, idx_t, E, xp, offs, row_of, src_of, scratch,
                                          pdtype, xp_scale)),
        "gemm1_swiglu": lambda: M.moe_grouped_gemm_swiglu(xp, w_gu, offs, h, gu, dtype,
                                                          xp_scale, w_gu_s, ws=skws),
        "gemm2": (lambda: M.moe_grouped_gemm(M.MOE_GEMM_NT, hq, w_down, offs, out, dtype,
                                             h_scale, w_down_s)) if w.fp8 else
                 (lambda: M.moe_grouped_gemm(M.MOE_GEMM_NN, h, w_down, offs, out, ws=skws)),
        "combine": lambda: M.moe_unpermute_combine(out, row_of, topk_prob, y, shared_out),
    }
    if w.fp8:
        launches["quantize_h"] = lambda: M.moe_quantize_fp8_rows(h, hq, h_scale)
    if args.mx:
        xq = vt("xq", (N, H), torch.uint8)
        xqs = vt("xq_scale", (N, H // 32), torch.uint8)
        hq = vt("hq", (N, I), torch.uint8)
        hqs = vt("hq_scale", (N, I // 32), torch.uint8)
        launches.update({
            "quantize_x": lambda: M.moe_quantize_mxfp8_rows(xp, xq, xqs),
            "gemm1_swiglu": lambda: M.moe_grouped_gemm_mxfp8(xq, xqs, w_gu, w_gu_s, offs, h,
                                                             swiglu=True),
            "quantize_h": lambda: M.moe_quantize_mxfp8_rows(h, hq, hqs),
            "gemm2": lambda: M.moe_grouped_gemm_mxfp8(hq, hqs, w_down, w_down_s, offs, out),
        })
        launches.update(mx_prep)
    if training:
        d_out = vt("d_out", (N, H), torch.bfloat16)
        dgu = vt("dgu", (N, 2 * I), torch.bfloat16)
        dxp = vt("dxp", (N, H), torch.bfloat16)
        launches.update({
            **({} if router else {
                "combine_bwd": lambda: M.moe_combine_backward(dy, row_of, topk_prob, d_out)}),
            "gemm2_bwd_swiglu": lambda: M.moe_grouped_gemm_swiglu_bwd(d_out, w_down, offs, gu, dgu),
            "dw_down": lambda: M.moe_grouped_gemm(M.MOE_GEMM_TN_DW, h, d_out, offs, dw_down),
            "gemm1_bwd_dx": lambda: M.moe_grouped_gemm(M.MOE_GEMM_NT, dgu, w_gu, offs, dxp),
            "dw_gu": lambda: M.moe_grouped_gemm(M.MOE_GEMM_TN_DW, xp, dgu, offs, dw_gu),
            **({} if router else {
                "dispatch_bwd": lambda: M.moe_unpermute_combine(dxp, row_of, None, dx)}),
        })
    if training and args.mx:
        Kp = v.mx_kp
        co = vt("mx_col_offsets", (E + 1,), torch.int32)
        dgq, dgqs = vt("dgq", (N, 2 * I), torch.uint8), vt("dgq_scale", (N, 2 * I // 32), torch.uint8)
        ta = lambda C: (vt("mx_ta", (C, Kp), torch.uint8), vt("mx_ta_scale", (C, Kp // 32), torch.uint8))
        tb = lambda C: (vt("mx_tb", (C, Kp), torch.uint8), vt("mx_tb_scale", (C, Kp // 32), torch.uint8))
        launches.update({
            "quantize_dout": lambda: M.moe_quantize_mxfp8_rows(d_out, xq, xqs),
            "gemm2_bwd_swiglu": lambda: M.moe_grouped_gemm_mxfp8_swiglu_bwd(
                xq, xqs, mx_bwd["w_down_bwd"], mx_bwd["w_down_bwd_scale"], offs, gu, dgu),
            "quantize_dgu": lambda: M.moe_quantize_mxfp8_rows(dgu, dgq, dgqs),
            "gemm1_bwd_dx": lambda: M.moe_grouped_gemm_mxfp8(
                dgq, dgqs, mx_bwd["w_gu_bwd"], mx_bwd["w_gu_bwd_scale"], offs, dxp),
            "col_offsets": lambda: M.moe_mxfp8_col_offsets(offs, co),
            "quantize_cols_h": lambda: M.moe_quantize_mxfp8_cols(h, offs, co, *ta(I)),
            "quantize_cols_dout": lambda: M.moe_quantize_mxfp8_cols(d_out, offs, co, *tb(H)),
            "dw_down": lambda: M.moe_grouped_gemm_mxfp8_wgrad(*ta(I), *tb(H), co, dw_down),
            "quantize_cols_x": lambda: M.moe_quantize_mxfp8_cols(xp, offs, co, *ta(H)),
            "quantize_cols_dgu": lambda: M.moe_quantize_mxfp8_cols(dgu, offs, co, *tb(2 * I)),
            "dw_gu": lambda: M.moe_grouped_gemm_mxfp8_wgrad(*ta(H), *tb(2 * I), co, dw_gu),
        })
    if router:
        r_logits = vt("logits", (T, E), torch.float32)
        launches["router_logits"] = lambda: M.moe_router_logits(x, w_router, r_logits)
        if training:
            d_logits = vt("d_logits", (T, E), torch.float32)
            rws = torch.empty(M.moe_router_weight_grad_workspace_bytes(T, H, E), dtype=torch.uint8,
                              device=dev)
            launches.update({
                "combine_bwd_router": lambda: M.moe_combine_backward_router(
                    dy, out, row_of, idx_t, topk_prob, w.score, d_out, d_logits),
                "router_wgrad": lambda: M.moe_router_weight_grad(x, d_logits, dw_router, rws),
                "dispatch_bwd_router": lambda: M.moe_dispatch_backward_router(
                    dxp, row_of, idx_t, d_logits, w_router, dx),
            })
    if args.pmc_pass:
        for name in GEMM_STAGES:
            if name in launches:
                launches[name]()
                torch.cuda.synchronize()
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": [n for n in GEMM_STAGES if n in launches]}), flush=True)
        return

    kernel_us = {}
    for name, fn in launches.items():
        fn()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(1_000_000)  # untimed: the repetitions are enqueued before they run
        ev0.record(stream)
        for _ in range(args.kernel_reps):
            fn()
        ev1.record(stream)
        ev1.synchronize()
        kernel_us[name] = ev0.elapsed_time(ev1) * 1e3 / args.kernel_reps
    kernel_us_warm = kernel_us
    # The same stages inside steps: the layer's launch sequence, stage by stage through the
    # entry points (the kernels moe_forward / moe_backward enqueue, in their order, on the same
    # inputs), with HIP events on the launch stream between the stages, for args.steps steps.
    # Each stage then runs on the cache state the stages before it leave, as in the timed
    # steps, rather than on its own warm inputs; these durations feed the roofline entry.
    order = [n for n in step_order(training, args.mx, w.fp8, router) if n in launches]
    in_step = {n: 0.0 for n in order}
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
        torch.cuda.synchronize()
        # hold the stream (untimed) while the host enqueues the pass, so that no stage's
        # interval includes the GPU waiting for the host's next launch
        torch.cuda._sleep(1_000_000)
        evs[0].record(stream)
        for i, n in enumerate(order):
            launches[n]()
            evs[i + 1].record(stream)
        evs[-1].synchronize()
        for i, n in enumerate(order):
            in_step[n] += evs[i].elapsed_time(evs[i + 1]) * 1e3 / args.steps
    kernel_us = {**kernel_us_warm, **in_step}
    step()  # leave the workspace as one full step wrote it
    torch.cuda.synchronize()
    _log("bench: per-launch us, warm repetitions " +
         json.dumps({k_: round(v_, 2) for k_, v_ in kernel_us_warm.items()}))
    _log("bench: per-launch us, inside steps " + json.dumps({k_: round(v_, 2) for k_, v_ in in_step.items()}))

    active = int((counts > 0).sum().item())  # experts that received rows in this step
    costs = stage_costs(w, training, active, mx=args.mx)
    peak_tf = MFMA_PEAK_TFLOPS["fp8" if (w.fp8 or args.mx) else "bf16"]
    gemm = {}
    for name, (fl, by) in costs.items():
        t = kernel_us[name] * 1e-6
        gemm[name] = {"us": round(kernel_us[name], 2), "tflops": round(fl / t / 1e12, 1),
                      "mfma_frac": round(fl / t / 1e12 / peak_tf, 4),
                      "gbs": round(by / t / 1e9, 1), "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    gemm_flops = sum(fl for fl, _ in costs.values())
    gemm_time = sum(kernel_us[n] for n in costs) * 1e-6
    rows = {}
    for name, by in row_costs(w, training, router).items():
        key = "permute" if name == "permute_scatter" else name
        t = kernel_us[key] * 1e-6
        rows[name] = {"us": round(kernel_us[key], 2), "gbs": round(by / t / 1e9, 1),
                      "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}

    rtr = {}
    if router:
        for name, (fl, by) in router_costs(w, training).items():
            t = kernel_us[name] * 1e-6
            rtr[name] = {"us": round(kernel_us[name], 2), "tflops": round(fl / t / 1e12, 1),
                         "gbs": round(by / t / 1e9, 1), "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}

    # dominant kernel: the GEMM launch with the longest duration
    dom = max(costs, key=lambda n: kernel_us[n])
    fl, by = costs[dom]
    t_dom = kernel_us[dom] * 1e-6
    t_at_mfma, t_at_hbm = fl / (peak_tf * 1e12), by / (HBM_PEAK_GBS * 1e9)
    if t_at_mfma >= t_at_hbm:
        roof = {"bound": "mfma", "achieved": round(fl / t_dom / 1e12, 2), "peak": peak_tf,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / t_dom / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    plain = not (args.mx or w.fp8 or router or args.align > 1 or args.groups or args.expert_bias
                 or args.score or args.scaling != 1.0 or placement != M.MOE_PLACE_COMBINE)
    roof["traffic"] = measured_traffic(dom, args.workload) if plain else None
    roof["kernel"] = dom
    roof["launch_us"] = round(kernel_us[dom], 2)       # inside steps (events between stages)
    roof["launch_us_warm"] = round(kernel_us_warm[dom], 2)  # back-to-back repetitions

    # ---- CPU oracle on a bounded sample -----------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from threadpoolctl import threadpool_info
        S = min(args.cpu_sample_tokens, w.T)
        _log(f"bench: timing the CPU oracle on {S} tokens")
        tc0 = time.perf_counter()
        lg = O.gate_logits(d["x"][:S], d["w_router"]) if router else d["logits"][:S]
        r = O.moe_forward(d["x"][:S], lg, d["w_gu"], d["w_down"], w.k, w.score,
                          w.I, d.get("shared_gu"), d.get("shared_down"),
                          fp8=w.fp8 and not args.mx, mx=args.mx)
        if training:
            O.moe_backward(r, d["dy"][:S], d["w_gu"], d["w_down"], w.I,
                           w_router_bits=d["w_router"] if router else None, mx=args.mx)
        tc = time.perf_counter() - tc0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), model)
        except OSError:
            pass
        # cores: the BLAS threads the oracle's float64 products ran on (its only parallel
        # part); host_cpus: every logical CPU of the host
        cpu = {"value": round(S / tc, 2), "unit": "tokens/s", "cores": threads,
               "host_cpus": os.cpu_count(), "cpu_model": model, "kind": "oracle",
               "sample": (f"the whole workload ({S} tokens)" if S == w.T else
                          f"first {S} of the {w.T} tokens") + ", full weights, "
                         f"{'forward+backward' if training else 'forward'}; {tc:.1f} s"}
        _log(f"bench: oracle {S} tokens in {tc:.1f} s")

    res = {
        "metric": "MoE layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), Qwen3-30B-A3B block",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if args.mx else ("fp8" if w.fp8 else "bf16"),
        "data": "synthetic",
        "config": {"workload": f"{w.name}-shaped MoE block " + ("with its router projection " if router else "")
                   + ("forward+backward" if training else "forward"),
                   "T": w.T, "H": w.H, "E": w.E, "top_k": w.k, "I": w.I, "shared_I": w.shared_I,
                   "score": ["softmax_pre_renorm", "softmax_post", "sigmoid", "sqrtsoftplus",
                             "softmax_pre"][w.score],
                   "parallelism": "single GPU", "active_experts": active,
                   "launch": "hip_graph" if graph is not None else "eager", "router": router,
                   **({"groups": list(groups)} if groups[0] else {}),
                   **({"expert_bias": True} if e_bias is not None else {}),
                   **({"scaling": args.scaling} if args.scaling != 1.0 else {}),
                   **({"placement": args.placement} if placement != M.MOE_PLACE_COMBINE else {}),
                   **({"align": args.align} if args.align > 1 else {})},
        "grouped_gemm_tflops": round(gemm_flops / gemm_time / 1e12, 1),
        "grouped_gemm_mfma_frac": round(gemm_flops / gemm_time / 1e12 / peak_tf, 4),
        "gemm": gemm,
        "rows": rows,
        **({"router": rtr} if router else {}),
        "kernel_us": {k_: round(v_, 2) for k_, v_ in kernel_us.items()},
        "kernel_us_warm": {k_: round(v_, 2) for k_, v_ in kernel_us_warm.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
