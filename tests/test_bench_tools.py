"""The bench's host-side tooling on synthetic profiler output (no GPU): the kernel-trace
summary finds the layer steps and the stage passes whose events give the roofline, the
HBM-traffic summary scales the counters by the calibration copy, and the stage order and
the traffic lookup follow the workload."""
import csv
import json
import os

import bench


def _write_trace(folder, events):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, t0, t1 in events:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t1})


def _timeline(seqs):
    """Back-to-back events from (kernel name, duration in ns) lists."""
    out, t = [], 1_000_000
    for name, dur in (e for s in seqs for e in s):
        out.append((name, t, t + dur))
        t += dur + 500
    return out


LAYER = [("void moe::router_row_kernel<8, true>(float const*)", 10_000),
         ("void moe::dispatch_rank_scan_kernel<4>(int const*)", 9_000),
         ("moe::scatter_rows_kernel(unsigned int)", 30_000),
         ("void moe::grouped_gemm_kernel<0, 1, false, 320, 256, 2, 4, 3, 64>(moe::GemmParams)", 300_000),
         ("void moe::combine_kernel<false>(unsigned int)", 25_000)]


def _pass(gemm_ns):
    return [("moe::fill_i32_kernel(int*, int, int)", 1_000),
            ("void moe::router_row_kernel<8, false>(float const*)", 11_000),
            ("moe::dispatch_hist_kernel(int const*)", 2_000),
            ("void moe::dispatch_rank_scan_kernel<4>(int const*)", 8_000),
            ("moe::scatter_rows_kernel(unsigned int)", 29_000),
            ("void moe::grouped_gemm_kernel<0, 1, false, 320, 256, 2, 4, 3, 64>(moe::GemmParams)", gemm_ns),
            ("void moe::combine_kernel<false>(unsigned int)", 24_000)]


SPIN = [("at::cuda::(anonymous namespace)::spin_kernel(long)", 500_000)]


def test_trace_summary_layer_steps_and_stage_passes(tmp_path):
    steps = 3
    warm = [("void moe::router_row_kernel<8, false>(float const*)", 11_000)] * 4
    passes = []
    for i in range(steps):
        passes += SPIN + _pass(280_000 + 10_000 * i)   # 280, 290, 300 us
    tail = [("void at::native::reduce_kernel<512, 1>(x)", 4_000)]
    ev = _timeline([LAYER] * 4 + [warm] + [passes] + [LAYER] + [tail])
    _write_trace(str(tmp_path / "tr"), ev)
    text = bench.trace_summary(str(tmp_path / "tr"), steps)
    assert "spin_kernel" not in text
    assert "Layer steps: 4 steps of 5 launches" in text
    assert f"{steps} passes of 7 launches" in text
    stage = text.split("Stages timed", 1)[1]
    gemm_row = [ln for ln in stage.splitlines() if "grouped_gemm_kernel" in ln][0]
    cells = [c.strip() for c in gemm_row.split("|")]
    assert cells[1] == "5"                     # position within the pass
    assert float(cells[3]) == 290.0            # average over the passes
    assert float(cells[4]) == 280.0 and float(cells[5]) == 300.0


def test_trace_summary_decode_step_starts_at_the_fused_launch(tmp_path):
    layer = [("void moe::route_dispatch_small_kernel<4>(float const*)", 6_000),
             ("void moe::grouped_gemm_kernel<0, 1, false, 32, 256, 1, 4, 3, 128>(moe::GemmParams)", 190_000),
             ("void moe::combine_kernel<false>(unsigned int)", 5_000)]
    warm = [("void moe::router_row_kernel<4, false>(float const*)", 3_000)] * 2
    passes = []
    for _ in range(2):
        passes += SPIN + [("moe::fill_i32_kernel(int*, int, int)", 1_000),
                          ("void moe::router_row_kernel<4, false>(float const*)", 3_000),
                          ("void moe::grouped_gemm_kernel<0, 1, false, 32, 256, 1, 4, 3, 128>(moe::GemmParams)", 185_000)]
    ev = _timeline([layer] * 3 + [warm] + [passes] + [layer])
    _write_trace(str(tmp_path / "tr"), ev)
    text = bench.trace_summary(str(tmp_path / "tr"), 2)
    assert "Layer steps: 3 steps of 3 launches" in text
    assert "2 passes of 3 launches" in text


def _write_counters(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path):
    gemm = "void moe::grouped_gemm_kernel<0, 1, false, 320, 256, 2, 4, 3, 64>(moe::GemmParams)"
    calib_kib = bench.CALIB_BYTES / 1024.0
    # FETCH reads the copy at twice its bytes, WRITE at its bytes: factors 0.5 and 1
    fetch = [(gemm, 7.0)] + [(gemm, 1000.0), (gemm, 2000.0)] + [("elementwise_kernel neg", 2 * calib_kib)]
    write = [(gemm, 7.0)] + [(gemm, 300.0), (gemm, 400.0)] + [("elementwise_kernel neg", calib_kib)]
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", write)
    md = bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), "mixtral")
    data = json.loads(md.split("```json", 1)[1].split("```", 1)[0])
    assert data["workload"] == "mixtral"
    assert abs(data["fetch_factor"] - 0.5) < 1e-9 and abs(data["write_factor"] - 1.0) < 1e-9
    # the last two GEMM dispatches are the two forward stages, in order
    assert data["fetch_bytes_per_launch"] == {"gemm1_swiglu": 512000, "gemm2": 1024000}
    assert data["write_bytes_per_launch"] == {"gemm1_swiglu": 307200, "gemm2": 409600}
    assert data["bytes_per_launch"]["gemm2"] == 1024000 + 409600
    assert data["gemm_source_sha256_16"] == bench._source_hash()
    assert "--workload mixtral --pmc-pass" in md


def test_stage_lists_follow_the_workload():
    assert bench.gemm_stages("qwen3") == bench.GEMM_STAGES
    assert bench.gemm_stages("mixtral") == ["gemm1_swiglu", "gemm2"]
    fwd = bench.step_order(False, False, False, False)
    assert fwd == ["router", "permute", "gemm1_swiglu", "gemm2", "combine"]
    assert "quantize_h" in bench.step_order(False, False, True, False)
    train = bench.step_order(True, False, False, True)
    assert train[0] == "router_logits" and train[-1] == "dispatch_bwd_router"
    assert train.index("dw_gu") > train.index("gemm1_bwd_dx")


def test_traffic_lookup_needs_the_same_source_and_workload(tmp_path, monkeypatch):
    body = {"workload": "qwen3", "gemm_source_sha256_16": bench._source_hash(),
            "bytes_per_launch": {"dw_gu": 123}}
    path = tmp_path / "grouped_gemm_hbm_traffic_qwen3.md"
    path.write_text("# t\n\n```json\n" + json.dumps(body) + "\n```\n")
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(tmp_path / f"grouped_gemm_hbm_traffic_{wl}.md"))
    assert bench.measured_traffic("dw_gu", "qwen3") == 123
    assert bench.measured_traffic("dw_gu", "mixtral") is None      # no summary for it
    body["gemm_source_sha256_16"] = "0" * 16                       # another kernel source
    path.write_text("```json\n" + json.dumps(body) + "\n```\n")
    assert bench.measured_traffic("dw_gu", "qwen3") is None
