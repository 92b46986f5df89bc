"""bench.py's output contract: one JSON line with the required fields (GPU), the refusal of
more than one GPU and the CPU-baseline leg (CPU)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_leg_reports_the_oracle_on_host_cores():
    sys.path.insert(0, ROOT)
    import bench
    from long_sequence_video_amd import inputs as gen
    res = bench.cpu_baseline(gen.make_config("tiny_s256_h4"), target_seconds=0.2)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["value"] > 0 and res["cores"] >= 1 and res["sample"]
    # the host's CPU model and numpy's BLAS are named beside the rate (null only where the host
    # does not say)
    assert "cpu_model" in res and "blas" in res
    assert res["blas"] is None or "blas" in res["blas"].lower()


def test_counter_summary_is_stale_once_a_device_header_changes(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hip"
    header = tmp_path / "tile_ops.h"
    header.write_text("// helpers v1\n")
    src.write_text('#include "lsv.h"\n#include "tile_ops.h"\n__global__ void k() {}\n')
    assert bench.kernel_device_headers(str(src)) == [str(header)]
    summary = tmp_path / "{kernel}_{workload}_hbm_traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    (tmp_path / "k_w_hbm_traffic.md").write_text(
        f"- kernel_source_sha256: `{bench.kernel_source_sha256(str(src))}`\n"
        f"- kernel_headers_sha256: `{bench.kernel_headers_sha256(str(src))}` (tile_ops.h)\n"
        "- hbm_bytes_per_launch: `1.5e+09`\n")
    assert bench.measured_traffic("w", kernel_source=str(src), kernel="k")[0] == 1.5e9
    header.write_text("// helpers v2\n")
    traffic, why = bench.measured_traffic("w", kernel_source=str(src), kernel="k")
    assert traffic is None and "header" in why
    header.write_text("// helpers v1\n")
    src.write_text(src.read_text() + "// edited\n")
    traffic, why = bench.measured_traffic("w", kernel_source=str(src), kernel="k")
    assert traffic is None and "kernel source" in why


@pytest.mark.gpu
def test_bench_json_line(gpu):
    cmd = [sys.executable, BENCH, "--config", "tiny_s256_h4", "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
           "--no-prologue", "--no-bwd", "--no-fp8", "--no-legs"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 1
    assert line["value"] > 0 and line["ms_per_step"] > 0 and line["higher_is_better"] is True
    assert line["dtype"] == "bf16" and line["unit"] == "TFLOP/s"
    assert line["config"]["workload"] == "tiny_s256_h4"
    roof = line["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    ref = line["mfma_reference"]  # the library GEMM calibration
    assert 0 < ref["tflops"] < 2500.0 and abs(ref["frac_of_peak"] - ref["tflops"] / 2500.0) < 1e-3
    assert abs(line["vs_library_gemm"] - line["value"] / ref["tflops"]) < 1e-3


@pytest.mark.gpu
def test_bench_json_line_with_key_split(gpu):
    """The forward leg through lsv_attn_fwd_split: the line names the split and the kernels, and
    carries no traffic figure (no counters were taken for that launch)."""
    cmd = [sys.executable, BENCH, "--config", "tiny_s256_h4", "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
           "--no-prologue", "--no-bwd", "--no-fp8", "--no-gemm-ref", "--no-legs", "--split", "2"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["config"]["key_split"] == 2 and line["value"] > 0
    assert line["roofline"]["kernel"] == "attn_fwd_split_kernel + attn_fwd_combine_kernel"
    assert line["roofline"]["traffic"] is None


@pytest.mark.gpu
def test_forward_leg_and_backward_roofline(gpu):
    """A forward leg reports its own timing and fraction of peak; the backward's roofline is
    stated on the counted flops (2.5 x the forward's), the executed count apart."""
    sys.path.insert(0, ROOT)
    import bench
    leg = bench.bench_forward_leg("tiny_s256_h4")
    assert leg["workload"] == "tiny_s256_h4" and leg["steps"] == bench.FORWARD_LEGS["tiny_s256_h4"]
    assert leg["ms_per_step"] > 0 and abs(leg["frac"] - leg["tflops"] / 2500.0) < 1e-3
    bwd = bench.bench_backward("tiny_s256_h4", 3, 1)
    roof = bwd["roofline"]
    assert abs(roof["achieved"] - bwd["tflops_counted"]) < 1e-2 and abs(roof["frac"] - roof["achieved"] / 2500) < 1e-3
    assert abs(bwd["mfma_flops_executed"] / bwd["flops_counted"] - 1.4) < 1e-12
    assert abs(bwd["frac_executed"] - bwd["tflops_executed"] / 2500.0) < 1e-3
