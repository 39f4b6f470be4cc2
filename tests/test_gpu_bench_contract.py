"""bench.py's JSON line on the GPU: one short run, every field the line promises, and the
roofline figure consistent with the per-kernel figure it is taken from."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_fields():
    say("bench.py --steps 5 --warmup 1 --no-cpu-baseline (child process)")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "1", "--no-cpu-baseline"], cwd=ROOT, capture_output=True,
                       text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "gemm"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["value"] > 0
    assert "workload" in d["config"] and "model" not in d["config"]
    step_bytes = d["config"]["step_bytes"]
    assert abs(d["value"] - step_bytes / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    kern = d["kernels"][rf["kernel"]]
    assert kern["gbs"] == rf["achieved"]
    # the dominant kernel is the one with the most time per step
    per_step = {k: v["us_per_launch"] * v["launches_per_step"] for k, v in d["kernels"].items()}
    assert rf["kernel"] == max(per_step, key=per_step.get)
    g = d["gemm"]
    assert g["bound"] == "mfma" and g["unit"] == "TFLOP/s" and g["peak"] == 5000.0
    assert abs(g["frac"] - g["achieved"] / g["peak"]) < 1e-3
    assert d["accuracy"]["ranks_bit_identical"] is True
    # per-kernel figures are medians of their samples
    import statistics
    for k, v in d["kernels"].items():
        assert len(v["samples_us"]) == 5, k
        assert abs(statistics.median(v["samples_us"]) - v["us_per_launch"]) <= 0.011, k
    for k in ("torch", "hip", "library", "device", "arch", "compute_units", "memory_gib", "clocks",
              "source_digest"):
        assert k in d["receipt"], k
    import bench
    assert d["receipt"]["source_digest"] == bench.kernel_source_digest()
    assert "gfx950" in d["receipt"]["arch"]
