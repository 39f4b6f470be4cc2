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


@pytest.mark.timeout(400)
def test_bench_line_fields():
    say("bench.py --steps 5 --warmup 1 --no-cpu-baseline (child process)")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "1", "--no-cpu-baseline"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "gemm", "value_region", "step", "configs", "elements_per_s"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["value"] > 0
    assert d["dtype"] == "bf16"
    assert "workload" in d["config"] and "model" not in d["config"]
    # value: the quantize of 3072x7168 values and three 4-rank hop steps over 768x7168 each
    vr = d["value_region"]
    assert vr["bytes_per_pass"] == 172032 * 388 + 3 * 172032 * 520
    assert vr["values_per_pass"] == 4 * 3072 * 7168
    assert d["value"] == vr["gbs"]
    assert abs(vr["gbs"] - vr["bytes_per_pass"] / (vr["us_per_pass"] * 1e-6) / 1e9) <= 0.01 * vr["gbs"]
    assert abs(vr["elements_frac"] - vr["frac"]) < 2e-3
    st = d["step"]
    assert abs(st["gbs"] - st["bytes"] / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * st["gbs"]
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # the roofline's kernel: the metric pass's kernel with the most time per pass (timed alone)
    kern = d["kernels"][rf["kernel"]]
    assert kern["gbs"] == rf["achieved"]
    metric_kernels = {"quant_i8 x4 (66748416 B)": 1, "ring_hop_i8 x4 (89456640 B)": 3}
    per_pass = {k: d["kernels"][k]["us_per_launch"] * c for k, c in metric_kernels.items()}
    assert rf["kernel"] == max(per_pass, key=per_pass.get)
    g = d["gemm"]
    assert g["bound"] == "mfma" and g["unit"] == "TFLOP/s" and g["peak"] == 5000.0
    assert abs(g["frac"] - g["achieved"] / g["peak"]) < 1e-3
    assert sorted(g["layouts"]) == ["mfma K=42880", "mfma K=43008", "row-major K=42880",
                                    "row-major K=43008"]
    assert g["us_per_launch"] == g["layouts"]["mfma K=43008"]["us_per_launch"]
    assert d["accuracy"]["ranks_bit_identical"] is True
    # one TP4 rank's share as single-segment launches: 43,008 blocks of 768x7168
    sk = d["share_kernels"]
    assert sk["quant_i8 one rank (16687104 B)"]["bytes_per_launch"] == 43008 * 388
    assert sk["ring_hop_i8 one rank (22364160 B)"]["bytes_per_launch"] == 43008 * 520
    for v in sk.values():
        assert v["us_per_launch"] > 0 and abs(v["frac"] - v["gbs"] / 8000.0) < 1e-3
    # per-kernel figures are medians of their samples
    import statistics
    for k, v in d["kernels"].items():
        assert len(v["samples_us"]) == 5, k
        assert abs(statistics.median(v["samples_us"]) - v["us_per_launch"]) <= 0.011, k
    # every workload configuration at full size, with its bytes per pass
    cf = d["configs"]
    assert len(cf) == 5
    want = {"cfg1": 28672 * 388 * 2, "cfg3: i8_a2a all-reduce, 4 ": None,
            "cfg3: i8_a2a all-reduce, 16 ": None, "cfg4": 2 * 6 * 229376 * 388,
            "cfg5": 917504 * (388 + 3 * 520 + 132 + 4 * 256 + 2 * 388)}
    for prefix, nbytes in want.items():
        match = [k for k in cf if k.startswith(prefix)]
        assert len(match) == 1, prefix
        c = cf[match[0]]
        if nbytes is not None:
            assert c["bytes_per_pass"] == nbytes, prefix
        assert c["gbs"] > 0 and abs(c["frac"] - c["gbs"] / 8000.0) < 1e-3
        assert abs(c["elements_frac"] - c["frac"]) < 2e-3
        assert c["kernels"]
    for k in ("torch", "hip", "library", "device", "arch", "compute_units", "memory_gib", "clocks",
              "source_digest"):
        assert k in d["receipt"], k
    import bench
    assert d["receipt"]["source_digest"] == bench.kernel_source_digest()
    assert "gfx950" in d["receipt"]["arch"]
