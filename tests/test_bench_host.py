"""bench.py's host-side logic, without a GPU: the throughput arithmetic, the comment-blind
digest that keys the HBM counters, and the kernel-trace summary (dispatch grouping,
back-to-back runs, the metric's passes) on a synthetic trace."""
from __future__ import annotations

import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_rate_arithmetic():
    r = bench.rate(335_118_336, 4 * 3072 * 7168, 57.80)
    assert r["gbs"] == pytest.approx(335_118_336 / 57.80e-6 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["gbs"] / 8000.0, abs=1e-4)
    assert r["bytes_per_element"] == pytest.approx(335_118_336 / (4 * 3072 * 7168), abs=1e-4)
    # values per second against the peak over the same bytes per value: the same fraction
    assert r["elements_frac"] == pytest.approx(r["frac"], abs=1e-3)


def test_metric_bytes_follow_the_per_block_counts():
    # 3072x7168 values quantized (388 B per 128) and three 4-rank hop steps (520 B per 128)
    assert bench.NB == 172_032
    assert bench.NB * bench.B_QUANT + 3 * bench.NB * bench.B_HOP == 335_118_336
    assert bench.B_A2A_REDUCE(4) == 916 and bench.B_DEQUANT_SHARED(4) == 1156


def test_code_only_drops_comments_and_blank_lines():
    src = "// header\nint a; // trailing\n\n  \nint b;\n"
    assert bench.code_only(src) == "int a;\nint b;"
    assert bench.code_only(src.replace("trailing", "other words")) == bench.code_only(src)
    assert bench.code_only(src.replace("int b", "int c")) != bench.code_only(src)


def _trace(path, seq):
    """A kernel-trace CSV: seq is a list of (kernel name, workgroups, segments, duration us)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Grid_Size_Y",
                               "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1_000_000
        for name, wg, seg, us in seq:
            w.writerow({"Kernel_Name": name, "Grid_Size_X": wg * 256, "Workgroup_Size_X": 256,
                        "Grid_Size_Y": seg, "Start_Timestamp": t,
                        "End_Timestamp": t + int(us * 1000)})
            t += int(us * 1000) + 500


def test_summarize_trace_groups_runs_and_passes(tmp_path):
    q = "void bq::(anonymous namespace)::k_quant_i8<1, true>(bq::QuantArgs)"
    h = "void bq::(anonymous namespace)::k_ring_hop_i8<1>(bq::HopArgs)"
    d = "void bq::(anonymous namespace)::k_dequant_i8<2, false>(bq::DequantArgs)"
    seq = [(q, 1344, 4, 14.0)] * 12                      # a back-to-back run of 12
    seq += [(d, 4096, 4, 30.0)]                          # (so no pass starts at the run's end)
    seq += [(h, 1344, 4, 18.0)] * 3                      # too short to count as a run
    for _ in range(5):                                   # five metric passes
        seq += [(q, 1344, 4, 13.0), (h, 1344, 4, 16.0), (h, 1344, 4, 15.0), (h, 1344, 4, 15.0)]
    seq += [(h, 5376, 1, 40.0)] * 10                     # another launch shape of the hop
    p = tmp_path / "trace.csv"
    _trace(p, seq)
    out = bench.summarize_trace(str(p))
    lines = {l.split("|")[1].strip() + l.split("|")[2].strip(): l for l in out.splitlines()
             if l.startswith("| `")}
    quant = lines["`k_quant_i8<1, true>`1344 x 4"].split("|")
    assert quant[3].strip() == "17"                               # dispatches
    assert float(quant[4]) == pytest.approx((12 * 14 + 5 * 13) / 17, abs=0.01)
    assert float(quant[7]) == pytest.approx(14.0, abs=0.01)       # only the run of 12
    hop = lines["`k_ring_hop_i8<1>`1344 x 4"].split("|")
    assert hop[3].strip() == "18" and hop[7].strip() == ""        # no run of 10 or more
    wide = lines["`k_ring_hop_i8<1>`5376 x 1"].split("|")
    assert float(wide[7]) == pytest.approx(40.0, abs=0.01)
    assert "Metric passes (quantize, hop 1, hop 2, hop 3): 5; average us 13.00, 16.00, 15.00, " \
           "15.00" in out
