"""Host-side contracts of the product path, checked without a GPU: the binding fails
loudly (no fallback) when the HIP library is missing, and bench.py refuses more than one
GPU with a message."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_fails_loudly_without_the_library(tmp_path):
    code = (
        "import block_quantized_wire_amd as bq\n"
        f"bq.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
        "bq._lib = None\n"
        "try:\n"
        "    bq.bq_version()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    raise SystemExit(0)\n"
        "raise SystemExit(3)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "is missing" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_runs_the_oracle_on_a_small_sample():
    """bench.py's one-core CPU leg on 8 rows of every rank: the oracle's whole step runs and
    the figure it reports is a positive rate for that fraction of the step."""
    sys.path.insert(0, ROOT)
    import bench
    r = bench.cpu_baseline(8)
    assert r["seconds"] > 0 and r["frac"] == 8 / bench.ROWS
