"""Host-side contracts of the product path, checked without a GPU: the binding fails
loudly (no fallback) when the HIP library is missing; bench.py refuses more than one GPU
with a message, and its one-core CPU leg runs the oracle; the C header is plain C99 (and
C++17) that a C program can link against the library with."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

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
    """bench.py's CPU leg: the metric's pass on two worker processes, and the whole step's
    oracle work on two rows of every chunk, run and report positive times."""
    sys.path.insert(0, ROOT)
    import numpy as np

    import bench
    import workloads
    r = bench.cpu_baseline_workers("metric", 2)
    assert r["seconds"] > 0 and r["workers"] == 2 and r["repeat"] == 1
    ch = bench.ROWS // bench.W
    parts = [np.concatenate([workloads.rows(2, k, c * ch, 2, bench.COLS) for c in range(bench.W)])
             for k in range(bench.W)]
    v = np.empty((2 * bench.W, bench.W * bench.COLS), np.uint8)
    e = np.empty((2 * bench.W, bench.W * bench.COLS // 32), np.uint8)
    bench._oracle_pass("step", parts, 2 * bench.COLS, v, e)
    bench._oracle_pass("metric", parts, 2 * bench.COLS, v, e)
    share = bench.host_cpu_share()
    assert 1 <= share["used"] <= 16 and share["used"] <= share["allowed"]


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "blockq.h"

int main(void) {
    int64_t values = 0, scales = 0;
    if (bq_wire_bytes_b128(128) != 132) return 1;
    if (bq_mx_staging_bytes(4096, 43008, &values, &scales) != BQ_OK) return 2;
    if (values != 4096LL * 43008 || scales != 4096LL * 1344) return 3;
    if (bq_mx_staging_bytes(4096, 100, &values, &scales) != BQ_ERR_SIZE) return 4;
    if (strcmp(bq_status_str(BQ_OK), "ok") != 0) return 5;
    /* a device call with a NULL pointer is refused on the host, before any launch */
    if (bq_quant_i8(NULL, 128, NULL, NULL, NULL) != BQ_ERR_NULL) return 6;
    printf("%s\n", bq_version());
    return 0;
}
"""


@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_header_is_plain_c_and_links(tmp_path, lang):
    """include/blockq.h compiles as C99 and as C++17 with every warning an error, and a
    program using it links against libblockq.so and runs its host-side calls."""
    import block_quantized_wire_amd as bq
    src = tmp_path / ("prog.c" if lang == "c99" else "prog.cpp")
    src.write_text(C_PROGRAM)
    exe = tmp_path / "prog"
    libdir = os.path.dirname(bq.LIB_PATH)
    cc = ["gcc", "-std=c99", "-pedantic"] if lang == "c99" else ["g++", "-std=c++17"]
    cmd = cc + ["-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                "-o", str(exe), f"-L{libdir}", "-lblockq", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert "gfx950" in r.stdout
