"""Regression: the library must work when the binding is loaded before torch.

torch ships its own HIP runtime under the same soname as the system one.  If
libblockq.so were loaded first it would bind the system runtime, torch would then
load its bundled copy, and the library's launches would fail with "no device".  The
binding therefore imports torch before loading the library; this runs that order in a
fresh process and checks a small quantization against the oracle.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu

SCRIPT = r'''
import sys
sys.path.insert(0, ROOT)
import block_quantized_wire_amd as bq
L = bq.lib                     # the library first, before any explicit torch import
import numpy as np, torch
import oracle, workloads
x = workloads.rows(6, 0, 0, 1, 128 * 64)[0]
xd = torch.from_numpy(x.view(np.int16)).to("cuda:0")
q = torch.empty(x.size, dtype=torch.int8, device="cuda:0")
s = torch.empty(x.size // 128, dtype=torch.float32, device="cuda:0")
bq.bq_quant_i8(xd, q, s)
torch.cuda.synchronize()
wq, ws = oracle.quant_i8(x)
assert np.array_equal(q.cpu().numpy(), wq) and np.array_equal(s.cpu().numpy(), ws)
print("load-order ok")
'''


def test_library_loaded_before_torch():
    code = SCRIPT.replace("ROOT", repr(ROOT))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "load-order ok" in r.stdout, r.stdout + r.stderr
