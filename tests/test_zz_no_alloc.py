"""The allocation-free ring all-reduce on the GPU, through the C ABI.

bq_ring_allreduce_i8_noalloc keeps the wire payload in the library's scratch array and
must give exactly what bq_ring_allreduce_i8 gives with caller-owned wire buffers (and
what the oracle gives): every rank's bf16 output, bit for bit.  Two calls in a row, the
second smaller, so the second runs on what the first left in the scratch array; then a
call too large for the array fails before anything is written.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import empty, filled, host, say, sync, to_dev

from block_quantized_wire_amd import build as _build

if _build.stale():
    _build.build()
import block_quantized_wire_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu


def _run_both(W: int, rows: int, cols: int, seed_rank: int):
    parts = [workloads.rows(2, seed_rank + r, 0, rows, cols).reshape(-1) for r in range(W)]
    n = parts[0].size
    pd = [to_dev(p) for p in parts]
    qw, sw = empty(n, np.int8), empty(n // 128, np.float32)
    want = [filled(n, np.uint16, 0xA5) for _ in range(W)]
    got = [filled(n, np.uint16, 0x5A) for _ in range(W)]
    bq.bq_ring_allreduce_i8(pd, qw, sw, want, n=n)
    bq.bq_ring_allreduce_i8_noalloc(pd, got, n=n)
    sync()
    return parts, [host(t, np.uint16) for t in want], [host(t, np.uint16) for t in got]


def test_noalloc_ring_equals_the_ring_driver_on_two_calls():
    # first call: the metric workload, 4 ranks x 3072x7168 (22.0M values, 22.7 MB of wire)
    say("noalloc ring: W=4, 3072x7168 per rank")
    parts, want, got = _run_both(4, 3072, 7168, 0)
    for r in range(4):
        assert np.array_equal(got[r], want[r]), f"rank {r}"
    # second call, smaller, on what the first left in the scratch array
    say("noalloc ring: W=3, 24x1024 per rank (second, smaller call)")
    parts, want, got = _run_both(3, 24, 1024, 7)
    _, _, wout = oracle.ring_allreduce_i8(parts)
    for r in range(3):
        assert np.array_equal(got[r], want[r]), f"rank {r}"
        assert np.array_equal(got[r], wout[r]), f"rank {r} vs oracle"


def test_noalloc_ring_rejects_a_call_beyond_its_scratch():
    say("noalloc ring: too large for the scratch array")
    W, n = 1, 65075200 + 128
    x = empty(n, np.uint16)
    out = filled(n, np.uint16, 0x3C)
    with pytest.raises(bq.BlockqError) as e:
        bq.bq_ring_allreduce_i8_noalloc([x], [out], n=n)
    assert e.value.name == "BQ_ERR_SCRATCH"
    sync()
    assert not np.any(host(out[-4096:], np.uint16) != 0x3C3C)
