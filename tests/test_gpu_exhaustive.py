"""Exhaustive GPU check of block-INT8 quantize + materialize over its whole bf16 domain.

Every block holds one amax value A (each positive finite bf16, alternating sign) and
bf16 values x with |x| <= A.  Over all blocks, every pair (x, A) with |x| <= A -- both
signs and both zeros -- occurs exactly once: about 1.07e9 values.  Payloads, scales
and materialized bf16 outputs are compared bit for bit with the oracle, chunk by chunk.
This covers the kernel's quotient (fl32 of x times an fp64 reciprocal of the scale
refined by two Newton steps, exact by a midpoint-distance argument) and its dequantize
(one binary32 product of the payload byte and the scale) on every input the codec can
receive from bf16 data.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import empty, host, say, sync, to_dev

from block_quantized_wire_amd import build as _build

if _build.stale():
    _build.build()
import block_quantized_wire_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu


def blocks_for(h_lo: int, h_hi: int) -> np.ndarray:
    """Blocks for amax bit patterns h in [h_lo, h_hi): column 0 is +-A, columns 1..127
    enumerate every bf16 value of magnitude <= A (padded with +0)."""
    out = []
    for h in range(h_lo, h_hi):
        mags = np.arange(0, h + 1, dtype=np.uint16)
        xs = np.concatenate([mags, mags | np.uint16(0x8000)])
        pad = (-xs.size) % 127
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        a = np.full((xs.shape[0], 1), h | (0x8000 if h % 2 else 0), np.uint16)
        out.append(np.concatenate([a, xs], axis=1))
    return np.concatenate(out).reshape(-1)


@pytest.mark.parametrize("chunk", range(8))
def test_i8_every_x_amax_pair(chunk):
    h_all = 0x7F80                                  # positive finite bf16 are 1 .. 0x7F7F
    edges = np.sqrt(np.linspace(0, 1, 9)) * h_all   # equal numbers of pairs per chunk
    lo, hi = max(1, int(edges[chunk])), int(edges[chunk + 1]) if chunk < 7 else h_all
    say(f"exhaustive i8 pairs, amax bits [{lo:#x}, {hi:#x})")
    x = blocks_for(lo, hi)
    n = x.size
    xd = to_dev(x)
    q, s = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_quant_i8(xd, q, s, n=n)
    y = empty(n, np.uint16)
    bq.bq_dequant_i8(q, s, y, n=n)
    sync()
    wq, ws = oracle.quant_i8(x)
    gq = host(q, np.int8)
    assert np.array_equal(host(s, np.float32).view(np.uint32), ws.view(np.uint32)), "scales"
    bad = np.flatnonzero(gq != wq)
    assert bad.size == 0, f"{bad.size} payload mismatches, first {bad[:4]}"
    wy = oracle.dequant_i8(wq, ws)
    assert np.array_equal(host(y, np.uint16), wy), "materialized bf16"
