"""GPU parity of the MXFP8 quantizer on IEEE binary16 input (the staged quantizer takes
BF16 or FP16 slices) against the CPU oracle, bit for bit."""
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


def assert_same(got, want, what):
    got, want = np.asarray(got).reshape(-1), np.asarray(want).reshape(-1)
    assert got.shape == want.shape, what
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"got {got[bad[:5]]} want {want[bad[:5]]}"


def gpu_quant_mx_f16(x: np.ndarray, ldv_pad: int = 0, lds_pad: int = 0):
    rows, cols = x.shape
    v = empty((rows, cols + ldv_pad), np.uint8)
    e = empty((rows, cols // 32 + lds_pad), np.uint8)
    bq.bq_quant_mx_f16(to_dev(x), v, e, rows=rows, cols=cols)
    sync()
    return host(v, np.uint8)[:, :cols], host(e, np.uint8)[:, :cols // 32]


@pytest.mark.parametrize("rows,cols,pad", [(1, 128, 0), (3, 384, 16), (7, 640, 0), (33, 1152, 32),
                                           (64, 7168, 0)])
def test_mx_f16_small_shapes(rows, cols, pad):
    say(f"mx f16 quant {rows}x{cols} pad={pad}")
    x = workloads.rows(4, 9, 0, rows, cols, fmt="f16")
    v, e = gpu_quant_mx_f16(x, ldv_pad=pad, lds_pad=4 if pad else 0)
    wv, we = oracle.quant_mx_f16(x)
    assert_same(e, we, "E8M0 scales")
    assert_same(v, wv, "E4M3 values")


def test_mx_f16_every_amax_and_every_value():
    """Groups with every positive finite binary16 amax (the E8M0 rule over the whole
    binary16 domain, subnormals included) and groups holding every finite binary16 value
    next to each of a few pilots (the scaled E4M3 encoding of every input)."""
    say("mx f16 every amax / every value")
    rng = np.random.default_rng(16)
    h = np.arange(1, 0x7C00, dtype=np.uint16)
    amax = h.view(np.float16).astype(np.float32)
    u = rng.uniform(-1, 1, (h.size, 31)).astype(np.float32)
    other = (u * amax[:, None]).astype(np.float16).view(np.uint16)
    groups = [np.concatenate([h[:, None], other], axis=1)]
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    allv = allv[((allv >> 10) & 0x1F) != 0x1F]
    pad = (-allv.size) % 31
    allv = np.concatenate([allv, np.zeros(pad, np.uint16)]).reshape(-1, 31)
    for pilot in (0x7BFF, 0x5C00, 0x3C00, 0x0400):        # 65504, 256, 1, 2^-14
        mag = allv & 0x7FFF
        keep = np.where(mag <= pilot, allv, np.uint16(0))
        groups.append(np.concatenate([np.full((allv.shape[0], 1), pilot, np.uint16), keep], axis=1))
    g = np.concatenate(groups)
    g = np.concatenate([g, np.zeros(((-g.shape[0]) % 4, 32), np.uint16)])
    x = g.reshape(-1, 128)
    v, e = gpu_quant_mx_f16(x)
    wv, we = oracle.quant_mx_f16(x)
    assert_same(e, we, "E8M0 over every binary16 amax")
    assert_same(v, wv, "E4M3 values")


def test_mx_f16_staged_slices_equal_one_call_and_oracle():
    """Six binary16 slices of 512x7168 (per-row gains over five decades) staged at their
    column offsets: equal to the one-call quantization of the concatenation, rows above
    the live rows untouched, and equal to the oracle."""
    say("mx f16 staged slices 6 x 512x7168")
    R, C, S = 512, 7168, 6
    cap = R + 64
    xs = [workloads.rows(4, j, 0, R, C, fmt="f16") for j in range(S)]
    v = filled((cap, S * C), np.uint8, 0xA5)
    e = filled((cap, S * C // 32), np.uint8, 0x5A)
    for j in (3, 0, 5, 1, 4, 2):
        bq.bq_quant_mx_slice_f16(to_dev(xs[j]), j * C, v, e, capacity_rows=cap)
    cat = np.concatenate(xs, axis=1)
    v1, e1 = gpu_quant_mx_f16(cat)
    gv, ge = host(v, np.uint8), host(e, np.uint8)
    assert_same(gv[:R], v1, "staged == one call (values)")
    assert_same(ge[:R], e1, "staged == one call (scales)")
    assert np.all(gv[R:] == 0xA5) and np.all(ge[R:] == 0x5A)
    wv, we = oracle.quant_mx_f16(np.ascontiguousarray(cat))
    assert_same(gv[:R], wv, "every row vs oracle (values)")
    assert_same(ge[:R], we, "every row vs oracle (scales)")
