"""GPU parity past 2^31 values: the 64-bit addressing of every kernel family.

The flat kernels address a value as a 64-bit block base plus a 32-bit offset inside one
wave step, the 2-D MXFP8 kernels as a 64-bit row base plus a column, and the GEMM as a
64-bit row base of each operand.  Each case here holds more than 2^31 values (or, for
the GEMM, more than 2^31 weight bytes), so an index computed in 32 bits anywhere would
land on the wrong data.  Outputs are compared bit for bit with the oracle on sampled
rows: the first row, the rows on both sides of value index 2^31, the last row, and
random rows in between.

Each large tensor repeats a block of P generated rows (row r holds the seeded
generator's row r mod P; P = 8191, or 1021 for the 43008-column cases), tiled on the
device, so that filling a few gigabytes takes seconds.  P divides neither 2^31 nor 2^32
values' worth of rows, so an index that wrapped at 32 bits would read other data.  The
oracle regenerates just the sampled rows (the generator draws every row from its own
counter-based stream).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import empty, host, say, sync

from block_quantized_wire_amd import build as _build

if _build.stale():
    _build.build()
import block_quantized_wire_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu

COLS = 7168
P = 8191                            # rows of generated data, tiled
ROWS = 2 ** 31 // COLS + 1          # 299,594 rows x 7168: 2,147,489,792 values
MX_COLS = 43008
MX_ROWS = 2 ** 31 // MX_COLS + 1    # 49,933 rows x 43008: 2,147,518,464 values
MX_P = 1021


def sampled_rows(rows: int, cols: int, seed: int) -> np.ndarray:
    """First and last rows, the rows holding value indexes 2^31 - 1 and 2^31, and 8 more."""
    edge = [0, (2 ** 31 - 1) // cols, 2 ** 31 // cols, rows - 1]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([edge, rng.integers(1, rows - 1, 8)]))


def fill(cfg: int, rank: int, rows: int, cols: int, period: int, fmt: str = "bf16") -> torch.Tensor:
    """rows x cols bf16 (or binary16) bits on the device, flat: row r is rank's generator row
    r % period."""
    base = torch.from_numpy(workloads.rows(cfg, rank, 0, period, cols, fmt=fmt).view(np.int16)).to("cuda")
    out = torch.empty(rows * cols, dtype=torch.int16, device="cuda")
    o = out.view(rows, cols)
    for r0 in range(0, rows, period):
        k = min(period, rows - r0)
        o[r0:r0 + k].copy_(base[:k])
    sync()
    return out


def gen_rows(cfg: int, rank: int, rows: np.ndarray, cols: int, period: int,
             fmt: str = "bf16") -> np.ndarray:
    return np.concatenate([workloads.rows(cfg, rank, int(r) % period, 1, cols, fmt=fmt)
                           for r in rows])


def take(t: torch.Tensor, rows: np.ndarray, per_row: int, dtype) -> np.ndarray:
    """The given rows of a flat device tensor with per_row elements per row."""
    idx = torch.from_numpy(rows.astype(np.int64)).to(t.device)
    return host(t.view(-1, per_row).index_select(0, idx), dtype)


def assert_same(got, want, what):
    got, want = np.asarray(got).reshape(-1), np.asarray(want).reshape(-1)
    assert got.shape == want.shape, what
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}"


@pytest.fixture(scope="module")
def x0():
    say(f"large: generating rank 0 of cfg 5 at {ROWS}x{COLS}")
    t = fill(5, 0, ROWS, COLS, P)
    yield t
    del t
    torch.cuda.empty_cache()


def test_i8_quant_dequant_hop_past_2p31(x0):
    n = ROWS * COLS
    assert n > 2 ** 31
    rows = sampled_rows(ROWS, COLS, 1)
    xs = gen_rows(5, 0, rows, COLS, P)
    assert_same(take(x0, rows, COLS, np.uint16), xs, "device input rows")
    say(f"large: i8 quantize + materialize, n={n}")
    q, s = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_quant_i8(x0, q, s, n=n)
    y = empty(n, np.uint16)
    bq.bq_dequant_i8(q, s, y, n=n)
    sync()
    wq, ws = oracle.quant_i8(xs)
    assert_same(take(q, rows, COLS, np.int8), wq, "payload")
    assert_same(take(s, rows, COLS // 128, np.float32), ws, "scales")
    assert_same(take(y, rows, COLS, np.uint16), oracle.dequant_i8(wq, ws), "materialized")
    del y
    say("large: i8 ring hop in place (rank 1's rows as the local partial)")
    x1 = fill(5, 1, ROWS, COLS, P)
    bq.bq_ring_hop_i8(q, s, x1, q, s, n=n)
    sync()
    hq, hs = oracle.ring_hop_i8(wq, ws, gen_rows(5, 1, rows, COLS, P))
    assert_same(take(q, rows, COLS, np.int8), hq, "hop payload")
    assert_same(take(s, rows, COLS // 128, np.float32), hs, "hop scales")


def test_i8_accumulate_two_sources_past_2p31(x0):
    n = ROWS * COLS
    rows = sampled_rows(ROWS, COLS, 2)
    say(f"large: i8 accumulate of 2 sources, n={n}")
    x1 = fill(5, 1, ROWS, COLS, P)
    q0, s0 = empty(n, np.int8), empty(n // 128, np.float32)
    q1, s1 = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_quant_i8(x0, q0, s0, n=n)
    bq.bq_quant_i8(x1, q1, s1, n=n)
    del x1
    y = empty(n, np.uint16)
    bq.bq_dequant_accum_i8([q0, q1], [s0, s1], y, n=n)
    sync()
    a = oracle.quant_i8(gen_rows(5, 0, rows, COLS, P))
    b = oracle.quant_i8(gen_rows(5, 1, rows, COLS, P))
    want = oracle.dequant_accum_i8([a[0], b[0]], [a[1], b[1]])
    assert_same(take(y, rows, COLS, np.uint16), want, "accumulated bf16")


def test_e4m3_b128_past_2p31(x0):
    n = ROWS * COLS
    rows = sampled_rows(ROWS, COLS, 3)
    say(f"large: e4m3 b128 quantize + dequantize, n={n}")
    v, s = empty(n, np.uint8), empty(n // 128, np.float32)
    bq.bq_quant_e4m3_b128(x0, v, s, n=n)
    y = empty(n, np.uint16)
    bq.bq_dequant_e4m3_b128(v, s, y, n=n)
    sync()
    wv, ws = oracle.quant_e4m3_b128(gen_rows(5, 0, rows, COLS, P))
    assert_same(take(v, rows, COLS, np.uint8), wv, "values")
    assert_same(take(s, rows, COLS // 128, np.float32), ws, "scales")
    assert_same(take(y, rows, COLS, np.uint16), oracle.dequant_e4m3_b128(wv, ws), "bf16")


def test_mx_flat_ring_hop_past_2p31(x0):
    """The MXFP8 collective codec (flat layout): quantize, hop in place, materialize."""
    n = ROWS * COLS
    rows = sampled_rows(ROWS, COLS, 4)
    say(f"large: mx flat quantize + hop + dequantize, n={n}")
    v, e = empty(n, np.uint8), empty(n // 32, np.uint8)
    bq.bq_quant_mx_batch([x0], [v], [e], n=n)
    x1 = fill(5, 1, ROWS, COLS, P)
    bq.bq_ring_hop_mx(v, e, x1, v, e, n=n)
    del x1
    y = empty(n, np.uint16)
    bq.bq_dequant_mx_batch([v], [e], [y], n=n)
    sync()
    wv, we = oracle.quant_mx_flat(gen_rows(5, 0, rows, COLS, P))
    hv, he = oracle.ring_hop_mx(wv, we, gen_rows(5, 1, rows, COLS, P))
    assert_same(take(v, rows, COLS, np.uint8), hv, "hop values")
    assert_same(take(e, rows, COLS // 32, np.uint8), he, "hop scales")
    assert_same(take(y, rows, COLS, np.uint16), oracle.dequant_mx_flat(hv, he), "bf16")


def test_mx_2d_past_2p31():
    """The staged-GEMM layout: 49,933 x 43008 bf16 (2^31 values end inside the last row),
    row-gain data, quantized and dequantized in one call each."""
    n = MX_ROWS * MX_COLS
    assert n > 2 ** 31
    rows = sampled_rows(MX_ROWS, MX_COLS, 5)
    say(f"large: mx 2-D quantize + dequantize {MX_ROWS}x{MX_COLS}")
    x = fill(4, 0, MX_ROWS, MX_COLS, MX_P).view(MX_ROWS, MX_COLS)
    v = empty((MX_ROWS, MX_COLS), np.uint8)
    e = empty((MX_ROWS, MX_COLS // 32), np.uint8)
    bq.bq_quant_mx(x, v, e)
    del x
    y = empty((MX_ROWS, MX_COLS), np.uint16)
    bq.bq_dequant_mx(v, e, y)
    sync()
    wv, we = oracle.quant_mx(gen_rows(4, 0, rows, MX_COLS, MX_P))
    assert_same(take(v, rows, MX_COLS, np.uint8), wv, "values")
    assert_same(take(e, rows, MX_COLS // 32, np.uint8), we, "scales")
    assert_same(take(y, rows, MX_COLS, np.uint16), oracle.dequant_mx(wv, we), "bf16")


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_mx_staged_slices_past_2p31(fmt):
    """Six 49,933 x 7168 slices (bf16, or binary16) quantized at offsets 0, 7168, ..., 35840
    of a 49,933 x 43008 staging buffer, whose last rows start past byte 2^31; sampled rows
    equal the oracle's quantization of the concatenated slices."""
    J, K = 6, 7168
    rows = sampled_rows(MX_ROWS, MX_COLS, 6)
    say(f"large: mx staged {fmt} slices {J}x{MX_ROWS}x{K} -> {MX_ROWS}x{MX_COLS}")
    v = empty((MX_ROWS, MX_COLS), np.uint8)
    e = empty((MX_ROWS, MX_COLS // 32), np.uint8)
    quant = bq.bq_quant_mx_slice if fmt == "bf16" else bq.bq_quant_mx_slice_f16
    for j in range(J):
        x = fill(4, j, MX_ROWS, K, MX_P, fmt).view(MX_ROWS, K)
        quant(x, K * j, v, e)
        sync()
        del x
    sub = np.concatenate([gen_rows(4, j, rows, K, MX_P, fmt) for j in range(J)], axis=1)
    wv, we = oracle.quant_mx(sub) if fmt == "bf16" else oracle.quant_mx_f16(sub)
    assert_same(take(v, rows, MX_COLS, np.uint8), wv, "values")
    assert_same(take(e, rows, MX_COLS // 32, np.uint8), we, "scales")


def test_mm_mx_weights_past_2p31_bytes():
    """200 x 49,933 x 43008: the weights hold 2,147,518,464 bytes, so the last weight rows
    start past byte 2^31.  Codes 0 and +-1 with block scales in [2^-1, 2^1] keep every
    block sum and binary32 partial sum exact (|sum| <= 4 K < 2^18 at a 2^-2 grain), so
    sampled output columns, the last included, are compared bit for bit."""
    M, N, K = 200, MX_ROWS, MX_COLS
    assert N * K > 2 ** 31
    rng = np.random.default_rng(77)
    codes = np.array([0x00, 0x38, 0xB8], np.uint8)          # 0, +1, -1
    say(f"large: mm_mx {M}x{N}x{K} (exact operands)")
    xv = codes[rng.integers(0, 3, (M, K), dtype=np.uint8)]
    xe = rng.integers(126, 129, (M, K // 32), dtype=np.uint8)
    wv_base = codes[rng.integers(0, 3, (MX_P, K), dtype=np.uint8)]      # weight row n: n % MX_P
    we_base = rng.integers(126, 129, (MX_P, K // 32), dtype=np.uint8)
    dev = lambda a: torch.from_numpy(a).to("cuda")
    wv, we = torch.empty((N, K), dtype=torch.uint8, device="cuda"), empty((N, K // 32), np.uint8)
    bv, be = dev(wv_base), dev(we_base)
    for r0 in range(0, N, MX_P):
        k = min(MX_P, N - r0)
        wv[r0:r0 + k].copy_(bv[:k])
        we[r0:r0 + k].copy_(be[:k])
    y = empty((M, N), np.uint16)
    bq.bq_mm_mx(dev(xv), dev(xe), wv, we, y)
    sync()
    cols = np.unique(np.concatenate([[0, 2 ** 31 // K - 1, N - 1], rng.integers(1, N - 1, 13)]))
    Y, _ = oracle.mm_mx(xv, xe, wv_base[cols % MX_P], we_base[cols % MX_P])
    assert np.all(np.abs(Y) < 2.0 ** 18)
    want = torch.from_numpy(Y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = host(y, np.uint16)[:, cols]
    assert np.array_equal(got, want), f"{int((got != want).sum())} outputs differ"
