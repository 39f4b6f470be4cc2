"""GPU parity of the MXFP8 scale layout for the scaled matrix instruction.

bq_quant_mx_slice_mfma(_f16) must write exactly what the oracle's slice quantizer and its
layout map give -- values and every layout byte, bytes it does not own untouched --
staged slices must equal the one-call quantization in that layout, the layout's
dequantizer must equal the row-major one, and the GEMM reading the layout must give the
same bits as the GEMM reading row-major scales (and the oracle's bits where the
arithmetic is exact).  Expected values come from `oracle` only.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import empty, filled, host, say, sync, to_dev

from block_quantized_wire_amd import build as _build

if _build.stale():
    _build.build()
import block_quantized_wire_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu


def layout_canary(rows: int, cols: int) -> tuple[np.ndarray, torch.Tensor]:
    n = oracle.mx_mfma_bytes(rows, cols)
    assert bq.bq_mx_scale_mfma_bytes(rows, cols) == n
    return np.full(n, 0xEE, np.uint8), filled(n, np.uint8, 0xEE)


@pytest.mark.parametrize("rows,cap,widths,f16", [
    (40, 48, [384] * 6, False),            # 128-column offsets that split 512-column groups
    (17, 17, [128, 256, 640], False),      # ragged rows, total 1024
    (33, 64, [512, 128, 384, 896], False),
    (9, 16, [256, 384, 128], True),        # binary16 input
])
def test_quant_mx_slice_mfma_matches_the_oracle(rows, cap, widths, f16):
    total = sum(widths)
    say(f"quant_mx_slice_mfma rows={rows} cap={cap} widths={widths} f16={f16}")
    cfgs = [workloads.rows(4, j, 0, rows, w, fmt="f16" if f16 else "bf16")
            for j, w in enumerate(widths)]
    ov = np.full((cap, total), 0xEE, np.uint8)
    oe, ge = layout_canary(cap, total)
    gv = filled((cap, total), np.uint8, 0xEE)
    off = 0
    for x, w in zip(cfgs, widths):
        oracle.quant_mx_slice_mfma(x, off, ov, oe, cap, f16=f16)
        bq.bq_quant_mx_slice_mfma(to_dev(x), off, gv, ge, capacity_rows=cap, total_cols=total,
                                  f16=f16)
        off += w
    sync()
    assert np.array_equal(host(gv, np.uint8), ov), "values"
    assert np.array_equal(host(ge, np.uint8), oe), "scale layout (canary bytes included)"


def test_dequant_mx_mfma_equals_row_major_and_oracle():
    """Every E4M3 code against E8M0 bytes 0..254: the layout's dequantizer gives the same
    bits as the row-major one and the oracle."""
    say("dequant_mx_mfma: every code x every scale byte")
    rows, cols = 255, 256 * 4
    v = np.tile(np.arange(256, dtype=np.uint8), (rows, cols // 256))
    v[(v & 0x7F) == 0x7F] = 0x00                              # no NaN codes
    e = (np.arange(rows)[:, None] + np.arange(cols // 32)[None, :]) % 255
    e = e.astype(np.uint8)
    want = oracle.dequant_mx(v, e)
    lay = np.full(oracle.mx_mfma_bytes(rows, cols), 0x7F, np.uint8)
    oracle.mx_scales_to_mfma(e, lay, -(-rows // 16))
    y1 = empty((rows, cols), np.uint16)
    y2 = empty((rows, cols), np.uint16)
    bq.bq_dequant_mx(to_dev(v), to_dev(e), y1)
    bq.bq_dequant_mx_mfma(to_dev(v), to_dev(lay), y2, scale_rows=rows)
    sync()
    assert np.array_equal(host(y2, np.uint16), want)
    assert np.array_equal(host(y1, np.uint16), host(y2, np.uint16))


def gemm_pair(xv, xe, wv, we, M, N, K):
    """(row-major-scale GEMM, MFMA-layout GEMM) on the same operands."""
    xl = np.full(oracle.mx_mfma_bytes(M, K), 0xFF, np.uint8)
    wl = np.full(oracle.mx_mfma_bytes(N, K), 0xFF, np.uint8)
    oracle.mx_scales_to_mfma(xe, xl, -(-M // 16))
    oracle.mx_scales_to_mfma(we, wl, -(-N // 16))
    y1 = filled((M, N), np.uint16, 0x7F)
    y2 = filled((M, N), np.uint16, 0x7F)
    dxv, dwv = to_dev(xv), to_dev(wv)
    bq.bq_mm_mx(dxv, to_dev(xe), dwv, to_dev(we), y1, M=M, N=N, K=K)
    bq.bq_mm_mx_mfma(dxv, to_dev(xl), dwv, to_dev(wl), y2, xe_rows=M, we_rows=N, M=M, N=N, K=K)
    sync()
    return host(y1, np.uint16), host(y2, np.uint16)


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (17, 48, 256), (130, 272, 384), (128, 128, 1024),
                                   (257, 129, 640), (64, 300, 2048), (96, 80, 1152)])
def test_mm_mx_mfma_equals_row_major_scales(M, N, K):
    """The padding of a partial 512-column group is the E8M0 NaN byte 0xFF, so a scale read
    from it would show."""
    say(f"mm_mx_mfma {M}x{N}x{K}")
    x = workloads.rows(4, 11, 0, M, K)
    w = workloads.rows(6, 12, 0, N, K)
    xv, xe = oracle.quant_mx(x)
    wv, we = oracle.quant_mx(w)
    y1, y2 = gemm_pair(xv, xe, wv, we, M, N, K)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("M,N,K", [(96, 80, 1152), (33, 130, 384)])
def test_mm_mx_mfma_exact_small_integers(M, N, K):
    """Codes 0, +-1, +-2, +-3 and block scales in [2^-2, 2^2]: every sum exact, so the
    result is the oracle's exact sum rounded to bf16 once, bit for bit."""
    say(f"mm_mx_mfma exact small integers {M}x{N}x{K}")
    rng = np.random.default_rng(31 + K)
    codes = np.array([0x00, 0x38, 0x40, 0x44, 0xB8, 0xC0, 0xC4], np.uint8)
    xv = codes[rng.integers(0, codes.size, (M, K))]
    wv = codes[rng.integers(0, codes.size, (N, K))]
    xe = rng.integers(125, 130, (M, K // 32)).astype(np.uint8)
    we = rng.integers(125, 130, (N, K // 32)).astype(np.uint8)
    Y, _ = oracle.mm_mx(xv, xe, wv, we)
    want = torch.from_numpy(Y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, y2 = gemm_pair(xv, xe, wv, we, M, N, K)
    assert np.array_equal(y2, want)


def test_staged_projection_in_the_mfma_layout():
    """The staged projection geometry: six 4096x7168 bf16 slices into a 4096 x 43008 staging
    buffer with the scales in the MFMA layout.  Staged == one-call quantization of the
    concatenation (values and layout, bit for bit); the layout == the oracle's map of the
    row-major staged scales; the GEMM with 7168 x 43008 weights in the layout == the GEMM
    with row-major scales, bit for bit, at K = 43008 and at K = 42880 (not a multiple of
    512, where the row-major GEMM fetches scales per K step)."""
    M, N, C, S_ = 4096, 7168, 7168, 6
    K = C * S_
    say(f"staged projection in the MFMA layout {M}x{N}x{K}")
    xs = [to_dev(workloads.rows(4, j, 0, M, C)) for j in range(S_)]
    xv = empty((M, K), np.uint8)
    xl = filled(bq.bq_mx_scale_mfma_bytes(M, K), np.uint8, 0xEE)
    for j in range(S_):
        bq.bq_quant_mx_slice_mfma(xs[j], j * C, xv, xl)
    cat = torch.cat(xs, dim=1)
    xv1 = empty((M, K), np.uint8)
    xl1 = filled(bq.bq_mx_scale_mfma_bytes(M, K), np.uint8, 0xEE)
    bq.bq_quant_mx_slice_mfma(cat, 0, xv1, xl1)
    xe_rm = empty((M, K // 32), np.uint8)
    xv_rm = empty((M, K), np.uint8)
    bq.bq_quant_mx(cat, xv_rm, xe_rm)
    sync()
    assert torch.equal(xv, xv1) and torch.equal(xl, xl1), "staged != concatenated"
    assert torch.equal(xv, xv_rm), "values differ from the row-major quantizer"
    lay = np.full(oracle.mx_mfma_bytes(M, K), 0xEE, np.uint8)
    oracle.mx_scales_to_mfma(host(xe_rm, np.uint8), lay, M // 16)
    assert np.array_equal(host(xl, np.uint8), lay), "layout != oracle map of row-major scales"
    del cat, xv1, xl1, xs
    w = to_dev(workloads.rows(6, 17, 0, N, K))
    wv = empty((N, K), np.uint8)
    we_rm = empty((N, K // 32), np.uint8)
    bq.bq_quant_mx(w, wv, we_rm)
    wl = filled(bq.bq_mx_scale_mfma_bytes(N, K), np.uint8, 0xEE)
    bq.bq_quant_mx_slice_mfma(w, 0, empty((N, K), np.uint8), wl)
    del w
    for k in (K, K - 128):
        say(f"  GEMM K={k}")
        y1 = empty((M, N), np.uint16)
        y2 = empty((M, N), np.uint16)
        bq.bq_mm_mx(xv, xe_rm, wv, we_rm, y1, K=k)
        bq.bq_mm_mx_mfma(xv, xl, wv, wl, y2, K=k)
        sync()
        assert torch.equal(y1, y2), f"K={k}: MFMA-layout GEMM differs from row-major"
