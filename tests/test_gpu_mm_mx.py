"""GPU parity of the dense MXFP8 GEMM from staged inputs against the CPU oracle.

The oracle is the definition Y = X W^T on the exact operand values (float64).  The
matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, measured on MI355X) form every product
exactly but sum the 32 products of one scale block in a fixed-point window that keeps 13
bits below the block's largest product and truncates the rest; the block sums, scaled,
are combined and accumulated in binary32, and the kernel rounds to bf16 once.  Two kinds
of check follow from that:

  * bit for bit, on operands whose block sums and binary32 partial sums are exact (small
    integer codes, block scales within two octaves): y == bf16_rne(Y);
  * on realistic data, the worst case of that arithmetic,
        |y - Y| <= 2^-8 |Y| + 2^-8 sum_b max_b |p| + (ceil(K/32) + 2) 2^-24 S + 2^-133,
    with S = sum |p| and max_b over the products of scale block b (32 window ulps per
    block, each at most 2^-13 of the block's largest product; bf16 half-ulp doubled),
    plus a normalized RMS error below 2^-8 (an empirical sanity bound: bf16 rounding
    alone contributes about 2^-10).

Operands for the oracle come from the oracle's own quantizer applied to the generators'
rows, never from the GPU.
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


def f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def block_max_sum(xv, xe, wv, we) -> np.ndarray:
    """sum over the 32-column scale blocks of max |x_k w_k|, for every (m, n)."""
    X = oracle.mx_values_f64(xv, xe)
    Wt = oracle.mx_values_f64(wv, we)
    M, K = X.shape
    out = np.zeros((M, Wt.shape[0]))
    Xb = np.abs(X).reshape(M, K // 32, 32)
    Wb = np.abs(Wt).reshape(Wt.shape[0], K // 32, 32)
    for m in range(M):
        out[m] = (Xb[m][None, :, :] * Wb).max(axis=2).sum(axis=1)
    return out


def check_close(y_bits, Y, S, B, K, what, rms_bound=2.0 ** -8):
    y = f32(y_bits).astype(np.float64)
    tol = 2.0 ** -8 * np.abs(Y) + 2.0 ** -8 * B + (-(-K // 32) + 2) * 2.0 ** -24 * S + 2.0 ** -133
    err = np.abs(y - Y)
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, f"{what}: {bad.size} outputs out of tolerance, worst " \
                          f"{float((err / np.maximum(tol, 1e-300)).max()):.3g} x tol"
    # normalized RMS error: bf16 rounding alone gives about 2^-10; the bound leaves room
    # for the matrix cores' truncation
    nrms = float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(Y ** 2)), 1e-300))
    assert nrms < rms_bound, f"{what}: normalized RMS error {nrms:.3g}"


def gpu_mm(xv, xe, wv, we, M, N, K, pad=0):
    y = filled((M, N + pad), np.uint16, 0x7F)
    bq.bq_mm_mx(to_dev(xv), to_dev(xe), to_dev(wv), to_dev(we), y, M=M, N=N, K=K)
    sync()
    return host(y, np.uint16)


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (17, 48, 256), (130, 272, 384), (128, 128, 1024),
                                   (257, 129, 640), (64, 300, 2048)])
def test_mm_mx_small_shapes(M, N, K):
    say(f"mm_mx {M}x{N}x{K}")
    x = workloads.rows(4, 1, 0, M, K)
    w = workloads.rows(6, 2, 0, N, K)
    xv, xe = oracle.quant_mx(x)
    wv, we = oracle.quant_mx(w)
    Y, S = oracle.mm_mx(xv, xe, wv, we)
    B = block_max_sum(xv, xe, wv, we)
    pad = 8
    y = gpu_mm(xv, xe, wv, we, M, N, K, pad=pad)
    check_close(y[:, :N], Y, S, B, K, "outputs")
    assert np.all(y[:, N:] == 0x7F7F), "wrote past N"
    y2 = gpu_mm(xv, xe, wv, we, M, N, K, pad=pad)
    assert np.array_equal(y, y2), "not deterministic"


@pytest.mark.parametrize("M,N,K", [(96, 80, 1024), (33, 130, 384), (128, 256, 2048)])
def test_mm_mx_exact_small_integers(M, N, K):
    """Codes 0, +-1, +-2, +-3 with every block scale in [2^-2, 2^2]: each block sum stays
    inside the matrix cores' window and every binary32 partial sum is exact, so the result
    is the exact sum rounded to bf16 once -- compared bit for bit.  Distinct scales per
    row, column and block pin which scale byte meets which 32 products."""
    say(f"mm_mx exact small integers {M}x{N}x{K}")
    rng = np.random.default_rng(21 + K)
    codes = np.array([0x00, 0x38, 0x40, 0x44, 0xB8, 0xC0, 0xC4], np.uint8)   # 0, +-1, +-2, +-3
    xv = codes[rng.integers(0, codes.size, (M, K))]
    wv = codes[rng.integers(0, codes.size, (N, K))]
    xe = rng.integers(125, 130, (M, K // 32)).astype(np.uint8)
    we = rng.integers(125, 130, (N, K // 32)).astype(np.uint8)
    Y, _ = oracle.mm_mx(xv, xe, wv, we)
    assert np.all(np.abs(Y) < 2.0 ** 20)                       # partial sums exact in binary32
    want = torch.from_numpy(Y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = gpu_mm(xv, xe, wv, we, M, N, K)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("M,N,K,pad_xe,pad_we", [(130, 272, 384, 12, 4), (257, 129, 640, 12, 4),
                                                 (130, 272, 1024, 16, 32), (257, 129, 2048, 12, 4)])
def test_mm_mx_padded_strides_match_dense(M, N, K, pad_xe, pad_we):
    """Every leading dimension padded: values by multiples of 16 bytes, scales by multiples
    of 4, the output by an odd count.  The value padding holds the E4M3 NaN code and the
    scale padding the E8M0 NaN byte, so a read past a row's K columns would show.  The
    result equals the dense-stride launch bit for bit, and the output padding is untouched.
    K = 1024 with 16-byte scale strides takes the grouped scale loads (4 K steps per load);
    K = 2048 with 4-byte ones falls back to per-step scales; both equal the dense launch."""
    say(f"mm_mx padded strides {M}x{N}x{K} scale pads ({pad_xe},{pad_we})")
    x = workloads.rows(4, 3, 0, M, K)
    w = workloads.rows(6, 4, 0, N, K)
    xv, xe = oracle.quant_mx(x)
    wv, we = oracle.quant_mx(w)
    dense = gpu_mm(xv, xe, wv, we, M, N, K)

    def padded(a, extra, byte):
        buf = filled((a.shape[0], a.shape[1] + extra), np.uint8, byte)
        buf[:, :a.shape[1]].copy_(to_dev(a))
        return buf[:, :a.shape[1]]

    xvp, wvp = padded(xv, 256, 0x7F), padded(wv, 48, 0xFF)
    xep, wep = padded(xe, pad_xe, 0xFF), padded(we, pad_we, 0xFF)
    assert xvp.stride(0) == K + 256 and wep.stride(0) == K // 32 + pad_we
    y = filled((M, N + 13), np.uint16, 0x5A)
    bq.bq_mm_mx(xvp, xep, wvp, wep, y[:, :N], M=M, N=N, K=K)
    sync()
    got = host(y, np.uint16)
    assert np.array_equal(got[:, :N], dense), "padded strides change the result"
    assert np.all(got[:, N:] == 0x5A5A), "wrote into the output padding"
    Y, S = oracle.mm_mx(xv, xe, wv, we)
    check_close(got[:, :N], Y, S, block_max_sum(xv, xe, wv, we), K, "outputs")


def test_mm_mx_staged_full_size_sampled():
    """The staged projection geometry: six 4096x7168 bf16 slices quantized into a 4096 x
    43008 staging buffer, times 7168 x 43008 MXFP8 weights.  The GEMM of the staged buffer
    equals, bit for bit, the GEMM of the one-call quantization of the concatenation, and
    sampled outputs agree with the oracle."""
    M, N, S_, C = 4096, 7168, 6, 7168
    K = S_ * C
    say(f"mm_mx staged {M}x{N}x{K}")
    xs = [workloads.rows(4, j, 0, M, C) for j in range(S_)]
    xv = empty((M, K), np.uint8)
    xe = empty((M, K // 32), np.uint8)
    for j in range(S_):
        bq.bq_quant_mx_slice(to_dev(xs[j]), j * C, xv, xe)
    w = workloads.rows(6, 7, 0, N, K)
    wv, we = empty((N, K), np.uint8), empty((N, K // 32), np.uint8)
    bq.bq_quant_mx(to_dev(w), wv, we)
    y = empty((M, N), np.uint16)
    bq.bq_mm_mx(xv, xe, wv, we, y)
    cat = torch.cat([to_dev(x) for x in xs], dim=1)
    xv1, xe1 = empty((M, K), np.uint8), empty((M, K // 32), np.uint8)
    bq.bq_quant_mx(cat, xv1, xe1)
    y1 = empty((M, N), np.uint16)
    bq.bq_mm_mx(xv1, xe1, wv, we, y1)
    sync()
    assert torch.equal(y, y1), "staged and concatenated GEMM outputs differ"
    del cat, xv1, xe1, y1
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, M - 1], rng.choice(M, 10, replace=False)])
    cols = np.concatenate([[0, N - 1], rng.choice(N, 10, replace=False)])
    xr = np.concatenate([x[rows] for x in xs], axis=1)
    ov, oe = oracle.quant_mx(np.ascontiguousarray(xr))
    pv, pe = oracle.quant_mx(np.ascontiguousarray(w[cols]))
    Y, S = oracle.mm_mx(ov, oe, pv, pe)
    B = block_max_sum(ov, oe, pv, pe)
    got = host(y, np.uint16)[np.ix_(rows, cols)]
    check_close(got, Y, S, B, K, "sampled outputs")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 384), (4096, 4096, 1024), (4000, 4000, 640)])
def test_mm_mx_tile_widths_agree(M, N, K):
    """The launcher picks 256- or 224-column tiles by how well they fill the compute units:
    a 4096 x 4096 product takes 256-column tiles (16 x 16 tiles, one round on 256 units,
    where 224-column tiles would make 304 and two rounds), and the same product computed in
    224-column pieces takes 224-column tiles.  Every output is the same sum in the same
    order either way, so the two agree bit for bit, for both scale layouts; sampled outputs
    agree with the oracle.  K = 384 and 640 stage each step's scales with its operands,
    K = 1024 four steps at once; 4000 x 4000 leaves ragged row and column tiles (still 16 x 16
    tiles of 256 against 16 x 18 of 224)."""
    say(f"mm_mx tile widths {M}x{N}x{K}")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if bq.bq_mm_tile_cols(M, N, cus) != 256:
        pytest.skip(f"{M}x{N} does not take 256-column tiles on {cus} compute units")
    assert bq.bq_mm_tile_cols(M, min(224, N), cus) == 224
    x = workloads.rows(4, 3, 0, M, K)
    w = workloads.rows(6, 4, 0, N, K)
    dx, dw = to_dev(x), to_dev(w)
    xv, xe = empty((M, K), np.uint8), empty((M, K // 32), np.uint8)
    wv, we = empty((N, K), np.uint8), empty((N, K // 32), np.uint8)
    bq.bq_quant_mx(dx, xv, xe)
    bq.bq_quant_mx(dw, wv, we)
    xl = filled(bq.bq_mx_scale_mfma_bytes(M, K), np.uint8, 0xEE)
    wl = filled(bq.bq_mx_scale_mfma_bytes(N, K), np.uint8, 0xEE)
    bq.bq_quant_mx_slice_mfma(dx, 0, xv, xl)
    bq.bq_quant_mx_slice_mfma(dw, 0, wv, wl)
    whole = filled((M, N), np.uint16, 0x7F)
    bq.bq_mm_mx(xv, xe, wv, we, whole)
    whole_l = filled((M, N), np.uint16, 0x7F)
    bq.bq_mm_mx_mfma(xv, xl, wv, wl, whole_l)
    pieces = filled((M, N), np.uint16, 0x7F)
    pieces_l = filled((M, N), np.uint16, 0x7F)
    for c in range(0, N, 224):
        n = min(224, N - c)
        bq.bq_mm_mx(xv, xe, wv[c:c + n], we[c:c + n], pieces[:, c:c + n])
        # a piece of the layout starts at its first 16-row block; the blocks per group stay N's
        bq.bq_mm_mx_mfma(xv, xl, wv[c:c + n], wl[(c // 16) * 256:], pieces_l[:, c:c + n],
                         we_rows=N)
    sync()
    assert torch.equal(whole, pieces), "256- and 224-column tiles differ (row-major scales)"
    assert torch.equal(whole_l, pieces_l), "256- and 224-column tiles differ (MFMA layout)"
    assert torch.equal(whole, whole_l), "the scale layouts give different products"
    rng = np.random.default_rng(9)
    rows = np.concatenate([[0, M - 1], rng.choice(M, 12, replace=False)])
    cols = np.concatenate([[0, 223, 224, 255, 256, N - 1], rng.choice(N, 12, replace=False)])
    ov, oe = oracle.quant_mx(np.ascontiguousarray(x[rows]))
    pv, pe = oracle.quant_mx(np.ascontiguousarray(w[cols]))
    Y, S = oracle.mm_mx(ov, oe, pv, pe)
    got = host(whole, np.uint16)[np.ix_(rows, cols)]
    check_close(got, Y, S, block_max_sum(ov, oe, pv, pe), K, "sampled outputs")
