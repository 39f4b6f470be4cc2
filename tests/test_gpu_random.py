"""Randomized GPU parity sweep: many small seeded cases of random shape against the oracle.

Each case draws its sizes (ragged block counts, rows, padded strides, ranks, sources,
owners) and a wide value mix: per-block magnitudes from 2^-130 to 2^90, values spread
20 octaves below their block's top, random signs, 3% zeros, bf16 subnormals and 2%
all-zero blocks.  Every output is compared bit for bit with the oracle, whose inputs are
the same host arrays (payloads for a hop or an accumulate are the oracle's own
quantization of drawn tensors, never the GPU's).  The case about to run is printed
first, so a failure names its seed and shape.

BQ_RANDOM_CASES (default 24) sets the number of seeds per codec family, and a twelfth of it
(at least 12) the number of GEMM shapes; the default seeds are the first ones of any
longer sweep.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from gpu_util import empty, filled, host, say, sync, to_dev

from block_quantized_wire_amd import build as _build

if _build.stale():
    _build.build()
import block_quantized_wire_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = int(os.environ.get("BQ_RANDOM_CASES", "24"))
MM_CASES = max(12, CASES // 12)


def assert_same(got, want, what):
    got, want = np.asarray(got).reshape(-1), np.asarray(want).reshape(-1)
    assert got.shape == want.shape, what
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"got {got[bad[:5]]} want {want[bad[:5]]}"


def draw(rng, n: int, lo: int = -130, hi: int = 90, fmt: str = "bf16") -> np.ndarray:
    """n finite values (n a multiple of 32) as bf16 (or binary16) bit patterns, truncated
    toward zero from binary32; the magnitudes are chosen per 32-value group."""
    groups = n // 32
    top = rng.integers(lo, hi + 1, groups).repeat(32)
    e = top - rng.integers(0, 21, n)
    m = 1.0 + rng.random(n)
    v = np.ldexp(m, e) * np.where(rng.random(n) < 0.5, -1.0, 1.0)
    v[rng.random(n) < 0.03] = 0.0
    v.reshape(groups, 32)[rng.random(groups) < 0.02] = 0.0
    if fmt == "f16":
        v = np.clip(v, -65504.0, 65504.0)
        return v.astype(np.float32).astype(np.float16).view(np.uint16)   # round, then finite
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def blocks(rng, lo=1, hi=300) -> int:
    return 128 * int(rng.integers(lo, hi + 1))


@pytest.mark.parametrize("seed", range(CASES))
def test_random_i8_codec_hop_and_accumulate(seed):
    rng = np.random.default_rng(1000 + seed)
    n = blocks(rng)
    nsrc = int(rng.integers(1, 65))
    in_place = bool(rng.integers(0, 2))
    say(f"random i8 seed={seed} n={n} nsrc={nsrc} hop in place={in_place}")
    x = draw(rng, n)
    q, s = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_quant_i8(to_dev(x), q, s, n=n)
    y = empty(n, np.uint16)
    bq.bq_dequant_i8(q, s, y, n=n)
    sync()
    wq, ws = oracle.quant_i8(x)
    assert_same(host(q, np.int8), wq, "payload")
    assert_same(host(s, np.float32), ws, "scales")
    assert_same(host(y, np.uint16), oracle.dequant_i8(wq, ws), "materialized")
    # hop: the oracle's payload of x plus a drawn local partial
    local = draw(rng, n, lo=-130, hi=89)
    qi, si = to_dev(wq), to_dev(ws)
    if in_place:
        qo, so = qi, si
    else:
        qo, so = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_ring_hop_i8(qi, si, to_dev(local), qo, so, n=n)
    sync()
    hq, hs = oracle.ring_hop_i8(wq, ws, local)
    assert_same(host(qo, np.int8), hq, "hop payload")
    assert_same(host(so, np.float32), hs, "hop scales")
    # accumulate of nsrc payloads in source order
    srcs = [oracle.quant_i8(draw(rng, n, hi=80)) for _ in range(nsrc)]
    ya = empty(n, np.uint16)
    bq.bq_dequant_accum_i8([to_dev(a) for a, _ in srcs], [to_dev(b) for _, b in srcs], ya, n=n)
    sync()
    want = oracle.dequant_accum_i8([a for a, _ in srcs], [b for _, b in srcs])
    assert_same(host(ya, np.uint16), want, "accumulated bf16")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_i8_collectives(seed):
    rng = np.random.default_rng(2000 + seed)
    W = int(rng.integers(1, 9))
    nseg = int(rng.integers(1, 9))
    nsrc = int(rng.integers(1, 17))
    n = W * blocks(rng, 1, 40)
    m = nseg * blocks(rng, 1, 40)
    say(f"random i8 collectives seed={seed} ring W={W} n={n}; owner step nseg={nseg} "
        f"nsrc={nsrc} n={m}")
    parts = [draw(rng, n, hi=80) for _ in range(W)]
    wq, ws, wouts = oracle.ring_allreduce_i8(parts)
    qw, sw = empty(n, np.int8), empty(n // 128, np.float32)
    outs = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_ring_allreduce_i8([to_dev(p) for p in parts], qw, sw, outs, n=n)
    sync()
    assert_same(host(qw, np.int8), wq, "ring payloads")
    assert_same(host(sw, np.float32), ws, "ring scales")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"ring rank {r}")
    srcs = [oracle.quant_i8(draw(rng, m, hi=80)) for _ in range(nsrc)]
    qs, ss = [a for a, _ in srcs], [b for _, b in srcs]
    oq, os_, oys, ored = oracle.a2a_reduce_i8(qs, ss, nseg)
    qo, so, red = empty(m, np.int8), empty(m // 128, np.float32), empty(m, np.uint16)
    ys = [empty(m // nseg, np.uint16) for _ in range(nseg)]
    bq.bq_a2a_reduce_i8(nseg, [to_dev(a) for a in qs], [to_dev(b) for b in ss], qo, so, ys, red)
    sync()
    assert_same(host(qo, np.int8), oq, "owner payload")
    assert_same(host(so, np.float32), os_, "owner scales")
    assert_same(host(red, np.uint16), ored, "owner bf16 sums")
    for j in range(nseg):
        assert_same(host(ys[j], np.uint16), oys[j], f"owner {j} materialization")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_mx_and_e4m3(seed):
    rng = np.random.default_rng(3000 + seed)
    rows = int(rng.integers(1, 41))
    cols = blocks(rng, 1, 20)
    padv, pads = 16 * int(rng.integers(0, 3)), 4 * int(rng.integers(0, 3))
    fmt = "f16" if rng.integers(0, 2) else "bf16"
    n = blocks(rng)
    nsrc = int(rng.integers(1, 65))
    # input and output row padding from a generator of their own, so the draws above and
    # below are the same as without it
    prng = np.random.default_rng(5000 + seed)
    padx, pady = 8 * int(prng.integers(0, 3)), 8 * int(prng.integers(0, 3))
    off, extra, spare = 128 * int(prng.integers(0, 3)), 128 * int(prng.integers(0, 2)), int(prng.integers(0, 3))
    say(f"random mx seed={seed} {fmt} {rows}x{cols} pads=({padv},{pads}) ldx pad {padx} "
        f"ldy pad {pady}; slice at column {off} of {off + cols + extra}, {spare} spare rows; "
        f"flat n={n} nsrc={nsrc}; e4m3-b128")
    # 2-D MXFP8 with padded strides (binary16 input: magnitudes within its range).  The input
    # padding holds NaN bit patterns, so reading it would corrupt a group's scale.
    x = draw(rng, rows * cols, lo=-20, hi=14, fmt=fmt) if fmt == "f16" else draw(rng, rows * cols)
    x = x.reshape(rows, cols)
    xbuf = filled((rows, cols + padx), np.uint16, 0xFF)
    xbuf[:, :cols].copy_(to_dev(x))
    ldv, lds = cols + padv, cols // 32 + pads
    v, e = empty((rows, ldv), np.uint8), empty((rows, lds), np.uint8)
    quant = bq.bq_quant_mx_f16 if fmt == "f16" else bq.bq_quant_mx
    quant(xbuf[:, :cols], v, e, rows=rows, cols=cols, ldx=cols + padx, ldv=ldv, lds=lds)
    ybuf = filled((rows, cols + pady), np.uint16, 0xA5)
    bq.bq_dequant_mx(v, e, ybuf[:, :cols], rows=rows, cols=cols, ldv=ldv, lds=lds, ldy=cols + pady)
    sync()
    wv, we = oracle.quant_mx_f16(x) if fmt == "f16" else oracle.quant_mx(x)
    assert_same(host(v, np.uint8)[:, :cols], wv, "E4M3 values")
    assert_same(host(e, np.uint8)[:, :cols // 32], we, "E8M0 scales")
    y = host(ybuf, np.uint16)
    assert_same(y[:, :cols], oracle.dequant_mx(wv, we), "MX bf16")
    assert np.all(y[:, cols:] == 0xA5A5), "dequantize wrote into the row padding"
    # the same padded input staged as a slice at a 128-column offset of a wider buffer with
    # spare rows: equal to the one-call quantization, every other column and row untouched
    total, cap = off + cols + extra, rows + spare
    sv, se = filled((cap, total), np.uint8, 0x5A), filled((cap, total // 32), np.uint8, 0x5A)
    stage = bq.bq_quant_mx_slice_f16 if fmt == "f16" else bq.bq_quant_mx_slice
    stage(xbuf[:, :cols], off, sv, se, capacity_rows=cap, rows=rows, cols=cols, ldx=cols + padx)
    sync()
    hv, he = host(sv, np.uint8), host(se, np.uint8)
    assert_same(hv[:rows, off:off + cols], wv, "staged slice values")
    assert_same(he[:rows, off // 32:(off + cols) // 32], we, "staged slice scales")
    hv[:rows, off:off + cols] = 0x5A
    he[:rows, off // 32:(off + cols) // 32] = 0x5A
    assert np.all(hv == 0x5A) and np.all(he == 0x5A), "the slice wrote outside its columns or rows"
    # flat MXFP8: hop in place, accumulate
    xf = draw(rng, n, hi=80)
    fv, fe = oracle.quant_mx_flat(xf)
    local = draw(rng, n, hi=80)
    vi, ei = to_dev(fv), to_dev(fe)
    bq.bq_ring_hop_mx(vi, ei, to_dev(local), vi, ei, n=n)
    sync()
    hv, he = oracle.ring_hop_mx(fv, fe, local)
    assert_same(host(vi, np.uint8), hv, "MX hop values")
    assert_same(host(ei, np.uint8), he, "MX hop scales")
    srcs = [oracle.quant_mx_flat(draw(rng, n, hi=80)) for _ in range(nsrc)]
    ya = empty(n, np.uint16)
    bq.bq_dequant_accum_mx([to_dev(a) for a, _ in srcs], [to_dev(b) for _, b in srcs], ya, n=n)
    sync()
    assert_same(host(ya, np.uint16), oracle.dequant_accum_mx([a for a, _ in srcs],
                                                             [b for _, b in srcs]), "MX accumulate")
    # E4M3 128-block codec
    xe = draw(rng, n)
    ev, es = empty(n, np.uint8), empty(n // 128, np.float32)
    bq.bq_quant_e4m3_b128(to_dev(xe), ev, es, n=n)
    ye = empty(n, np.uint16)
    bq.bq_dequant_e4m3_b128(ev, es, ye, n=n)
    sync()
    wev, wes = oracle.quant_e4m3_b128(xe)
    assert_same(host(ev, np.uint8), wev, "E4M3-b128 values")
    assert_same(host(es, np.float32), wes, "E4M3-b128 scales")
    assert_same(host(ye, np.uint16), oracle.dequant_e4m3_b128(wev, wes), "E4M3-b128 bf16")


@pytest.mark.parametrize("seed", range(MM_CASES))
def test_random_mm_mx(seed):
    """Random GEMM shapes (ragged M and N, K up to 2048): operands are the oracle's MXFP8
    quantization of drawn values, within the bound derived from the matrix cores'
    arithmetic and deterministic; plus an exact small-integer case compared bit for bit."""
    from test_gpu_mm_mx import block_max_sum, check_close
    import torch
    rng = np.random.default_rng(4000 + seed)
    M, N = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    K = 128 * int(rng.integers(1, 17))
    say(f"random mm_mx seed={seed} {M}x{N}x{K}")
    xv, xe = oracle.quant_mx(draw(rng, M * K, lo=-30, hi=30).reshape(M, K))
    wv, we = oracle.quant_mx(draw(rng, N * K, lo=-30, hi=30).reshape(N, K))
    Y, S = oracle.mm_mx(xv, xe, wv, we)
    B = block_max_sum(xv, xe, wv, we)
    y = empty((M, N), np.uint16)
    bq.bq_mm_mx(to_dev(xv), to_dev(xe), to_dev(wv), to_dev(we), y)
    y2 = empty((M, N), np.uint16)
    bq.bq_mm_mx(to_dev(xv), to_dev(xe), to_dev(wv), to_dev(we), y2)
    sync()
    got = host(y, np.uint16)
    check_close(got, Y, S, B, K, "outputs")
    assert np.array_equal(got, host(y2, np.uint16)), "not deterministic"
    # exact: codes 0, +-1, +-2 and block scales in [2^-1, 2^1] keep every sum exact
    codes = np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], np.uint8)
    xv = codes[rng.integers(0, 5, (M, K))]
    wv = codes[rng.integers(0, 5, (N, K))]
    xe = rng.integers(126, 129, (M, K // 32)).astype(np.uint8)
    we = rng.integers(126, 129, (N, K // 32)).astype(np.uint8)
    Y, _ = oracle.mm_mx(xv, xe, wv, we)
    want = torch.from_numpy(Y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bq.bq_mm_mx(to_dev(xv), to_dev(xe), to_dev(wv), to_dev(we), y)
    sync()
    assert np.array_equal(host(y, np.uint16), want), "exact case differs"


@pytest.mark.parametrize("seed", range(CASES))
def test_random_mx_mfma_layout(seed):
    """Staged slices with the scales in the scaled-MFMA layout (random rows, spare capacity,
    slice count and widths, padded input rows, bf16 or binary16): values and every layout byte
    against the oracle's map, bytes no slice owns untouched; then the GEMM reading the layout
    (layouts laid out for more rows than M and N) against the GEMM reading row-major scales,
    bit for bit."""
    import torch
    rng = np.random.default_rng(6000 + seed)
    rows = int(rng.integers(1, 41))
    cap = rows + int(rng.integers(0, 21))
    widths = [blocks(rng, 1, 6) for _ in range(int(rng.integers(1, 5)))]
    total = sum(widths) + 128 * int(rng.integers(0, 3))
    fmt = "f16" if rng.integers(0, 2) else "bf16"
    padx = 8 * int(rng.integers(0, 3))
    say(f"random mx mfma layout seed={seed} {fmt} rows={rows} cap={cap} widths={widths} "
        f"total={total} ldx pad {padx}")
    ov = np.full((cap, total), 0xEE, np.uint8)
    oe = np.full(oracle.mx_mfma_bytes(cap, total), 0xEE, np.uint8)
    gv = filled((cap, total), np.uint8, 0xEE)
    ge = filled(oracle.mx_mfma_bytes(cap, total), np.uint8, 0xEE)
    off = 0
    for w in widths:
        x = draw(rng, rows * w, lo=-20, hi=14, fmt=fmt) if fmt == "f16" else draw(rng, rows * w)
        x = x.reshape(rows, w)
        xbuf = filled((rows, w + padx), np.uint16, 0xFF)
        xbuf[:, :w].copy_(to_dev(x))
        oracle.quant_mx_slice_mfma(x, off, ov, oe, cap, f16=fmt == "f16")
        bq.bq_quant_mx_slice_mfma(xbuf[:, :w], off, gv, ge, capacity_rows=cap, total_cols=total,
                                  rows=rows, cols=w, ldx=w + padx, f16=fmt == "f16")
        off += w
    sync()
    assert_same(host(gv, np.uint8), ov, "staged values")
    assert_same(host(ge, np.uint8), oe, "scale layout")
    M, N = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    K = 128 * int(rng.integers(1, 17))
    xrows, wrows = M + int(rng.integers(0, 40)), N + int(rng.integers(0, 40))
    say(f"  gemm {M}x{N}x{K}, layouts for {xrows} and {wrows} rows")
    xv, xe = oracle.quant_mx(draw(rng, M * K, lo=-30, hi=30).reshape(M, K))
    wv, we = oracle.quant_mx(draw(rng, N * K, lo=-30, hi=30).reshape(N, K))
    xl = np.full(oracle.mx_mfma_bytes(xrows, K), 0xFF, np.uint8)
    wl = np.full(oracle.mx_mfma_bytes(wrows, K), 0xFF, np.uint8)
    oracle.mx_scales_to_mfma(xe, xl, -(-xrows // 16))
    oracle.mx_scales_to_mfma(we, wl, -(-wrows // 16))
    y1, y2 = empty((M, N), np.uint16), empty((M, N), np.uint16)
    dxv, dwv = to_dev(xv), to_dev(wv)
    bq.bq_mm_mx(dxv, to_dev(xe), dwv, to_dev(we), y1)
    bq.bq_mm_mx_mfma(dxv, to_dev(xl), dwv, to_dev(wl), y2, xe_rows=xrows, we_rows=wrows)
    sync()
    assert torch.equal(y1, y2), "scaled-MFMA layout GEMM differs from row-major scales"


@pytest.mark.parametrize("nblocks", range(1, 18))
def test_every_tile_residue(nblocks):
    """1..17 blocks: every residue of the block count modulo the 8-block tiles of the
    16-values-per-lane kernels (and the 4-block tiles of the others), for each kernel
    that walks them: INT8 quantize and hop, E4M3-b128 quantize, MXFP8 flat quantize and
    hop, 2-D MXFP8 quantize of one row; bit for bit, and nothing written past the end."""
    import torch
    rng = np.random.default_rng(5000 + nblocks)
    n = 128 * nblocks
    say(f"tile residues nblocks={nblocks}")
    x, local = draw(rng, n, hi=60), draw(rng, n, hi=60)
    pad = 4096                                         # canary bytes past the end
    q = torch.full((n + pad,), 0x5A, dtype=torch.int8, device="cuda")
    s = torch.full((n // 128 + 64,), -1.0, dtype=torch.float32, device="cuda")
    bq.bq_quant_i8(to_dev(x), q, s, n=n)
    sync()
    wq, ws = oracle.quant_i8(x)
    assert_same(host(q, np.int8)[:n], wq, "INT8 payload")
    assert_same(host(s, np.float32)[:n // 128], ws, "INT8 scales")
    assert bool((q[n:] == 0x5A).all()) and bool((s[n // 128:] == -1.0).all()), "INT8 wrote past n"
    bq.bq_ring_hop_i8(q, s, to_dev(local), q, s, n=n)
    sync()
    hq, hs = oracle.ring_hop_i8(wq, ws, local)
    assert_same(host(q, np.int8)[:n], hq, "hop payload")
    assert_same(host(s, np.float32)[:n // 128], hs, "hop scales")
    assert bool((q[n:] == 0x5A).all()) and bool((s[n // 128:] == -1.0).all()), "hop wrote past n"
    v = torch.full((n + pad,), 0xA5, dtype=torch.uint8, device="cuda")
    es = torch.full((n // 128 + 64,), -1.0, dtype=torch.float32, device="cuda")
    bq.bq_quant_e4m3_b128(to_dev(x), v, es, n=n)
    sync()
    wv, wes = oracle.quant_e4m3_b128(x)
    assert_same(host(v, np.uint8)[:n], wv, "E4M3-b128 values")
    assert_same(host(es, np.float32)[:n // 128], wes, "E4M3-b128 scales")
    assert bool((v[n:] == 0xA5).all()), "E4M3-b128 wrote past n"
    e = torch.full((n // 32 + pad,), 0xA5, dtype=torch.uint8, device="cuda")
    bq.bq_quant_mx_batch([to_dev(x)], [v], [e], n=n)
    sync()
    fv, fe = oracle.quant_mx_flat(x)
    assert_same(host(v, np.uint8)[:n], fv, "MX flat codes")
    assert_same(host(e, np.uint8)[:n // 32], fe, "MX flat scales")
    assert bool((v[n:] == 0xA5).all()) and bool((e[n // 32:] == 0xA5).all()), "MX wrote past n"
    bq.bq_ring_hop_mx(v, e, to_dev(local), v, e, n=n)
    sync()
    hv, he = oracle.ring_hop_mx(fv, fe, local)
    assert_same(host(v, np.uint8)[:n], hv, "MX hop codes")
    assert_same(host(e, np.uint8)[:n // 32], he, "MX hop scales")
    assert bool((v[n:] == 0xA5).all()) and bool((e[n // 32:] == 0xA5).all()), "MX hop wrote past n"
    v2 = torch.full((1, n + 128), 0xA5, dtype=torch.uint8, device="cuda")
    e2 = torch.full((1, n // 32 + 4), 0xA5, dtype=torch.uint8, device="cuda")
    bq.bq_quant_mx(to_dev(x.reshape(1, n)), v2, e2, rows=1, cols=n)
    sync()
    assert_same(host(v2, np.uint8)[0, :n], fv, "MX 2-D codes")
    assert_same(host(e2, np.uint8)[0, :n // 32], fe, "MX 2-D scales")
    assert bool((v2[0, n:] == 0xA5).all()) and bool((e2[0, n // 32:] == 0xA5).all()), "MX 2-D wrote past cols"


@pytest.mark.parametrize("seed", range(MM_CASES))
def test_random_mm_wide_tiles(seed):
    """Random ragged shapes the launcher runs on 256-column tiles (drawn until the device's
    compute units make that the choice), K up to 1024: the product equals, bit for bit, the
    same product computed in 224-column pieces (which take 224-column tiles), with row-major
    and with MFMA-layout scales; a few outputs against the oracle's bound."""
    from test_gpu_mm_mx import block_max_sum, check_close
    import torch
    rng = np.random.default_rng(8000 + seed)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for _ in range(200):
        M, N = int(rng.integers(1, 4700)), int(rng.integers(2000, 4700))
        if bq.bq_mm_tile_cols(M, N, cus) == 256:
            break
    else:
        pytest.skip(f"no drawn shape takes 256-column tiles on {cus} compute units")
    K = 128 * int(rng.integers(1, 9))
    say(f"random mm wide tiles seed={seed} {M}x{N}x{K}")
    x = draw(rng, M * K, lo=-30, hi=30).reshape(M, K)
    w = draw(rng, N * K, lo=-30, hi=30).reshape(N, K)
    dx, dw = to_dev(x), to_dev(w)
    xv, xe = empty((M, K), np.uint8), empty((M, K // 32), np.uint8)
    wv, we = empty((N, K), np.uint8), empty((N, K // 32), np.uint8)
    bq.bq_quant_mx(dx, xv, xe)
    bq.bq_quant_mx(dw, wv, we)
    xl = filled(bq.bq_mx_scale_mfma_bytes(M, K), np.uint8, 0xEE)
    wl = filled(bq.bq_mx_scale_mfma_bytes(N, K), np.uint8, 0xEE)
    bq.bq_quant_mx_slice_mfma(dx, 0, xv, xl)
    bq.bq_quant_mx_slice_mfma(dw, 0, wv, wl)
    whole, whole_l = empty((M, N), np.uint16), empty((M, N), np.uint16)
    bq.bq_mm_mx(xv, xe, wv, we, whole)
    bq.bq_mm_mx_mfma(xv, xl, wv, wl, whole_l)
    pieces, pieces_l = empty((M, N), np.uint16), empty((M, N), np.uint16)
    for c in range(0, N, 224):
        n = min(224, N - c)
        assert bq.bq_mm_tile_cols(M, n, cus) == 224
        bq.bq_mm_mx(xv, xe, wv[c:c + n], we[c:c + n], pieces[:, c:c + n])
        bq.bq_mm_mx_mfma(xv, xl, wv[c:c + n], wl[(c // 16) * 256:], pieces_l[:, c:c + n],
                         we_rows=N)
    sync()
    assert torch.equal(whole, pieces), "256- and 224-column tiles differ (row-major scales)"
    assert torch.equal(whole_l, pieces_l), "256- and 224-column tiles differ (MFMA layout)"
    assert torch.equal(whole, whole_l), "the scale layouts give different products"
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 6)]))
    ov, oe = oracle.quant_mx(np.ascontiguousarray(x[rows]))
    pv, pe = oracle.quant_mx(np.ascontiguousarray(w[cols]))
    Y, S = oracle.mm_mx(ov, oe, pv, pe)
    check_close(host(whole, np.uint16)[np.ix_(rows, cols)], Y, S, block_max_sum(ov, oe, pv, pe),
                K, "sampled outputs")
