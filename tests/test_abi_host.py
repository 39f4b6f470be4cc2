"""The C ABI on the host: the library loads, exports every declared entry point, and
rejects every invalid argument with its status code before anything is launched.

No call here reaches a kernel launch: every case fails validation, so the tests run
without a GPU.  The addresses used are never dereferenced.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

from block_quantized_wire_amd import build as _build  # noqa: E402

if _build.stale():
    _build.build()

import block_quantized_wire_amd as bq  # noqa: E402

# Every call below passes fake device addresses and must fail validation.  Should a case
# be wrong and validate, the call would launch; with a GPU present that launch would touch
# the fake addresses, so the module only runs where no GPU is visible.
import torch  # noqa: E402

if torch.cuda.device_count() > 0:
    pytest.skip("host-only ABI tests run where no GPU is visible", allow_module_level=True)

L = bq.lib
OK, NULL, SIZE, ALIGN, BOUNDS, NSRC, ALIAS = range(7)
A = 1 << 32          # a 16-byte aligned fake device address
S = 0                # default stream


def arr(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "blockq.h")).read()
    return sorted(set(re.findall(r"\b(bq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = declared_symbols()
    assert len(names) >= 18
    for name in names:
        assert hasattr(L, name), name


def test_gemm_tile_width_rule():
    """Rounds of one tile per compute unit times the tile width, the smaller wins, ties to 256."""
    f = bq.bq_mm_tile_cols
    assert f(4096, 7168, 256) == 224     # 512 tiles of 224 (2 rounds) against 448 of 256 (2 rounds)
    assert f(4096, 4096, 256) == 256     # 256 tiles of 256 (1 round) against 304 of 224 (2)
    assert f(4000, 4000, 256) == 256     # ragged: 16 x 16 against 16 x 18
    assert f(1, 16, 256) == 224          # one round either way: the narrower tile is shorter
    assert f(256, 1792, 1) == 256        # 8 tiles of 224 = 7 tiles of 256 in time: a tie
    assert f(256, 1793, 1) == 224        # 9 x 224 = 2016 against 8 x 256 = 2048
    assert f(4096, 7168, 304) == 224
    for bad in ((0, 16, 256), (16, 0, 256), (1 << 31, 16, 256), (16, 1 << 31, 256), (16, 16, 0)):
        assert f(*bad) == -1, bad


def test_host_helpers():
    assert L.bq_wire_bytes_b128(128) == 132
    assert L.bq_wire_bytes_b128(512 * 7168) == 132 * 512 * 56
    assert L.bq_wire_bytes_b128(0) == 0
    assert L.bq_wire_bytes_b128(100) == -1 and L.bq_wire_bytes_b128(-128) == -1
    assert bq.bq_mx_staging_bytes(4096, 43008) == (4096 * 43008, 4096 * 1344)
    with pytest.raises(bq.BlockqError) as e:
        bq.bq_mx_staging_bytes(4096, 100)
    assert e.value.status == SIZE
    assert bq.bq_status_str(0) == "ok"
    assert "alias" in bq.bq_status_str(6) or "overlap" in bq.bq_status_str(6)
    assert "gfx950" in bq.bq_version()


def test_quant_i8_errors():
    n = 1024
    assert L.bq_quant_i8(A, 100, A + 8192, A + 16384, S) == SIZE
    assert L.bq_quant_i8(A, -128, A + 8192, A + 16384, S) == SIZE
    assert L.bq_quant_i8(A, 0, A + 8192, A + 16384, S) == OK          # empty: nothing to do
    assert L.bq_quant_i8(None, n, A + 8192, A + 16384, S) == NULL
    assert L.bq_quant_i8(A, n, None, A + 16384, S) == NULL
    assert L.bq_quant_i8(A + 8, n, A + 8192, A + 16384, S) == ALIGN
    assert L.bq_quant_i8(A, n, A + 8200, A + 16384, S) == ALIGN
    assert L.bq_quant_i8(A, n, A + 8192, A + 16386, S) == ALIGN
    assert L.bq_quant_i8(A, n, A + 1024, A + 16384, S) == ALIAS      # q inside x
    assert L.bq_quant_i8(A, n, A + 8192, A + 8192 + 512, S) == ALIAS  # scales inside q


def test_dequant_and_e4m3_errors():
    n = 1024
    assert L.bq_dequant_i8(A, A + 4096, 130, A + 8192, S) == SIZE
    assert L.bq_dequant_i8(A, None, n, A + 8192, S) == NULL
    assert L.bq_dequant_i8(A, A + 4096, n, A + 4, S) == ALIGN
    assert L.bq_dequant_i8(A, A + 4096, n, A + 512, S) == ALIAS
    assert L.bq_quant_e4m3_b128(A, n, A + 1024, A + 8192, S) == ALIAS
    assert L.bq_quant_e4m3_b128(A, n, None, A + 8192, S) == NULL
    assert L.bq_dequant_e4m3_b128(A, A + 4096, n, A + 4096 + 16, S) == ALIAS
    assert L.bq_dequant_e4m3_b128(A, A + 4096, 7, A + 8192, S) == SIZE


def test_batch_counts_and_cross_segment_overlap():
    n = 1024
    x = arr(A, A + 4096)
    q = arr(A + 8192, A + 8192 + 1024)
    s = arr(A + 16384, A + 16384 + 64)
    assert L.bq_quant_i8_batch(0, x, n, q, s, S) == NSRC
    assert L.bq_quant_i8_batch(17, x, n, q, s, S) == NSRC
    q_bad = arr(A + 8192, A + 8192 + 512)          # second segment's q overlaps the first's
    assert L.bq_quant_i8_batch(2, x, n, q_bad, s, S) == ALIAS
    y = arr(A + 32768, A + 32768 + 1024)            # outputs overlap each other
    assert L.bq_dequant_i8_batch(2, q, s, n, y, S) == ALIAS


def test_ring_hop_in_place_rules():
    n = 1024
    qi, si, loc = A, A + 4096, A + 8192
    # partial overlap of q_out with q_in
    assert L.bq_ring_hop_i8(qi, si, loc, n, qi + 16, si, S) == ALIAS
    # q in place but scales not in place (and not disjoint either)
    assert L.bq_ring_hop_i8(qi, si, loc, n, qi, si + 4, S) == ALIAS
    # q in place, scales to a disjoint buffer: not an exact in-place pair
    assert L.bq_ring_hop_i8(qi, si, loc, n, qi, A + 65536, S) == ALIAS
    # output over the local partial
    assert L.bq_ring_hop_i8(qi, si, loc, n, loc + 16, A + 65536, S) == ALIAS
    assert L.bq_ring_hop_i8(qi, si, None, n, A + 65536, A + 70000, S) == NULL
    assert L.bq_ring_hop_i8(qi, si, loc, n, A + 65536 + 8, A + 70000, S) == ALIGN
    assert L.bq_ring_hop_i8(qi, si, loc, 1000, A + 65536, A + 70000, S) == SIZE


def test_accum_errors():
    n = 1024
    qs = arr(A, A + 4096)
    ss = arr(A + 8192, A + 8192 + 64)
    assert L.bq_dequant_accum_i8(0, qs, ss, n, A + 65536, S) == NSRC
    big = arr(*([A] * 65))
    assert L.bq_dequant_accum_i8(65, big, big, n, A + 65536, S) == NSRC
    assert L.bq_dequant_accum_i8(2, qs, ss, n, A + 4096 - 16, S) == ALIAS
    assert L.bq_dequant_accum_i8(2, qs, ss, n, None, S) == NULL
    assert L.bq_dequant_accum_i8(2, None, ss, n, A + 65536, S) == NULL
    f = L.bq_dequant_accum_i8_batch
    assert f(0, 2, qs, ss, n, A + 65536, S) == NSRC
    assert f(17, 2, qs, ss, n, A + 65536, S) == NSRC
    assert f(2, 0, qs, ss, n, A + 65536, S) == NSRC
    assert f(2, 2, qs, ss, 100, A + 65536, S) == SIZE
    assert f(4, 2, qs, ss, n, A + 2048, S) == ALIAS       # y over the sources' 4*n values


def test_collective_driver_errors():
    n = 4 * 1024
    parts = arr(A, A + 16384, A + 32768, A + 49152)
    outs = arr(A + 2 ** 20, A + 2 ** 20 + 16384, A + 2 ** 20 + 32768, A + 2 ** 20 + 49152)
    qw, sw = A + 2 ** 21, A + 2 ** 21 + 8192
    assert L.bq_ring_allreduce_i8(0, n, parts, qw, sw, outs, S) == NSRC
    assert L.bq_ring_allreduce_i8(17, n, parts, qw, sw, outs, S) == NSRC
    assert L.bq_ring_allreduce_i8(4, 128 * 6, parts, qw, sw, outs, S) == SIZE   # not 128*W
    bad_outs = arr(A + 2 ** 20, A + 2 ** 20 + 16384, A + 2 ** 20 + 32768, A + 100 * 16)
    assert L.bq_ring_allreduce_i8(4, n, parts, qw, sw, bad_outs, S) == ALIAS
    assert L.bq_ring_allreduce_i8(4, n, parts, qw, qw + 1024, outs, S) == ALIAS  # wire overlap
    assert L.bq_ring_allreduce_i8(4, n, parts, None, sw, outs, S) == NULL
    qsend = arr(A + 2 ** 22, A + 2 ** 22 + 8192, A + 2 ** 22 + 16384, A + 2 ** 22 + 24576)
    ssend = arr(A + 2 ** 23, A + 2 ** 23 + 256, A + 2 ** 23 + 512, A + 2 ** 23 + 768)
    red, qb, sb = A + 2 ** 24, A + 2 ** 24 + 16384, A + 2 ** 24 + 32768
    assert L.bq_a2a_allreduce_i8(4, n, parts, qsend, ssend, A, qb, sb, outs, S) == ALIAS
    assert L.bq_a2a_allreduce_i8(4, 128 * 2, parts, qsend, ssend, red, qb, sb, outs, S) == SIZE
    assert L.bq_a2a_allreduce_i8(0, n, parts, qsend, ssend, red, qb, sb, outs, S) == NSRC


def test_noalloc_ring_errors():
    """The allocation-free ring all-reduce checks counts and sizes first -- a call whose
    wire payload would not fit the library's scratch array fails with BQ_ERR_SCRATCH --
    then NULL host arrays, before it looks up the scratch array or launches anything."""
    n = 4 * 1024
    parts = arr(A, A + 16384, A + 32768, A + 49152)
    outs = arr(A + 2 ** 20, A + 2 ** 20 + 16384, A + 2 ** 20 + 32768, A + 2 ** 20 + 49152)
    SCRATCH = 8
    assert bq.BQ_STATUS[SCRATCH] == "BQ_ERR_SCRATCH"
    assert b"scratch" in L.bq_status_str(SCRATCH)
    assert L.bq_ring_allreduce_i8_noalloc(0, n, parts, outs, S) == NSRC
    assert L.bq_ring_allreduce_i8_noalloc(17, n, parts, outs, S) == NSRC
    assert L.bq_ring_allreduce_i8_noalloc(4, 128 * 6, parts, outs, S) == SIZE
    assert L.bq_ring_allreduce_i8_noalloc(4, -512, parts, outs, S) == SIZE
    assert L.bq_ring_allreduce_i8_noalloc(4, n, None, outs, S) == NULL
    assert L.bq_ring_allreduce_i8_noalloc(4, n, parts, None, S) == NULL
    # 64 MiB hold 508400 blocks of 132 bytes: 65,075,200 values
    most = (64 * 2 ** 20 // 132) * 128
    assert most == 65075200
    assert L.bq_ring_allreduce_i8_noalloc(1, most + 128, parts, outs, S) == SCRATCH
    assert L.bq_ring_allreduce_i8_noalloc(4, 2 ** 40, parts, outs, S) == SCRATCH


def test_a2a_reduce_and_allgather_errors():
    n = 1024
    qs = arr(A, A + 4096)
    ss = arr(A + 8192, A + 8192 + 64)
    qo, so, red = A + 65536, A + 65536 + 8192, A + 65536 + 16384
    ys = arr(A + 2 ** 20, A + 2 ** 20 + 4096)
    f = L.bq_a2a_reduce_i8
    assert f(0, 2, qs, ss, n, qo, so, ys, red, S) == NSRC
    assert f(2, 0, qs, ss, n, qo, so, ys, red, S) == NSRC
    assert f(2, 65, qs, ss, n, qo, so, ys, red, S) == NSRC
    assert f(2, 2, qs, ss, 100, qo, so, ys, red, S) == SIZE
    assert f(2, 2, None, ss, n, qo, so, ys, red, S) == NULL
    assert f(2, 2, qs, ss, n, None, so, ys, red, S) == NULL
    assert f(2, 2, qs, ss, n, A + 16, so, ys, red, S) == ALIAS        # q_out over a source
    assert f(2, 2, qs, ss, n, qo, so, arr(A + 2 ** 20, A + 2 ** 20 + 1024), red, S) == ALIAS
    assert f(2, 2, qs, ss, n, qo, so, ys, qo + 64, S) == ALIAS        # red over q_out
    assert f(2, 2, qs, ss, n, qo, so, arr(A + 2 ** 20 + 8, A + 2 ** 21), None, S) == ALIGN
    g = L.bq_allgather_dequant_i8
    outs = arr(A + 2 ** 22, A + 2 ** 22 + 8192)
    assert g(0, A, A + 4096, n, outs, 1, S) == NSRC
    assert g(2, A, A + 4096, 128 * 3, outs, 1, S) == SIZE
    assert g(2, A, A + 4096, n, arr(A + 2 ** 22, A + 2 ** 22 + 1024), 1, S) == ALIAS
    assert g(2, A, A + 4096, n, arr(A + 2 ** 22, A + 512), 0, S) == ALIAS
    assert g(2, None, A + 4096, n, outs, 1, S) == NULL


def test_mx_errors():
    rows, cols = 16, 512
    x, v, e = A, A + 2 ** 20, A + 2 ** 21
    assert L.bq_quant_mx(x, rows, 100, 512, v, 512, e, 16, S) == SIZE
    assert L.bq_quant_mx(x, rows, cols, 256, v, 512, e, 16, S) == BOUNDS        # ldx < cols
    assert L.bq_quant_mx(x, rows, cols, 512, v, 512, e, 8, S) == BOUNDS         # lds < cols/32
    assert L.bq_quant_mx(x, rows, cols, 516, v, 512, e, 16, S) == ALIGN         # ldx % 8
    assert L.bq_quant_mx(x, rows, cols, 512, v, 520, e, 16, S) == ALIGN         # ldv % 16
    assert L.bq_quant_mx(x, rows, cols, 512, v, 512, e, 18, S) == ALIGN         # lds % 4
    assert L.bq_quant_mx(x, rows, cols, 512, v, 512, e + 2, 16, S) == ALIGN     # e8m0 ptr
    assert L.bq_quant_mx(x, rows, cols, 512, x + 1024, 512, e, 16, S) == ALIAS
    assert L.bq_quant_mx(None, rows, cols, 512, v, 512, e, 16, S) == NULL
    assert L.bq_quant_mx(x, 0, cols, 512, v, 512, e, 16, S) == OK
    assert L.bq_dequant_mx(v, 512, e, 16, rows, cols, v + 64, 512, S) == ALIAS
    assert L.bq_dequant_mx(v, 512, e, 16, rows, cols, x, 500, S) == BOUNDS
    # a row stride whose operand would span more than 2^48 bytes (and whose extent would
    # overflow int64) is refused before any arithmetic on it
    huge = 2 ** 62
    assert L.bq_quant_mx(x, rows, cols, huge, v, 512, e, 16, S) == BOUNDS
    assert L.bq_quant_mx(x, rows, cols, 512, v, huge, e, 16, S) == BOUNDS
    assert L.bq_quant_mx(x, rows, cols, 512, v, 512, e, huge, S) == BOUNDS
    assert L.bq_quant_mx(x, 2, cols, 2 ** 47, v, 512, e, 16, S) == BOUNDS      # 2^48 + 1024 bytes
    assert L.bq_dequant_mx(v, huge, e, 16, rows, cols, x, 512, S) == BOUNDS
    assert L.bq_dequant_mx(v, 512, e, 16, rows, cols, x, huge, S) == BOUNDS


def test_mx_slice_errors():
    rows, cols, total = 16, 256, 1024
    x, v, e = A, A + 2 ** 20, A + 2 ** 21
    f = L.bq_quant_mx_slice
    assert f(x, rows, cols, cols, 64, v, total, e, total // 32, rows, S) == SIZE   # offset % 128
    assert f(x, rows, 96, cols, 0, v, total, e, total // 32, rows, S) == SIZE      # cols % 128
    assert f(x, rows, cols, cols, 896, v, total, e, total // 32, rows, S) == BOUNDS  # past ldv
    assert f(x, rows, cols, cols, 0, v, total, e, total // 32 - 4, rows, S) == BOUNDS
    assert f(x, rows, cols, cols, 0, v, total, e, total // 32, rows - 1, S) == BOUNDS  # capacity
    assert f(x, rows, cols, cols, 0, None, total, e, total // 32, rows, S) == NULL
    top = 2 ** 63 - 128                      # col_off + cols would overflow int64
    assert f(x, rows, cols, cols, top, v, total, e, total // 32, rows, S) == BOUNDS


def test_mx_collective_errors():
    """The flat MXFP8 collectives share the INT8 validation: payload 16-byte aligned,
    E8M0 arrays 4-byte aligned and n/32 bytes long, the same counts and overlap rules."""
    n = 1024
    v, e, loc = A, A + 4096, A + 8192
    h = L.bq_ring_hop_mx
    assert h(v, e, loc, 100, v, e, S) == SIZE
    assert h(None, e, loc, n, v, e, S) == NULL
    assert h(v + 8, e, loc, n, A + 2 ** 20, A + 2 ** 21, S) == ALIGN         # payload
    assert h(v, e + 2, loc, n, A + 2 ** 20, A + 2 ** 21, S) == ALIGN         # E8M0 bytes
    assert h(v, e, loc, n, v, A + 2 ** 21, S) == ALIAS                       # half in place
    assert h(v, e, loc, n, v + 16, e, S) == ALIAS                            # partial overlap
    assert h(v, e, loc, n, A + 2 ** 20, e + 16, S) == ALIAS                  # e_out inside e_in (n/32 B)
    assert h(v, e, loc, n, loc + 64, A + 2 ** 21, S) == ALIAS                # over the local partial
    assert h(v, e, loc, 0, v, e, S) == OK
    b = L.bq_ring_hop_mx_batch
    assert b(0, arr(v), arr(e), arr(loc), n, arr(v), arr(e), S) == NSRC
    assert b(17, arr(v), arr(e), arr(loc), n, arr(v), arr(e), S) == NSRC
    qb = L.bq_quant_mx_batch
    assert qb(1, arr(A), n, arr(A + 2 ** 20), arr(A + 2 ** 20 + 512), S) == ALIAS   # v over e
    assert qb(1, arr(A), 100, arr(A + 2 ** 20), arr(A + 2 ** 21), S) == SIZE
    db = L.bq_dequant_mx_batch
    assert db(1, arr(v), arr(e), n, arr(e - 64), S) == ALIAS
    vs, es = arr(A, A + 4096), arr(A + 8192, A + 8192 + 64)
    acc = L.bq_dequant_accum_mx
    assert acc(0, vs, es, n, A + 2 ** 20, S) == NSRC
    assert acc(65, vs, es, n, A + 2 ** 20, S) == NSRC
    assert acc(2, vs, es, n, A + 8, S) == ALIGN
    assert acc(2, vs, es, n, A + 512, S) == ALIAS                 # y over source 0
    r = L.bq_a2a_reduce_mx
    vo, eo = A + 65536, A + 65536 + 8192
    ys = arr(A + 2 ** 20, A + 2 ** 20 + 4096)
    assert r(2, 2, vs, es, n, A + 16, eo, ys, None, S) == ALIAS               # v_out over a source
    assert r(2, 2, vs, es, n, vo, eo + 2, ys, None, S) == ALIGN
    assert r(2, 2, vs, es, n, vo, eo, arr(A + 2 ** 20, A + 2 ** 20 + 1024), None, S) == ALIAS
    assert r(17, 2, vs, es, n, vo, eo, ys, None, S) == NSRC
    g = L.bq_allgather_dequant_mx
    outs = arr(A + 2 ** 22, A + 2 ** 22 + 8192)
    assert g(2, v, e, 128 * 3, outs, 1, S) == SIZE
    assert g(2, v, e, n, arr(A + 2 ** 22, A + 2 ** 22 + 1024), 1, S) == ALIAS
    assert g(2, v, e, n, arr(e, A + 2 ** 23), 0, S) == ALIAS
    parts = arr(A, A + 4096)
    routs = arr(A + 2 ** 21, A + 2 ** 21 + 4096)
    ra = L.bq_ring_allreduce_mx
    assert ra(3, n, parts, A + 2 ** 22, A + 2 ** 23, routs, S) == SIZE      # n % (128*3)
    assert ra(2, n, parts, A + 2 ** 22, A + 2 ** 22 + 512, routs, S) == ALIAS   # wire v over e
    assert ra(2, n, parts, A + 2 ** 22, A + 2 ** 23 + 1, routs, S) == ALIGN
    aa = L.bq_a2a_allreduce_mx
    vsend, esend = arr(A + 2 ** 24, A + 2 ** 24 + 4096), arr(A + 2 ** 25, A + 2 ** 25 + 64)
    assert aa(2, n, parts, vsend, esend, None, A + 2 ** 26, A + 2 ** 26 + 512, routs, S) == ALIAS
    assert aa(2, n, parts, vsend, arr(A + 2 ** 25, A + 2 ** 25 + 2), None, A + 2 ** 26,
              A + 2 ** 27, routs, S) == ALIGN
    assert aa(0, n, parts, vsend, esend, None, A + 2 ** 26, A + 2 ** 27, routs, S) == NSRC


def test_mx_mfma_layout_errors():
    """The scaled-MFMA scale layout: its size helper, and the slice quantizer, the
    dequantizer and the GEMM that use it reject bad sizes, bounds, alignment (the layout
    must be 16-byte aligned) and overlaps before launching."""
    f = L.bq_mx_scale_mfma_bytes
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64, ctypes.c_int64]
    assert f(4096, 43008) == 256 * 256 * 84
    assert f(17, 640) == 256 * 2 * 2 and f(0, 0) == 0 and f(16, 128) == 256
    assert f(-1, 128) == -1 and f(16, 100) == -1 and f(16, -128) == -1
    x, v, e = A, A + 2 ** 24, A + 2 ** 26
    q = L.bq_quant_mx_slice_mfma
    assert q(x, 64, 100, 256, 0, v, 512, 512, e, 64, S) == SIZE          # cols off the block
    assert q(x, 64, 256, 256, 64, v, 512, 512, e, 64, S) == SIZE         # offset off the block
    assert q(x, 64, 256, 256, 0, v, 512, 500, e, 64, S) == SIZE          # total off the block
    assert q(x, 64, 256, 256, 384, v, 512, 512, e, 64, S) == BOUNDS      # past total_cols
    assert q(x, 64, 256, 256, 0, v, 384, 512, e, 64, S) == BOUNDS        # total_cols > ldv
    assert q(x, 65, 256, 256, 0, v, 512, 512, e, 64, S) == BOUNDS        # rows > capacity
    assert q(x, 64, 256, 256, 0, v, 512, 512, None, 64, S) == NULL
    assert q(x, 64, 256, 256, 0, v, 512, 512, e + 4, 64, S) == ALIGN    # layout not 16-aligned
    assert q(x, 64, 256, 256, 0, v, 512, 512, v + 256, 64, S) == ALIAS   # layout over the values
    d = L.bq_dequant_mx_mfma
    y = A + 2 ** 27
    assert d(v, 512, e, 16, 17, 256, y, 256, S) == BOUNDS                # rows > scale_rows
    assert d(v, 512, e + 8, 32, 17, 256, y, 256, S) == ALIGN
    assert d(v, 512, e, 32, 17, 250, y, 256, S) == SIZE
    assert d(v, 512, y + 64, 32, 17, 256, y, 256, S) == ALIAS
    m = L.bq_mm_mx_mfma
    xv, xe, wv, we, yy = A, A + 2 ** 24, A + 2 ** 25, A + 2 ** 26, A + 2 ** 27
    assert m(xv, 512, xe, 32, wv, 512, we, 64, 33, 64, 512, yy, 64, S) == BOUNDS   # xe_rows < M
    assert m(xv, 512, xe, 64, wv, 512, we, 32, 33, 64, 512, yy, 64, S) == BOUNDS   # we_rows < N
    assert m(xv, 512, xe, 64, wv, 512, we, 64, 33, 64, 500, yy, 64, S) == SIZE
    assert m(xv, 512, xe + 4, 64, wv, 512, we, 64, 33, 64, 512, yy, 64, S) == ALIGN
    assert m(xv, 512, xe, 64, wv, 512, yy + 128, 64, 33, 64, 512, yy, 64, S) == ALIAS


def test_mx_f16_errors():
    rows, cols = 16, 512
    x, v, e = A, A + 2 ** 20, A + 2 ** 21
    assert L.bq_quant_mx_f16(x, rows, 100, 512, v, 512, e, 16, S) == SIZE
    assert L.bq_quant_mx_f16(x, rows, cols, 512, v, 512, e + 2, 16, S) == ALIGN
    assert L.bq_quant_mx_f16(x, rows, cols, 512, x + 1024, 512, e, 16, S) == ALIAS
    assert L.bq_quant_mx_f16(x, 0, cols, 512, v, 512, e, 16, S) == OK
    f = L.bq_quant_mx_slice_f16
    assert f(x, rows, cols, 512, 64, v, 2048, e, 64, rows, S) == SIZE          # offset % 128
    assert f(x, rows, cols, 512, 1664, v, 2048, e, 64, rows, S) == BOUNDS      # past ldv
    assert f(x, rows, cols, 512, 0, v, 2048, e, 64, rows - 1, S) == BOUNDS     # capacity


def test_mm_mx_errors():
    M, N, K = 64, 48, 256
    xv, xe, wv, we, y = A, A + 2 ** 20, A + 2 ** 21, A + 2 ** 22, A + 2 ** 23
    f = L.bq_mm_mx
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, 0, y, N, S) == SIZE             # K == 0
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, 100, y, N, S) == SIZE           # K % 128
    assert f(xv, K, xe, 8, wv, K, we, 8, -1, N, K, y, N, S) == SIZE
    assert f(xv, K, xe, 8, wv, K, we, 8, 0, N, K, y, N, S) == OK               # nothing to do
    assert f(None, K, xe, 8, wv, K, we, 8, M, N, K, y, N, S) == NULL
    assert f(xv, 128, xe, 8, wv, K, we, 8, M, N, K, y, N, S) == BOUNDS         # ldxv < K
    assert f(xv, K, xe, 4, wv, K, we, 8, M, N, K, y, N, S) == BOUNDS           # ldxe < K/32
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, K, y, N - 1, S) == BOUNDS       # ldy < N
    huge = 2 ** 62                                                             # extent > 2^48 bytes
    assert f(xv, huge, xe, 8, wv, K, we, 8, M, N, K, y, N, S) == BOUNDS
    assert f(xv, K, xe, huge, wv, K, we, 8, M, N, K, y, N, S) == BOUNDS
    assert f(xv, K, xe, 8, wv, huge, we, 8, M, N, K, y, N, S) == BOUNDS
    assert f(xv, K, xe, 8, wv, K, we, huge, M, N, K, y, N, S) == BOUNDS
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, K, y, huge, S) == BOUNDS
    assert f(xv + 8, K, xe, 8, wv, K, we, 8, M, N, K, y, N, S) == ALIGN
    assert f(xv, K + 8, xe, 8, wv, K, we, 8, M, N, K, y, N, S) == ALIGN
    assert f(xv, K, xe + 1, 8, wv, K, we, 8, M, N, K, y, N, S) == ALIGN
    assert f(xv, K, xe, 8, wv, K, we, 10, M, N, K, y, N, S) == ALIGN
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, K, y + 1, N, S) == ALIGN
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, K, xv + 256, N, S) == ALIAS
    assert f(xv, K, xe, 8, wv, K, we, 8, M, N, K, we + 16, N, S) == ALIAS


def test_every_entry_point_accepts_empty_input():
    # n == 0 (rows == 0, M == 0 ...) is valid for every call and launches nothing (without a
    # GPU a launch would fail with BQ_ERR_LAUNCH, so OK shows none was tried); counts
    # and shapes are still validated first.
    p, q, e, y = A, A + 8192, A + 16384, A + 24576
    one = arr(p)
    two = arr(p, q)
    calls = {
        "bq_quant_i8": lambda: L.bq_quant_i8(p, 0, q, e, S),
        "bq_dequant_i8": lambda: L.bq_dequant_i8(q, e, 0, y, S),
        "bq_dequant_accum_i8": lambda: L.bq_dequant_accum_i8(2, two, two, 0, y, S),
        "bq_dequant_accum_i8_batch": lambda: L.bq_dequant_accum_i8_batch(3, 2, two, two, 0, y, S),
        "bq_a2a_reduce_i8": lambda: L.bq_a2a_reduce_i8(2, 2, two, two, 0, q, e, two, y, S),
        "bq_ring_hop_i8": lambda: L.bq_ring_hop_i8(q, e, p, 0, q, e, S),
        "bq_quant_i8_batch": lambda: L.bq_quant_i8_batch(1, one, 0, one, one, S),
        "bq_dequant_i8_batch": lambda: L.bq_dequant_i8_batch(1, one, one, 0, one, S),
        "bq_ring_hop_i8_batch": lambda: L.bq_ring_hop_i8_batch(1, one, one, one, 0, one, one, S),
        "bq_allgather_dequant_i8": lambda: L.bq_allgather_dequant_i8(3, q, e, 0, two, 1, S),
        "bq_ring_allreduce_i8": lambda: L.bq_ring_allreduce_i8(3, 0, two, q, e, two, S),
        "bq_ring_allreduce_i8_noalloc": lambda: L.bq_ring_allreduce_i8_noalloc(3, 0, two, two, S),
        "bq_a2a_allreduce_i8": lambda: L.bq_a2a_allreduce_i8(3, 0, two, two, two, y, q, e, two,
                                                             S),
        "bq_quant_mx": lambda: L.bq_quant_mx(p, 0, 256, 256, q, 256, e, 8, S),
        "bq_dequant_mx": lambda: L.bq_dequant_mx(q, 256, e, 8, 0, 256, y, 256, S),
        "bq_quant_mx_slice": lambda: L.bq_quant_mx_slice(p, 0, 128, 128, 128, q, 256, e, 8, 0,
                                                         S),
        "bq_quant_mx_f16": lambda: L.bq_quant_mx_f16(p, 5, 0, 0, q, 0, e, 0, S),
        "bq_quant_mx_slice_f16": lambda: L.bq_quant_mx_slice_f16(p, 0, 128, 128, 0, q, 128, e,
                                                                 4, 0, S),
        "bq_quant_mx_batch": lambda: L.bq_quant_mx_batch(1, one, 0, one, one, S),
        "bq_dequant_mx_batch": lambda: L.bq_dequant_mx_batch(1, one, one, 0, one, S),
        "bq_ring_hop_mx": lambda: L.bq_ring_hop_mx(q, e, p, 0, q, e, S),
        "bq_ring_hop_mx_batch": lambda: L.bq_ring_hop_mx_batch(1, one, one, one, 0, one, one, S),
        "bq_dequant_accum_mx": lambda: L.bq_dequant_accum_mx(2, two, two, 0, y, S),
        "bq_a2a_reduce_mx": lambda: L.bq_a2a_reduce_mx(2, 2, two, two, 0, q, e, None, None, S),
        "bq_allgather_dequant_mx": lambda: L.bq_allgather_dequant_mx(3, q, e, 0, two, 0, S),
        "bq_ring_allreduce_mx": lambda: L.bq_ring_allreduce_mx(3, 0, two, q, e, two, S),
        "bq_a2a_allreduce_mx": lambda: L.bq_a2a_allreduce_mx(3, 0, two, two, two, None, q, e,
                                                             two, S),
        "bq_mm_mx": lambda: L.bq_mm_mx(p, 256, e, 8, q, 256, e, 8, 0, 64, 256, y, 64, S),
        "bq_quant_mx_slice_mfma": lambda: L.bq_quant_mx_slice_mfma(p, 0, 128, 128, 128, q, 256,
                                                                   256, e, 0, S),
        "bq_quant_mx_slice_mfma_f16": lambda: L.bq_quant_mx_slice_mfma_f16(p, 5, 0, 0, 0, q, 0, 0,
                                                                           e, 5, S),
        "bq_dequant_mx_mfma": lambda: L.bq_dequant_mx_mfma(q, 256, e, 16, 0, 256, y, 256, S),
        "bq_mm_mx_mfma": lambda: L.bq_mm_mx_mfma(p, 256, e, 16, q, 256, e, 64, 0, 64, 256, y, 64, S),
        "bq_quant_e4m3_b128": lambda: L.bq_quant_e4m3_b128(p, 0, q, e, S),
        "bq_dequant_e4m3_b128": lambda: L.bq_dequant_e4m3_b128(q, e, 0, y, S),
    }
    compute = [n for n in declared_symbols()
               if n not in ("bq_status_str", "bq_version", "bq_wire_bytes_b128",
                            "bq_mx_staging_bytes", "bq_mx_scale_mfma_bytes", "bq_mm_tile_cols")]
    assert sorted(calls) == compute
    for name, call in calls.items():
        assert call() == OK, name
    # an empty call reads no pointer, so NULL ones are accepted too
    assert L.bq_quant_i8(None, 0, None, None, S) == OK
    assert L.bq_ring_allreduce_i8(3, 0, None, None, None, None, S) == OK
    assert L.bq_a2a_allreduce_mx(3, 0, None, None, None, None, None, None, None, S) == OK
    assert L.bq_quant_mx_slice(None, 0, 128, 128, 0, None, 128, None, 4, 0, S) == OK
    assert L.bq_mm_mx(None, 256, None, 8, None, 256, None, 8, 0, 64, 256, None, 64, S) == OK
    # N == 0 is empty too; K is not a size that may be zero
    assert L.bq_mm_mx(p, 256, e, 8, q, 256, e, 8, 64, 0, 256, y, 64, S) == OK
    assert L.bq_mm_mx(p, 256, e, 8, q, 256, e, 8, 0, 0, 0, y, 64, S) == SIZE
    # an empty call still rejects a bad count or a size off its block
    assert L.bq_quant_i8_batch(0, one, 0, one, one, S) == NSRC
    assert L.bq_dequant_accum_i8(0, two, two, 0, y, S) == NSRC
    assert L.bq_ring_allreduce_i8(17, 0, two, q, e, two, S) == NSRC   # 16 ranks at most
    assert L.bq_quant_mx(p, 0, 100, 128, q, 128, e, 4, S) == SIZE
    assert L.bq_quant_mx_slice(p, 1, 128, 128, 128, q, 256, e, 8, 0, S) == BOUNDS
