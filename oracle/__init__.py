"""CPU oracle for the block-quantized wire codecs (ctypes wrapper over bq_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports it, and it imports nothing from the GPU library.

All arrays are numpy: bf16 tensors as uint16 bit patterns, INT8 payloads as
int8, E4M3 / E8M0 bytes as uint8, scales as float32.  Functions allocate their
outputs zero-filled (so an output a planted mistake leaves unwritten reads as
zeros, deterministically) and return them.  The C functions they wrap cite the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bq_oracle.c")
_HDR = os.path.join(_HERE, "bq_oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build() -> str:
    """Compile ``liboracle.so`` next to its source with gcc (IEEE binary32, no contraction)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "orc_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
    "orc_f32_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
    "orc_e4m3_encode": ([ctypes.c_float], ctypes.c_uint8),
    "orc_e4m3_decode": ([ctypes.c_uint8], ctypes.c_float),
    "orc_e8m0_scale": ([ctypes.c_float], ctypes.c_uint8),
    "orc_quant_i8": ([_P, _I64, _P, _P], None),
    "orc_dequant_i8": ([_P, _P, _I64, _P], None),
    "orc_dequant_accum_i8": ([ctypes.c_int, _P, _P, _I64, _P], None),
    "orc_ring_hop_i8": ([_P, _P, _P, _I64, _P, _P], None),
    "orc_a2a_reduce_i8": ([ctypes.c_int, ctypes.c_int, _P, _P, _I64, _P, _P, _P, _P], None),
    "orc_ring_allreduce_i8": ([ctypes.c_int, _I64, _P, _P, _P, _P], None),
    "orc_a2a_allreduce_i8": ([ctypes.c_int, _I64, _P, _P, _P, _P, _P], None),
    "orc_quant_mx": ([_P, _I64, _I64, _I64, _P, _I64, _P, _I64], None),
    "orc_dequant_mx": ([_P, _I64, _P, _I64, _I64, _I64, _P, _I64], None),
    "orc_quant_mx_slice": ([_P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64], None),
    "orc_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
    "orc_quant_mx_f16": ([_P, _I64, _I64, _I64, _P, _I64, _P, _I64], None),
    "orc_quant_mx_slice_f16": ([_P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64], None),
    "orc_ring_hop_mx": ([_P, _P, _P, _I64, _P, _P], None),
    "orc_dequant_accum_mx": ([ctypes.c_int, _P, _P, _I64, _P], None),
    "orc_a2a_reduce_mx": ([ctypes.c_int, ctypes.c_int, _P, _P, _I64, _P, _P, _P, _P], None),
    "orc_ring_allreduce_mx": ([ctypes.c_int, _I64, _P, _P, _P, _P], None),
    "orc_a2a_allreduce_mx": ([ctypes.c_int, _I64, _P, _P, _P, _P, _P], None),
    "orc_mx_mfma_offset": ([_I64, _I64, _I64], _I64),
    "orc_mx_scales_to_mfma": ([_P, _I64, _I64, _I64, _I64, _I64, _P], None),
    "orc_quant_e4m3_b128": ([_P, _I64, _P, _P], None),
    "orc_dequant_e4m3_b128": ([_P, _P, _I64, _P], None),
}


def lib():
    global _lib
    if _lib is None:
        stale = (not os.path.exists(_LIB) or
                 os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
        if stale:
            build()
        L = ctypes.CDLL(_LIB)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptrs(arrs):
    arr = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    return arr


# ---- scalars -------------------------------------------------------------

def bf16_to_f32(h: int) -> float:
    return lib().orc_bf16_to_f32(h)


def f32_to_bf16(f: float) -> int:
    return lib().orc_f32_to_bf16(f)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e8m0_scale(amax: float) -> int:
    return lib().orc_e8m0_scale(amax)


# ---- block INT8 ------------------------------------------------------------

def quant_i8(x: np.ndarray):
    x = _c(x, np.uint16).reshape(-1)
    q = np.zeros(x.size, np.int8)
    s = np.zeros(x.size // 128, np.float32)
    lib().orc_quant_i8(x.ctypes.data, x.size, q.ctypes.data, s.ctypes.data)
    return q, s


def dequant_i8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8).reshape(-1)
    s = _c(s, np.float32).reshape(-1)
    assert s.size * 128 == q.size
    y = np.zeros(q.size, np.uint16)
    lib().orc_dequant_i8(q.ctypes.data, s.ctypes.data, q.size, y.ctypes.data)
    return y


def dequant_accum_i8(qs, ss) -> np.ndarray:
    qs = [_c(q, np.int8).reshape(-1) for q in qs]
    ss = [_c(s, np.float32).reshape(-1) for s in ss]
    n = qs[0].size
    assert all(q.size == n for q in qs) and all(s.size * 128 == n for s in ss)
    y = np.zeros(n, np.uint16)
    lib().orc_dequant_accum_i8(len(qs), _ptrs(qs), _ptrs(ss), n, y.ctypes.data)
    return y


def ring_hop_i8(q_in: np.ndarray, s_in: np.ndarray, local: np.ndarray):
    q_in = _c(q_in, np.int8).reshape(-1)
    s_in = _c(s_in, np.float32).reshape(-1)
    local = _c(local, np.uint16).reshape(-1)
    n = q_in.size
    assert local.size == n and s_in.size * 128 == n
    q = np.zeros(n, np.int8)
    s = np.zeros(n // 128, np.float32)
    lib().orc_ring_hop_i8(q_in.ctypes.data, s_in.ctypes.data, local.ctypes.data, n,
                          q.ctypes.data, s.ctypes.data)
    return q, s


def a2a_reduce_i8(qs, ss, nseg: int):
    """Owner step of the all-to-all for nseg owners: returns (q, s, ys, red) where segment j
    of q/s/red is owner j's payload / scales / bf16 sum and ys[j] its materialized shard."""
    qs = [_c(q, np.int8).reshape(-1) for q in qs]
    ss = [_c(s, np.float32).reshape(-1) for s in ss]
    n = qs[0].size
    seg_n = n // nseg
    q = np.zeros(n, np.int8)
    s = np.zeros(n // 128, np.float32)
    red = np.zeros(n, np.uint16)
    ys = [np.zeros(seg_n, np.uint16) for _ in range(nseg)]
    lib().orc_a2a_reduce_i8(nseg, len(qs), _ptrs(qs), _ptrs(ss), seg_n, q.ctypes.data,
                            s.ctypes.data, _ptrs(ys), red.ctypes.data)
    return q, s, ys, red


def ring_allreduce_i8(partials):
    """Returns (q_final, s_final, outs): final payload of every chunk and each rank's bf16 output."""
    ps = [_c(p, np.uint16).reshape(-1) for p in partials]
    W, n = len(ps), ps[0].size
    q = np.zeros(n, np.int8)
    s = np.zeros(n // 128, np.float32)
    outs = [np.zeros(n, np.uint16) for _ in range(W)]
    lib().orc_ring_allreduce_i8(W, n, _ptrs(ps), q.ctypes.data, s.ctypes.data, _ptrs(outs))
    return q, s, outs


def a2a_allreduce_i8(partials):
    """Returns (red, q_final, s_final, outs): owner bf16 sums, broadcast payloads, outputs."""
    ps = [_c(p, np.uint16).reshape(-1) for p in partials]
    W, n = len(ps), ps[0].size
    red = np.zeros(n, np.uint16)
    q = np.zeros(n, np.int8)
    s = np.zeros(n // 128, np.float32)
    outs = [np.zeros(n, np.uint16) for _ in range(W)]
    lib().orc_a2a_allreduce_i8(W, n, _ptrs(ps), red.ctypes.data, q.ctypes.data, s.ctypes.data,
                               _ptrs(outs))
    return red, q, s, outs


# ---- MXFP8 -----------------------------------------------------------------

def quant_mx(x: np.ndarray):
    """x: (rows, cols) uint16 bf16 -> (values uint8 (rows, cols), e8m0 uint8 (rows, cols/32))."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    v = np.zeros((rows, cols), np.uint8)
    e = np.zeros((rows, cols // 32), np.uint8)
    lib().orc_quant_mx(x.ctypes.data, rows, cols, cols, v.ctypes.data, cols, e.ctypes.data,
                       cols // 32)
    return v, e


def dequant_mx(v: np.ndarray, e: np.ndarray) -> np.ndarray:
    v = _c(v, np.uint8)
    e = _c(e, np.uint8)
    rows, cols = v.shape
    assert e.shape == (rows, cols // 32)
    y = np.zeros((rows, cols), np.uint16)
    lib().orc_dequant_mx(v.ctypes.data, cols, e.ctypes.data, cols // 32, rows, cols,
                         y.ctypes.data, cols)
    return y


def quant_mx_slice(x: np.ndarray, col_off: int, v: np.ndarray, e: np.ndarray) -> None:
    """Quantize slice x (rows, cols) into v[:, col_off:col_off+cols] and e[:, col_off/32:...] in place."""
    x = _c(x, np.uint16)
    assert v.dtype == np.uint8 and e.dtype == np.uint8
    assert v.flags.c_contiguous and e.flags.c_contiguous
    rows, cols = x.shape
    assert rows <= v.shape[0] and col_off + cols <= v.shape[1]
    assert e.shape[1] * 32 >= v.shape[1] and e.shape[0] == v.shape[0]
    lib().orc_quant_mx_slice(x.ctypes.data, rows, cols, cols, col_off, v.ctypes.data,
                             v.shape[1], e.ctypes.data, e.shape[1])


def f16_to_f32(h: int) -> float:
    return lib().orc_f16_to_f32(h)


def quant_mx_f16(x: np.ndarray):
    """x: (rows, cols) uint16 IEEE binary16 -> (values (rows, cols), e8m0 (rows, cols/32))."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    v = np.zeros((rows, cols), np.uint8)
    e = np.zeros((rows, cols // 32), np.uint8)
    lib().orc_quant_mx_f16(x.ctypes.data, rows, cols, cols, v.ctypes.data, cols, e.ctypes.data,
                           cols // 32)
    return v, e


def quant_mx_slice_f16(x: np.ndarray, col_off: int, v: np.ndarray, e: np.ndarray) -> None:
    """quant_mx_slice for a binary16 slice."""
    x = _c(x, np.uint16)
    assert v.dtype == np.uint8 and e.dtype == np.uint8
    assert v.flags.c_contiguous and e.flags.c_contiguous
    rows, cols = x.shape
    assert rows <= v.shape[0] and col_off + cols <= v.shape[1]
    assert e.shape[1] * 32 >= v.shape[1] and e.shape[0] == v.shape[0]
    lib().orc_quant_mx_slice_f16(x.ctypes.data, rows, cols, cols, col_off, v.ctypes.data,
                                 v.shape[1], e.ctypes.data, e.shape[1])


# ---- the MXFP8 GEMM from staged inputs (b12x PR #241, Behavior: mm_quantized) ----------

def mx_values_f64(v: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Exact values of an MXFP8 matrix (rows, cols) in float64: each E4M3 code (decoded by
    orc_e4m3_decode) times 2^(byte - 127) of its 32-column group."""
    v = _c(v, np.uint8)
    e = _c(e, np.uint8)
    rows, cols = v.shape
    assert e.shape[0] == rows and e.shape[1] * 32 >= cols
    table = np.array([lib().orc_e4m3_decode(c) for c in range(256)], np.float64)
    scale = np.ldexp(1.0, np.repeat(e[:, :cols // 32].astype(np.int64) - 127, 32, axis=1))
    return table[v] * scale


def mm_mx(xv: np.ndarray, xe: np.ndarray, wv: np.ndarray, we: np.ndarray):
    """The dense GEMM of MXFP8 activations X (M, K) and weights W (N, K): returns
    (Y, S) with Y = X W^T and S = |X| |W|^T, both float64 from the exact operand values
    (every product is exact in float64; a float64 matmul is the one library step)."""
    X = mx_values_f64(xv, xe)
    Wt = mx_values_f64(wv, we)
    assert X.shape[1] == Wt.shape[1]
    return X @ Wt.T, np.abs(X) @ np.abs(Wt).T


# ---- MXFP8 scales in the scaled-MFMA operand order ------------------------------

def mx_mfma_bytes(rows: int, cols: int) -> int:
    """Bytes of the layout for `rows` rows and `cols` columns: 256-byte tiles of 16 rows x
    512 columns."""
    return 256 * (-(-rows // 16)) * (-(-cols // 512))


def mx_mfma_offset(row: int, group: int, row_blocks: int) -> int:
    return lib().orc_mx_mfma_offset(row, group, row_blocks)


def mx_scales_to_mfma(e: np.ndarray, out: np.ndarray, row_blocks: int, group_off: int = 0) -> None:
    """Place row-major scales e (rows, groups) into `out` (uint8, the layout) in place, group
    g of e at layout group group_off + g; other bytes of `out` are left as they are."""
    e = _c(e, np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous
    rows, groups = e.shape
    assert rows <= 16 * row_blocks
    assert out.size >= 256 * row_blocks * (-(-(group_off + groups) // 16))
    lib().orc_mx_scales_to_mfma(e.ctypes.data, groups, rows, groups, group_off, row_blocks,
                                out.ctypes.data)


def quant_mx_slice_mfma(x: np.ndarray, col_off: int, v: np.ndarray, e_mfma: np.ndarray,
                        capacity_rows: int, f16: bool = False) -> None:
    """The staged slice quantization with the scales in the MFMA layout: values as
    quant_mx_slice writes them, scale (row, group) of the slice at layout group
    col_off/32 + group of a layout with ceil(capacity_rows/16) row blocks."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    assert col_off % 128 == 0 and cols % 128 == 0 and rows <= capacity_rows
    vs, es = (quant_mx_f16 if f16 else quant_mx)(x)
    v[:rows, col_off:col_off + cols] = vs
    mx_scales_to_mfma(es, e_mfma, -(-capacity_rows // 16), col_off // 32)


def mx_scales_from_mfma(e_mfma: np.ndarray, rows: int, groups: int, row_blocks: int) -> np.ndarray:
    """Row-major (rows, groups) scales read back from the layout through the offset map."""
    e_mfma = _c(e_mfma, np.uint8).reshape(-1)
    out = np.empty((rows, groups), np.uint8)
    for r in range(rows):
        for g in range(groups):
            out[r, g] = e_mfma[mx_mfma_offset(r, g, row_blocks)]
    return out


# ---- MXFP8 on the collective topologies (flat: n E4M3 bytes, n/32 E8M0 bytes) ----

def quant_mx_flat(x: np.ndarray):
    x = _c(x, np.uint16).reshape(1, -1)
    v, e = quant_mx(x)
    return v.reshape(-1), e.reshape(-1)


def dequant_mx_flat(v: np.ndarray, e: np.ndarray) -> np.ndarray:
    v = _c(v, np.uint8).reshape(1, -1)
    e = _c(e, np.uint8).reshape(1, -1)
    return dequant_mx(v, e).reshape(-1)


def ring_hop_mx(v_in: np.ndarray, e_in: np.ndarray, local: np.ndarray):
    v_in = _c(v_in, np.uint8).reshape(-1)
    e_in = _c(e_in, np.uint8).reshape(-1)
    local = _c(local, np.uint16).reshape(-1)
    n = v_in.size
    assert local.size == n and e_in.size * 32 == n
    v = np.zeros(n, np.uint8)
    e = np.zeros(n // 32, np.uint8)
    lib().orc_ring_hop_mx(v_in.ctypes.data, e_in.ctypes.data, local.ctypes.data, n,
                          v.ctypes.data, e.ctypes.data)
    return v, e


def dequant_accum_mx(vs, es) -> np.ndarray:
    vs = [_c(v, np.uint8).reshape(-1) for v in vs]
    es = [_c(e, np.uint8).reshape(-1) for e in es]
    n = vs[0].size
    assert all(v.size == n for v in vs) and all(e.size * 32 == n for e in es)
    y = np.zeros(n, np.uint16)
    lib().orc_dequant_accum_mx(len(vs), _ptrs(vs), _ptrs(es), n, y.ctypes.data)
    return y


def a2a_reduce_mx(vs, es, nseg: int):
    """MX owner step for nseg owners: returns (v, e, ys, red) as a2a_reduce_i8 does."""
    vs = [_c(v, np.uint8).reshape(-1) for v in vs]
    es = [_c(e, np.uint8).reshape(-1) for e in es]
    n = vs[0].size
    seg_n = n // nseg
    v = np.zeros(n, np.uint8)
    e = np.zeros(n // 32, np.uint8)
    red = np.zeros(n, np.uint16)
    ys = [np.zeros(seg_n, np.uint16) for _ in range(nseg)]
    lib().orc_a2a_reduce_mx(nseg, len(vs), _ptrs(vs), _ptrs(es), seg_n, v.ctypes.data,
                            e.ctypes.data, _ptrs(ys), red.ctypes.data)
    return v, e, ys, red


def ring_allreduce_mx(partials):
    """Returns (v_final, e_final, outs)."""
    ps = [_c(p, np.uint16).reshape(-1) for p in partials]
    W, n = len(ps), ps[0].size
    v = np.zeros(n, np.uint8)
    e = np.zeros(n // 32, np.uint8)
    outs = [np.zeros(n, np.uint16) for _ in range(W)]
    lib().orc_ring_allreduce_mx(W, n, _ptrs(ps), v.ctypes.data, e.ctypes.data, _ptrs(outs))
    return v, e, outs


def a2a_allreduce_mx(partials):
    """Returns (red, v_final, e_final, outs)."""
    ps = [_c(p, np.uint16).reshape(-1) for p in partials]
    W, n = len(ps), ps[0].size
    red = np.zeros(n, np.uint16)
    v = np.zeros(n, np.uint8)
    e = np.zeros(n // 32, np.uint8)
    outs = [np.zeros(n, np.uint16) for _ in range(W)]
    lib().orc_a2a_allreduce_mx(W, n, _ptrs(ps), red.ctypes.data, v.ctypes.data, e.ctypes.data,
                               _ptrs(outs))
    return red, v, e, outs


# ---- E4M3 128-block codec ----------------------------------------------------

def quant_e4m3_b128(x: np.ndarray):
    x = _c(x, np.uint16).reshape(-1)
    v = np.zeros(x.size, np.uint8)
    s = np.zeros(x.size // 128, np.float32)
    lib().orc_quant_e4m3_b128(x.ctypes.data, x.size, v.ctypes.data, s.ctypes.data)
    return v, s


def dequant_e4m3_b128(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    v = _c(v, np.uint8).reshape(-1)
    s = _c(s, np.float32).reshape(-1)
    assert s.size * 128 == v.size
    y = np.zeros(v.size, np.uint16)
    lib().orc_dequant_e4m3_b128(v.ctypes.data, s.ctypes.data, v.size, y.ctypes.data)
    return y
