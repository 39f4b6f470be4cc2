"""libblockq: block-quantized wire codecs for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI declared in ``include/blockq.h``.  Every
function here has the name of the C entry point it calls and only marshals
arguments: torch tensors give device pointers, the stream defaults to torch's
current stream, and a non-OK status raises :class:`BlockqError`.  All compute
runs in the HIP kernels of ``libblockq.so``; there is no fallback, so importing
fails loudly when the library has not been built.

Tensor conventions: bf16 data as ``torch.bfloat16`` (or int16/uint16 bit
views), INT8 payloads ``torch.int8``, E4M3 / E8M0 bytes ``torch.uint8``, block
scales ``torch.float32``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "BlockqError", "lib", "LIB_PATH",
    "bq_quant_i8", "bq_dequant_i8", "bq_dequant_accum_i8", "bq_dequant_accum_i8_batch",
    "bq_a2a_reduce_i8",
    "bq_ring_hop_i8",
    "bq_quant_i8_batch", "bq_dequant_i8_batch", "bq_ring_hop_i8_batch",
    "bq_allgather_dequant_i8", "bq_ring_allreduce_i8", "bq_ring_allreduce_i8_noalloc",
    "bq_a2a_allreduce_i8",
    "bq_quant_mx", "bq_dequant_mx", "bq_quant_mx_slice", "bq_mx_staging_bytes",
    "bq_quant_mx_f16", "bq_quant_mx_slice_f16", "bq_mm_mx",
    "bq_quant_mx_batch", "bq_dequant_mx_batch", "bq_ring_hop_mx", "bq_ring_hop_mx_batch",
    "bq_dequant_accum_mx", "bq_a2a_reduce_mx", "bq_allgather_dequant_mx",
    "bq_ring_allreduce_mx", "bq_a2a_allreduce_mx",
    "bq_quant_e4m3_b128", "bq_dequant_e4m3_b128",
    "bq_mx_scale_mfma_bytes", "bq_quant_mx_slice_mfma", "bq_quant_mx_slice_mfma_f16",
    "bq_dequant_mx_mfma", "bq_mm_mx_mfma",
    "bq_wire_bytes_b128", "bq_mm_tile_cols", "bq_status_str", "bq_version",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libblockq.so")

BQ_OK = 0
BQ_STATUS = {0: "BQ_OK", 1: "BQ_ERR_NULL", 2: "BQ_ERR_SIZE", 3: "BQ_ERR_ALIGN",
             4: "BQ_ERR_BOUNDS", 5: "BQ_ERR_NSRC", 6: "BQ_ERR_ALIAS", 7: "BQ_ERR_LAUNCH",
             8: "BQ_ERR_SCRATCH"}


class BlockqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.name = BQ_STATUS.get(status, str(status))
        super().__init__(f"{fn}: {self.name} ({_L().bq_status_str(status).decode()})")


_P, _I, _I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
_PP = ctypes.POINTER(ctypes.c_void_p)
_SIGS = {
    "bq_quant_i8": [_P, _I64, _P, _P, _P],
    "bq_dequant_i8": [_P, _P, _I64, _P, _P],
    "bq_dequant_accum_i8": [_I, _PP, _PP, _I64, _P, _P],
    "bq_dequant_accum_i8_batch": [_I, _I, _PP, _PP, _I64, _P, _P],
    "bq_a2a_reduce_i8": [_I, _I, _PP, _PP, _I64, _P, _P, _PP, _P, _P],
    "bq_ring_hop_i8": [_P, _P, _P, _I64, _P, _P, _P],
    "bq_quant_i8_batch": [_I, _PP, _I64, _PP, _PP, _P],
    "bq_dequant_i8_batch": [_I, _PP, _PP, _I64, _PP, _P],
    "bq_ring_hop_i8_batch": [_I, _PP, _PP, _PP, _I64, _PP, _PP, _P],
    "bq_allgather_dequant_i8": [_I, _P, _P, _I64, _PP, _I, _P],
    "bq_ring_allreduce_i8": [_I, _I64, _PP, _P, _P, _PP, _P],
    "bq_a2a_allreduce_i8": [_I, _I64, _PP, _PP, _PP, _P, _P, _P, _PP, _P],
    "bq_ring_allreduce_i8_noalloc": [_I, _I64, _PP, _PP, _P],
    "bq_quant_mx": [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P],
    "bq_dequant_mx": [_P, _I64, _P, _I64, _I64, _I64, _P, _I64, _P],
    "bq_quant_mx_slice": [_P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _I64, _P],
    "bq_mx_staging_bytes": [_I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
    "bq_quant_mx_f16": [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P],
    "bq_mm_mx": [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _I64, _P],
    "bq_quant_mx_slice_f16": [_P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _I64, _P],
    "bq_quant_mx_batch": [_I, _PP, _I64, _PP, _PP, _P],
    "bq_dequant_mx_batch": [_I, _PP, _PP, _I64, _PP, _P],
    "bq_ring_hop_mx": [_P, _P, _P, _I64, _P, _P, _P],
    "bq_ring_hop_mx_batch": [_I, _PP, _PP, _PP, _I64, _PP, _PP, _P],
    "bq_dequant_accum_mx": [_I, _PP, _PP, _I64, _P, _P],
    "bq_a2a_reduce_mx": [_I, _I, _PP, _PP, _I64, _P, _P, _PP, _P, _P],
    "bq_allgather_dequant_mx": [_I, _P, _P, _I64, _PP, _I, _P],
    "bq_ring_allreduce_mx": [_I, _I64, _PP, _P, _P, _PP, _P],
    "bq_a2a_allreduce_mx": [_I, _I64, _PP, _PP, _PP, _P, _P, _P, _PP, _P],
    "bq_quant_mx_slice_mfma": [_P, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _P],
    "bq_quant_mx_slice_mfma_f16": [_P, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _P],
    "bq_dequant_mx_mfma": [_P, _I64, _P, _I64, _I64, _I64, _P, _I64, _P],
    "bq_mm_mx_mfma": [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _I64, _P],
    "bq_quant_e4m3_b128": [_P, _I64, _P, _P, _P],
    "bq_dequant_e4m3_b128": [_P, _P, _I64, _P, _P],
}
_lib = None


def _L() -> ctypes.CDLL:
    """The loaded libblockq.so (loaded on first use; a missing library is an error)."""
    global _lib
    if _lib is None:
        # torch brings its own HIP runtime (same soname, libamdhip64.so.7).  Loading it
        # first makes libblockq.so bind to that one runtime; loaded the other way round,
        # the process would hold two HIP runtimes and ours would see no device.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python block_quantized_wire_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.bq_wire_bytes_b128.argtypes = [_I64]
        L.bq_wire_bytes_b128.restype = _I64
        L.bq_mx_scale_mfma_bytes.argtypes = [_I64, _I64]
        L.bq_mx_scale_mfma_bytes.restype = _I64
        L.bq_mm_tile_cols.argtypes = [_I64, _I64, ctypes.c_int]
        L.bq_mm_tile_cols.restype = ctypes.c_int
        L.bq_status_str.argtypes = [ctypes.c_int]
        L.bq_status_str.restype = ctypes.c_char_p
        L.bq_version.argtypes = []
        L.bq_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def __getattr__(name: str):
    if name == "lib":
        return _L()
    raise AttributeError(name)


# ---- marshalling helpers ---------------------------------------------------------------

def _ptr(t) -> int | None:
    """Device pointer of a tensor (or an int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ptrs(ts) -> ctypes.Array:
    return (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _numel(t) -> int:
    return t.numel()


def _check(fn: str, status: int) -> None:
    if status != BQ_OK:
        raise BlockqError(fn, status)


# ---- block INT8 ----------------------------------------------------------------------------

def bq_quant_i8(x, q, scale, n: int | None = None, stream=None) -> None:
    n = _numel(x) if n is None else n
    _check("bq_quant_i8", _L().bq_quant_i8(_ptr(x), n, _ptr(q), _ptr(scale), _stream(stream)))


def bq_dequant_i8(q, scale, y, n: int | None = None, stream=None) -> None:
    n = _numel(q) if n is None else n
    _check("bq_dequant_i8", _L().bq_dequant_i8(_ptr(q), _ptr(scale), n, _ptr(y), _stream(stream)))


def bq_dequant_accum_i8(q_srcs, s_srcs, y, n: int | None = None, stream=None) -> None:
    n = _numel(y) if n is None else n
    _check("bq_dequant_accum_i8",
           _L().bq_dequant_accum_i8(len(q_srcs), _ptrs(q_srcs), _ptrs(s_srcs), n, _ptr(y),
                                   _stream(stream)))


def bq_dequant_accum_i8_batch(nseg: int, q_srcs, s_srcs, y, seg_n: int | None = None,
                              stream=None) -> None:
    seg_n = _numel(y) // nseg if seg_n is None else seg_n
    _check("bq_dequant_accum_i8_batch",
           _L().bq_dequant_accum_i8_batch(nseg, len(q_srcs), _ptrs(q_srcs), _ptrs(s_srcs), seg_n,
                                         _ptr(y), _stream(stream)))


def bq_a2a_reduce_i8(nseg: int, q_srcs, s_srcs, q_out, s_out, y_out=None, red=None,
                     seg_n: int | None = None, stream=None) -> None:
    seg_n = _numel(q_out) // nseg if seg_n is None else seg_n
    ys = _ptrs(y_out) if y_out is not None else None
    _check("bq_a2a_reduce_i8",
           _L().bq_a2a_reduce_i8(nseg, len(q_srcs), _ptrs(q_srcs), _ptrs(s_srcs), seg_n,
                                 _ptr(q_out), _ptr(s_out), ys, _ptr(red), _stream(stream)))


def bq_ring_hop_i8(q_in, s_in, local, q_out, s_out, n: int | None = None, stream=None) -> None:
    n = _numel(local) if n is None else n
    _check("bq_ring_hop_i8", _L().bq_ring_hop_i8(_ptr(q_in), _ptr(s_in), _ptr(local), n,
                                                _ptr(q_out), _ptr(s_out), _stream(stream)))


def bq_quant_i8_batch(xs, qs, ss, n: int | None = None, stream=None) -> None:
    n = _numel(xs[0]) if n is None else n
    _check("bq_quant_i8_batch", _L().bq_quant_i8_batch(len(xs), _ptrs(xs), n, _ptrs(qs), _ptrs(ss),
                                                      _stream(stream)))


def bq_dequant_i8_batch(qs, ss, ys, n: int | None = None, stream=None) -> None:
    n = _numel(ys[0]) if n is None else n
    _check("bq_dequant_i8_batch", _L().bq_dequant_i8_batch(len(qs), _ptrs(qs), _ptrs(ss), n,
                                                          _ptrs(ys), _stream(stream)))


def bq_ring_hop_i8_batch(q_in, s_in, local, q_out, s_out, n: int | None = None,
                         stream=None) -> None:
    n = _numel(local[0]) if n is None else n
    _check("bq_ring_hop_i8_batch",
           _L().bq_ring_hop_i8_batch(len(q_in), _ptrs(q_in), _ptrs(s_in), _ptrs(local), n,
                                    _ptrs(q_out), _ptrs(s_out), _stream(stream)))


def bq_allgather_dequant_i8(q, s, outs, skip_own: bool = False, n: int | None = None,
                            stream=None) -> None:
    n = _numel(q) if n is None else n
    _check("bq_allgather_dequant_i8",
           _L().bq_allgather_dequant_i8(len(outs), _ptr(q), _ptr(s), n, _ptrs(outs), int(skip_own),
                                        _stream(stream)))


def bq_ring_allreduce_i8(partials, q_wire, s_wire, outs, n: int | None = None,
                         stream=None) -> None:
    n = _numel(partials[0]) if n is None else n
    _check("bq_ring_allreduce_i8",
           _L().bq_ring_allreduce_i8(len(partials), n, _ptrs(partials), _ptr(q_wire), _ptr(s_wire),
                                    _ptrs(outs), _stream(stream)))


def bq_ring_allreduce_i8_noalloc(partials, outs, n: int | None = None, stream=None) -> None:
    n = _numel(partials[0]) if n is None else n
    _check("bq_ring_allreduce_i8_noalloc",
           _L().bq_ring_allreduce_i8_noalloc(len(partials), n, _ptrs(partials), _ptrs(outs),
                                            _stream(stream)))


def bq_a2a_allreduce_i8(partials, q_send, s_send, red, q_bcast, s_bcast, outs,
                        n: int | None = None, stream=None) -> None:
    n = _numel(partials[0]) if n is None else n
    _check("bq_a2a_allreduce_i8",
           _L().bq_a2a_allreduce_i8(len(partials), n, _ptrs(partials), _ptrs(q_send), _ptrs(s_send),
                                   _ptr(red), _ptr(q_bcast), _ptr(s_bcast), _ptrs(outs),
                                   _stream(stream)))


# ---- MXFP8 -----------------------------------------------------------------------------------

def bq_quant_mx(x, v, e8m0, rows: int | None = None, cols: int | None = None,
                ldx: int | None = None, ldv: int | None = None, lds: int | None = None,
                stream=None) -> None:
    rows = x.shape[0] if rows is None else rows
    cols = x.shape[1] if cols is None else cols
    ldx = x.stride(0) if ldx is None else ldx
    ldv = v.stride(0) if ldv is None else ldv
    lds = e8m0.stride(0) if lds is None else lds
    _check("bq_quant_mx", _L().bq_quant_mx(_ptr(x), rows, cols, ldx, _ptr(v), ldv, _ptr(e8m0), lds,
                                          _stream(stream)))


def bq_dequant_mx(v, e8m0, y, rows: int | None = None, cols: int | None = None,
                  ldv: int | None = None, lds: int | None = None, ldy: int | None = None,
                  stream=None) -> None:
    rows = y.shape[0] if rows is None else rows
    cols = y.shape[1] if cols is None else cols
    ldv = v.stride(0) if ldv is None else ldv
    lds = e8m0.stride(0) if lds is None else lds
    ldy = y.stride(0) if ldy is None else ldy
    _check("bq_dequant_mx", _L().bq_dequant_mx(_ptr(v), ldv, _ptr(e8m0), lds, rows, cols, _ptr(y),
                                              ldy, _stream(stream)))


def bq_quant_mx_slice(x, col_off: int, v, e8m0, capacity_rows: int | None = None,
                      rows: int | None = None, cols: int | None = None, ldx: int | None = None,
                      ldv: int | None = None, lds: int | None = None, stream=None) -> None:
    rows = x.shape[0] if rows is None else rows
    cols = x.shape[1] if cols is None else cols
    ldx = x.stride(0) if ldx is None else ldx
    ldv = v.stride(0) if ldv is None else ldv
    lds = e8m0.stride(0) if lds is None else lds
    capacity_rows = v.shape[0] if capacity_rows is None else capacity_rows
    _check("bq_quant_mx_slice",
           _L().bq_quant_mx_slice(_ptr(x), rows, cols, ldx, col_off, _ptr(v), ldv, _ptr(e8m0), lds,
                                 capacity_rows, _stream(stream)))


def bq_quant_mx_f16(x, v, e8m0, rows: int | None = None, cols: int | None = None,
                    ldx: int | None = None, ldv: int | None = None, lds: int | None = None,
                    stream=None) -> None:
    """bq_quant_mx on IEEE binary16 input (x: torch.float16 or int16 bit views)."""
    rows = x.shape[0] if rows is None else rows
    cols = x.shape[1] if cols is None else cols
    ldx = x.stride(0) if ldx is None else ldx
    ldv = v.stride(0) if ldv is None else ldv
    lds = e8m0.stride(0) if lds is None else lds
    _check("bq_quant_mx_f16", _L().bq_quant_mx_f16(_ptr(x), rows, cols, ldx, _ptr(v), ldv,
                                                  _ptr(e8m0), lds, _stream(stream)))


def bq_quant_mx_slice_f16(x, col_off: int, v, e8m0, capacity_rows: int | None = None,
                          rows: int | None = None, cols: int | None = None,
                          ldx: int | None = None, ldv: int | None = None, lds: int | None = None,
                          stream=None) -> None:
    """bq_quant_mx_slice on an IEEE binary16 slice."""
    rows = x.shape[0] if rows is None else rows
    cols = x.shape[1] if cols is None else cols
    ldx = x.stride(0) if ldx is None else ldx
    ldv = v.stride(0) if ldv is None else ldv
    lds = e8m0.stride(0) if lds is None else lds
    capacity_rows = v.shape[0] if capacity_rows is None else capacity_rows
    _check("bq_quant_mx_slice_f16",
           _L().bq_quant_mx_slice_f16(_ptr(x), rows, cols, ldx, col_off, _ptr(v), ldv, _ptr(e8m0),
                                     lds, capacity_rows, _stream(stream)))


def bq_mm_mx(xv, xe, wv, we, y, M: int | None = None, N: int | None = None,
             K: int | None = None, stream=None) -> None:
    """Y = bf16(X W^T) from MXFP8 X (xv (M, K) u8, xe (M, K/32) u8) and W (wv (N, K),
    we (N, K/32)) into y (M, N) bf16; leading dimensions from the tensors' row strides."""
    M = y.shape[0] if M is None else M
    N = y.shape[1] if N is None else N
    K = xv.shape[1] if K is None else K
    _check("bq_mm_mx", _L().bq_mm_mx(_ptr(xv), xv.stride(0), _ptr(xe), xe.stride(0), _ptr(wv),
                                    wv.stride(0), _ptr(we), we.stride(0), M, N, K, _ptr(y),
                                    y.stride(0), _stream(stream)))


def bq_mx_scale_mfma_bytes(rows: int, cols: int) -> int:
    """Bytes of the scaled-MFMA scale layout for rows x cols (-1 for invalid sizes)."""
    return _L().bq_mx_scale_mfma_bytes(rows, cols)


def bq_quant_mx_slice_mfma(x, col_off: int, v, e8m0, capacity_rows: int | None = None,
                           total_cols: int | None = None, rows: int | None = None,
                           cols: int | None = None, ldx: int | None = None,
                           ldv: int | None = None, f16: bool = False, stream=None) -> None:
    """Staged slice x (rows, cols) into columns [col_off, col_off+cols) of v and its scale
    bytes into e8m0, the scaled-MFMA layout of capacity_rows x total_cols (defaults: v's
    rows and columns)."""
    rows = x.shape[0] if rows is None else rows
    cols = x.shape[1] if cols is None else cols
    ldx = x.stride(0) if ldx is None else ldx
    ldv = v.stride(0) if ldv is None else ldv
    capacity_rows = v.shape[0] if capacity_rows is None else capacity_rows
    total_cols = v.shape[1] if total_cols is None else total_cols
    name = "bq_quant_mx_slice_mfma_f16" if f16 else "bq_quant_mx_slice_mfma"
    _check(name, getattr(_L(), name)(_ptr(x), rows, cols, ldx, col_off, _ptr(v), ldv, total_cols,
                                     _ptr(e8m0), capacity_rows, _stream(stream)))


def bq_quant_mx_slice_mfma_f16(x, col_off: int, v, e8m0, **kw) -> None:
    bq_quant_mx_slice_mfma(x, col_off, v, e8m0, f16=True, **kw)


def bq_dequant_mx_mfma(v, e8m0, y, scale_rows: int | None = None, rows: int | None = None,
                       cols: int | None = None, stream=None) -> None:
    rows = y.shape[0] if rows is None else rows
    cols = y.shape[1] if cols is None else cols
    scale_rows = v.shape[0] if scale_rows is None else scale_rows
    _check("bq_dequant_mx_mfma",
           _L().bq_dequant_mx_mfma(_ptr(v), v.stride(0), _ptr(e8m0), scale_rows, rows, cols,
                                  _ptr(y), y.stride(0), _stream(stream)))


def bq_mm_mx_mfma(xv, xe, wv, we, y, xe_rows: int | None = None, we_rows: int | None = None,
                  M: int | None = None, N: int | None = None, K: int | None = None,
                  stream=None) -> None:
    """bq_mm_mx with xe, we in the scaled-MFMA layout (laid out for xe_rows / we_rows rows,
    default xv's and wv's row counts)."""
    M = y.shape[0] if M is None else M
    N = y.shape[1] if N is None else N
    K = xv.shape[1] if K is None else K
    xe_rows = xv.shape[0] if xe_rows is None else xe_rows
    we_rows = wv.shape[0] if we_rows is None else we_rows
    _check("bq_mm_mx_mfma",
           _L().bq_mm_mx_mfma(_ptr(xv), xv.stride(0), _ptr(xe), xe_rows, _ptr(wv), wv.stride(0),
                             _ptr(we), we_rows, M, N, K, _ptr(y), y.stride(0), _stream(stream)))


def bq_mx_staging_bytes(capacity_rows: int, total_cols: int) -> tuple[int, int]:
    vb, sb = ctypes.c_int64(), ctypes.c_int64()
    _check("bq_mx_staging_bytes",
           _L().bq_mx_staging_bytes(capacity_rows, total_cols, ctypes.byref(vb), ctypes.byref(sb)))
    return vb.value, sb.value


# ---- flat MXFP8 on the collective topologies (v: u8[n] E4M3, e8m0: u8[n/32]) -----------

def bq_quant_mx_batch(xs, vs, es, n: int | None = None, stream=None) -> None:
    n = _numel(xs[0]) if n is None else n
    _check("bq_quant_mx_batch", _L().bq_quant_mx_batch(len(xs), _ptrs(xs), n, _ptrs(vs), _ptrs(es),
                                                      _stream(stream)))


def bq_dequant_mx_batch(vs, es, ys, n: int | None = None, stream=None) -> None:
    n = _numel(ys[0]) if n is None else n
    _check("bq_dequant_mx_batch", _L().bq_dequant_mx_batch(len(vs), _ptrs(vs), _ptrs(es), n,
                                                          _ptrs(ys), _stream(stream)))


def bq_ring_hop_mx(v_in, e_in, local, v_out, e_out, n: int | None = None, stream=None) -> None:
    n = _numel(local) if n is None else n
    _check("bq_ring_hop_mx", _L().bq_ring_hop_mx(_ptr(v_in), _ptr(e_in), _ptr(local), n,
                                                _ptr(v_out), _ptr(e_out), _stream(stream)))


def bq_ring_hop_mx_batch(v_in, e_in, local, v_out, e_out, n: int | None = None,
                         stream=None) -> None:
    n = _numel(local[0]) if n is None else n
    _check("bq_ring_hop_mx_batch",
           _L().bq_ring_hop_mx_batch(len(v_in), _ptrs(v_in), _ptrs(e_in), _ptrs(local), n,
                                    _ptrs(v_out), _ptrs(e_out), _stream(stream)))


def bq_dequant_accum_mx(v_srcs, e_srcs, y, n: int | None = None, stream=None) -> None:
    n = _numel(y) if n is None else n
    _check("bq_dequant_accum_mx",
           _L().bq_dequant_accum_mx(len(v_srcs), _ptrs(v_srcs), _ptrs(e_srcs), n, _ptr(y),
                                   _stream(stream)))


def bq_a2a_reduce_mx(nseg: int, v_srcs, e_srcs, v_out, e_out, y_out=None, red=None,
                     seg_n: int | None = None, stream=None) -> None:
    seg_n = _numel(v_out) // nseg if seg_n is None else seg_n
    ys = _ptrs(y_out) if y_out is not None else None
    _check("bq_a2a_reduce_mx",
           _L().bq_a2a_reduce_mx(nseg, len(v_srcs), _ptrs(v_srcs), _ptrs(e_srcs), seg_n,
                                 _ptr(v_out), _ptr(e_out), ys, _ptr(red), _stream(stream)))


def bq_allgather_dequant_mx(v, e8m0, outs, skip_own: bool = False, n: int | None = None,
                            stream=None) -> None:
    n = _numel(v) if n is None else n
    _check("bq_allgather_dequant_mx",
           _L().bq_allgather_dequant_mx(len(outs), _ptr(v), _ptr(e8m0), n, _ptrs(outs),
                                        int(skip_own), _stream(stream)))


def bq_ring_allreduce_mx(partials, v_wire, e_wire, outs, n: int | None = None,
                         stream=None) -> None:
    n = _numel(partials[0]) if n is None else n
    _check("bq_ring_allreduce_mx",
           _L().bq_ring_allreduce_mx(len(partials), n, _ptrs(partials), _ptr(v_wire), _ptr(e_wire),
                                    _ptrs(outs), _stream(stream)))


def bq_a2a_allreduce_mx(partials, v_send, e_send, red, v_bcast, e_bcast, outs,
                        n: int | None = None, stream=None) -> None:
    n = _numel(partials[0]) if n is None else n
    _check("bq_a2a_allreduce_mx",
           _L().bq_a2a_allreduce_mx(len(partials), n, _ptrs(partials), _ptrs(v_send), _ptrs(e_send),
                                   _ptr(red), _ptr(v_bcast), _ptr(e_bcast), _ptrs(outs),
                                   _stream(stream)))


# ---- E4M3 128-block codec ------------------------------------------------------------------

def bq_quant_e4m3_b128(x, v, scale, n: int | None = None, stream=None) -> None:
    n = _numel(x) if n is None else n
    _check("bq_quant_e4m3_b128", _L().bq_quant_e4m3_b128(_ptr(x), n, _ptr(v), _ptr(scale),
                                                        _stream(stream)))


def bq_dequant_e4m3_b128(v, scale, y, n: int | None = None, stream=None) -> None:
    n = _numel(v) if n is None else n
    _check("bq_dequant_e4m3_b128", _L().bq_dequant_e4m3_b128(_ptr(v), _ptr(scale), n, _ptr(y),
                                                            _stream(stream)))


# ---- host helpers --------------------------------------------------------------------------

def bq_mm_tile_cols(M: int, N: int, cus: int) -> int:
    """Column count (224 or 256) of the GEMM's workgroup tiles for M x N on `cus` compute
    units (-1 for invalid sizes)."""
    return _L().bq_mm_tile_cols(M, N, cus)


def bq_wire_bytes_b128(n: int) -> int:
    return _L().bq_wire_bytes_b128(n)


def bq_status_str(status: int) -> str:
    return _L().bq_status_str(status).decode()


def bq_version() -> str:
    return _L().bq_version().decode()
