"""Seeded synthetic inputs for the block-quantized wire codecs.

A thin ctypes wrapper over ``bqgen.c``.  This module draws numbers only; it
holds none of the codecs' arithmetic, and both the CPU oracle's tests and the
GPU tests / benchmark take their inputs from it.

Config ids (shapes are one rank's or one slice's tensor):

====  ==============  =====================================================
cfg   rows x cols     values
====  ==============  =====================================================
1     512 x 7168      N(0,1), x50 outliers w.p. 1e-3, 2% zero blocks
2     3072 x 7168     N(0, 0.5) per rank
3     3072 x 7168     0.3 * Student-t(4) per rank
4     4096 x 7168     N(0,1) * per-row gain, log-uniform in [1e-3, 1e2]
5     16384 x 7168    Student-t(3), 1% zero blocks, +-1e3 spikes w.p. 1e-5
6     any             N(0,1)
7     any             0.3 * Student-t(4)
====  ==============  =====================================================
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bqgen.c")
_LIB = os.path.join(_HERE, "libbqgen.so")
_lib = None


def build() -> str:
    """Compile ``libbqgen.so`` next to its source (gcc, OpenMP)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.bqgen_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        lib.bqgen_rows.restype = None
        lib.bqgen_rows_fmt.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.bqgen_rows_fmt.restype = None
        lib.bqgen_shape.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int64)]
        lib.bqgen_shape.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Worker threads for generation: OMP_NUM_THREADS if set, else the CPU count (max 16)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def shape(cfg: int) -> tuple[int, int]:
    """(rows, cols) of one rank's tensor for a named config (1..5)."""
    r, c = ctypes.c_int64(), ctypes.c_int64()
    if _load().bqgen_shape(cfg, ctypes.byref(r), ctypes.byref(c)) != 0:
        raise ValueError(f"config {cfg} has no fixed shape")
    return r.value, c.value


def rows(cfg: int, rank: int, row0: int, nrows: int, cols: int | None = None,
         out: np.ndarray | None = None, fmt: str = "bf16") -> np.ndarray:
    """bf16 (or, with fmt="f16", IEEE binary16) bit patterns (uint16) of rows
    [row0, row0+nrows) of rank's tensor."""
    if cols is None:
        cols = shape(cfg)[1]
    if cols % 128 != 0:
        raise ValueError("cols must be a multiple of 128")
    if out is None:
        out = np.empty((nrows, cols), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == nrows * cols
    if fmt not in ("bf16", "f16"):
        raise ValueError(f"unknown format {fmt}")
    _load().bqgen_rows_fmt(cfg, rank, row0, nrows, cols, out.ctypes.data, threads(),
                           1 if fmt == "f16" else 0)
    return out


def tensor(cfg: int, rank: int, nrows: int | None = None, cols: int | None = None,
           out: np.ndarray | None = None) -> np.ndarray:
    """A whole rank tensor (or its first nrows rows) as uint16 bf16 bits, shape (rows, cols)."""
    r, c = (shape(cfg) if cfg <= 5 else (nrows, cols))
    if nrows is not None:
        r = nrows
    if cols is not None:
        c = cols
    return rows(cfg, rank, 0, r, c, out=out)
