"""Helpers for GPU tests: numpy <-> device tensors of bit patterns, and logging of the
case that is about to run (flushed, so a failing GPU step is always named)."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"

_TORCH = {np.uint16: torch.int16, np.int8: torch.int8, np.uint8: torch.uint8,
          np.float32: torch.float32, np.int16: torch.int16}


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def empty(shape, dtype) -> torch.Tensor:
    return torch.empty(shape, dtype=_TORCH[np.dtype(dtype).type], device=DEV)


def filled(shape, dtype, byte: int) -> torch.Tensor:
    """A device buffer whose every byte is `byte` (canary)."""
    t = torch.full((int(np.prod(shape)) * np.dtype(dtype).itemsize,), byte, dtype=torch.uint8,
                   device=DEV)
    return t.view(_TORCH[np.dtype(dtype).type]).reshape(shape)


def host(t: torch.Tensor, dtype) -> np.ndarray:
    a = t.detach().cpu().contiguous().numpy()
    return a.view(dtype)


def sync() -> None:
    torch.cuda.synchronize()
