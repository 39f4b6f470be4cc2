"""Reader for the hand-derived worked examples in tests/golden/*.txt."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name: str) -> list[dict[str, list[str]]]:
    """Records separated by blank lines; lines 'key: v1 v2 ...'; '#' starts a comment."""
    recs, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                if cur:
                    recs.append(cur)
                    cur = {}
                continue
            key, _, val = line.partition(":")
            cur[key.strip()] = val.split()
    if cur:
        recs.append(cur)
    return recs


def read_kv(name: str) -> dict[str, str]:
    out = {}
    for rec in read(name):
        for k, v in rec.items():
            out[k] = v[0]
    return out


def bf16_bits_exact(tok: str) -> int:
    """bf16 bits of a decimal or hex-float literal that must be exactly a bf16 value."""
    hexfloat = tok.lstrip("-").startswith("0x") and "p" in tok
    v = float.fromhex(tok) if hexfloat else float(tok)
    f32 = np.array([v], dtype=np.float32)
    exact = Fraction(v) if hexfloat else Fraction(tok)
    if Fraction(float(f32[0])) != exact and not (v == 0.0):
        raise ValueError(f"{tok} is not exactly a binary32 value")
    bits = int(f32.view(np.uint32)[0])
    if bits & 0xFFFF:
        raise ValueError(f"{tok} is not exactly a bf16 value")
    if tok.startswith("-") and v == 0.0:
        return 0x8000
    return bits >> 16


def padded_block(tokens: list[str], size: int) -> np.ndarray:
    out = np.zeros(size, np.uint16)
    for i, t in enumerate(tokens):
        out[i] = bf16_bits_exact(t)
    return out


def hexint(tok: str) -> int:
    return int(tok, 16)
