"""Exact-rational brute force for tiny inputs, written independently of the C oracle.

Every value is a ``fractions.Fraction``; each IEEE binary32 or bf16 rounding
the codec definitions call for is applied explicitly by ``round_binary`` (round
to nearest, ties to even, gradual underflow), and every "round to integer" is
an argmin over the candidate integers.  Nothing here uses hardware floating
point for the arithmetic under test, so a mistake in the C oracle's use of
float operations, rintf, frexpf or ldexpf shows up as a mismatch.
"""
from __future__ import annotations

from fractions import Fraction
from math import floor

import numpy as np

F32 = (24, -149, 128)     # (significand bits, smallest quantum exponent, overflow exponent)
BF16 = (8, -133, 128)


def round_binary(v: Fraction, fmt=F32) -> Fraction:
    """Nearest value of the binary format to v, ties to an even last significand bit."""
    p, qmin, emax = fmt
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - (p - 1), qmin)
    quantum = Fraction(2) ** qexp
    k = a / quantum
    fl = floor(k)
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** emax:
        raise OverflowError("rounds to infinity")
    return sign * r


def rn32(v: Fraction) -> Fraction:
    return round_binary(v, F32)


def bf16_bits_to_fraction(h: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern, decoded from its fields."""
    sign = -1 if (h >> 15) & 1 else 1
    ex = (h >> 7) & 0xFF
    man = h & 0x7F
    assert ex != 0xFF, "non-finite"
    if ex == 0:
        return sign * Fraction(man) * Fraction(2) ** -133
    return sign * Fraction(128 + man) * Fraction(2) ** (ex - 127 - 7)


def fraction_to_bf16_bits(v: Fraction) -> int:
    """bf16 bit pattern of the bf16 rounding of v (v must round to a finite value).  Zero
    gives +0; a negative v that rounds to zero gives -0, as IEEE rounding keeps the sign."""
    r = round_binary(v, BF16)
    if r == 0:
        return 0x8000 if v < 0 else 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if e < -126:                                   # subnormal
        return sign | int(a / Fraction(2) ** -133)
    man = int(a / Fraction(2) ** (e - 7)) - 128
    return sign | ((e + 127) << 7) | man


def nearest_int_even(t: Fraction, lo: int, hi: int) -> int:
    """argmin over k in [lo, hi] of |t - k|, ties to the even k.  With t = N/D (D > 0) the
    distances are compared as the integers |N - kD|, which orders them the same way."""
    t = Fraction(t)
    num, den = t.numerator, t.denominator
    best = None
    for k in range(lo, hi + 1):
        key = (abs(num - k * den), k % 2)
        if best is None or key < best[0]:
            best = (key, k)
    return best[1]


# ---- E4M3FN from its field definition ---------------------------------------------

def e4m3_value(code: int) -> Fraction | None:
    ex = (code >> 3) & 0xF
    man = code & 7
    if ex == 0xF and man == 7:
        return None
    mag = Fraction(man, 512) if ex == 0 else Fraction(8 + man, 8) * Fraction(2) ** (ex - 7)
    return -mag if code & 0x80 else mag


def e4m3_nearest(v: Fraction, negative_zero: bool = False) -> int:
    """Nearest finite code by search over all 127 magnitudes, ties to even mantissa,
    saturating at 448; the sign bit follows the sign of v (and of a negative zero)."""
    a = abs(v)
    best = None
    for c in range(0x7F):
        d = abs(e4m3_value(c) - a)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    code = best[1]
    neg = v < 0 or (v == 0 and negative_zero)
    return code | (0x80 if neg else 0)


# ---- block codecs -------------------------------------------------------------------

def quant_i8_block(xs: list[Fraction]):
    """(q list, scale Fraction) by the block-INT8 definition."""
    amax = max(abs(x) for x in xs)
    if amax == 0:
        return [0] * len(xs), Fraction(0)
    s = rn32(amax / 127)
    return [nearest_int_even(rn32(x / s), -127, 127) for x in xs], s


def dequant_i8_value(q: int, s: Fraction) -> int:
    return fraction_to_bf16_bits(rn32(q * s))


def hop_block(q_in, s_in: Fraction, local_bits):
    sums = [rn32(rn32(q * s_in) + bf16_bits_to_fraction(h)) for q, h in zip(q_in, local_bits)]
    return quant_i8_block(sums)


def accum_value(qs, ss) -> int:
    acc = Fraction(0)
    for q, s in zip(qs, ss):
        acc = rn32(acc + rn32(q * s))
    return fraction_to_bf16_bits(acc)


def e8m0_byte(amax: Fraction) -> int:
    if amax == 0:
        return 127
    d = rn32(amax / 448)
    for e in range(-127, 128):
        if Fraction(2) ** e >= d:
            return e + 127
    return 254


# ---- MXFP8 collectives ----------------------------------------------------------------

def mx_group(values: list[Fraction], neg_zero: list[bool]):
    """(byte, codes) of one 32-value group of binary32 values by the MXFP8 definition;
    neg_zero[i] marks a value that is an IEEE negative zero."""
    byte = e8m0_byte(max(abs(t) for t in values))
    sc = Fraction(2) ** (byte - 127)
    codes = [e4m3_nearest(rn32(t / sc), negative_zero=nz) for t, nz in zip(values, neg_zero)]
    return byte, codes


def mx_hop_group(codes_in, byte_in: int, local_bits):
    """One group of the MX ring hop: binary32 sums of the dequantized payload and the bf16
    local partial, requantized.  IEEE signed zeros: a sum is -0 only when both addends
    are -0 (an exact zero sum of opposite values is +0 under round-to-nearest)."""
    sc = Fraction(2) ** (byte_in - 127)
    sums, negz = [], []
    for c, h in zip(codes_in, local_bits):
        dq = rn32(e4m3_value(c) * sc)
        s = rn32(dq + bf16_bits_to_fraction(h))
        sums.append(s)
        negz.append(s == 0 and c == 0x80 and h == 0x8000)
    return mx_group(sums, negz)


def mx_accum_value(codes, bytes_) -> int:
    """bf16 bits of the in-order binary32 sum of the sources' MX values (from +0)."""
    acc = Fraction(0)
    for c, b in zip(codes, bytes_):
        acc = rn32(acc + rn32(e4m3_value(c) * Fraction(2) ** (b - 127)))
    return fraction_to_bf16_bits(acc)


def f16_bits_to_fraction(h: int) -> Fraction:
    """Exact value of a finite IEEE binary16 bit pattern, decoded from its fields."""
    sign = -1 if (h >> 15) & 1 else 1
    ex = (h >> 10) & 0x1F
    man = h & 0x3FF
    assert ex != 0x1F, "non-finite"
    if ex == 0:
        return sign * Fraction(man) * Fraction(2) ** -24
    return sign * Fraction(1024 + man) * Fraction(2) ** (ex - 25)
