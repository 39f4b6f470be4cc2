"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with itself.  The pins are:
  * worked examples derived by hand from the pages' rules (tests/golden/);
  * an exact-rational brute force written independently (tests/bruteforce.py);
  * library routines for the special cases that reduce to them (torch's
    round-to-nearest-even bf16 and E4M3FN conversions);
  * closed forms, exhaustive sweeps and invariants (half-step bound, zero
    blocks, canonical payload, ring/A2A sums that are exact by construction).
"""
from __future__ import annotations

import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import bruteforce as bf
import goldens
import oracle
import workloads


def f32(bits_u16: np.ndarray) -> np.ndarray:
    return (bits_u16.astype(np.uint32) << 16).view(np.float32)


def all_finite_bf16() -> np.ndarray:
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return h[((h >> 7) & 0xFF) != 0xFF]


# ---------------------------------------------------------------------------------------
# scalar conversions
# ---------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_structured_sweep():
    """Every bf16 upper half with the interesting lower halves (exact, just above, just
    below and exactly at the tie, both parities) against torch's RNE conversion."""
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    hi = np.arange(65536, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]
    bits = ((hi[:, None] << 16) | lows[None, :]).reshape(-1)
    vals = bits.view(np.float32)
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    L = oracle.lib()
    got = np.fromiter((L.orc_f32_to_bf16(float(v)) for v in vals), dtype=np.uint16, count=vals.size)
    finite_in = np.isfinite(vals)
    assert np.array_equal(got[finite_in], want[finite_in])


def test_bf16_rounding_matches_exact_nearest_even():
    rng = random.Random(11)
    L = oracle.lib()
    for _ in range(3000):
        bits = rng.getrandbits(32)
        if (bits >> 23) & 0xFF == 0xFF:
            continue
        v = np.array([bits], np.uint32).view(np.float32)[0]
        want = bf.fraction_to_bf16_bits(Fraction(float(v))) if abs(float(v)) < 3.38e38 else None
        if want is None:
            continue
        got = L.orc_f32_to_bf16(float(v))
        if float(v) == 0.0:
            assert got & 0x7FFF == 0
            continue
        assert got == want, hex(bits)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        ref = bf.e4m3_value(c)
        if ref is None:
            assert np.isnan(got) and np.isnan(want[c])
            continue
        assert Fraction(got) == ref and got == want[c], c
    # closed forms of the format: largest finite, smallest normal, smallest subnormal, one
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x38) == 1.0


def _torch_e4m3_saturating(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_inputs_match_torch():
    h = all_finite_bf16()
    vals = f32(h)
    L = oracle.lib()
    got = np.fromiter((L.orc_e4m3_encode(float(v)) for v in vals), dtype=np.uint8, count=vals.size)
    want = _torch_e4m3_saturating(vals)
    assert np.array_equal(got, want)


def test_e4m3_encode_midpoints_and_random_fp32():
    L = oracle.lib()
    mags = sorted(float(bf.e4m3_value(c)) for c in range(0x7F))
    probes = []
    for a, b in zip(mags[:-1], mags[1:]):
        m = np.float32((a + b) / 2)
        for d in (-1, 0, 1):
            probes.append(np.nextafter(m, np.float32(np.inf)) if d > 0 else
                          (np.nextafter(m, np.float32(-np.inf)) if d < 0 else m))
    rng = np.random.default_rng(5)
    probes = np.array(probes, np.float32)
    rand = (rng.standard_normal(40000) * np.exp(rng.uniform(-14, 7, 40000))).astype(np.float32)
    vals = np.concatenate([probes, -probes, rand, np.array([448, 449, 463.99, 464, 480, 1e30, -1e30,
                                                           2.0 ** -10, 2.0 ** -149], np.float32)])
    got = np.fromiter((L.orc_e4m3_encode(float(v)) for v in vals), dtype=np.uint8, count=vals.size)
    assert np.array_equal(got, _torch_e4m3_saturating(vals))
    # brute-force nearest search on a subsample (independent of torch)
    for v in list(vals[:200]) + list(rand[:200]):
        assert L.orc_e4m3_encode(float(v)) == bf.e4m3_nearest(Fraction(float(v)),
                                                              negative_zero=np.signbit(v))


def test_e4m3_encode_signed_zero_and_saturation():
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(464.0) == 0x7E        # torch would give NaN here; we saturate
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(-(2.0 ** -11)) == 0x80


def test_e8m0_exhaustive_over_bf16_amax():
    """Smallest power of two >= fl32(amax/448) by brute force, for every positive finite
    bf16 amax, and the closed form for amax = m * 2^k: e = k - 8 + [m > 1.75]."""
    h = all_finite_bf16()
    h = h[(h > 0) & (h < 0x8000)]
    amax = f32(h)
    d = (amax / np.float32(448.0)).astype(np.float64)       # IEEE binary32 division
    e = np.full(d.shape, 200, np.int64)
    for k in range(127, -128, -1):
        e = np.where(2.0 ** k >= d, k, e)
    e = np.where(e == 200, 127, e)                            # (never hit for bf16 amax)
    want = (e + 127).astype(np.uint8)
    L = oracle.lib()
    got = np.fromiter((L.orc_e8m0_scale(float(a)) for a in amax), dtype=np.uint8, count=amax.size)
    assert np.array_equal(got, want)
    # closed form where no clamping happens
    m, k = np.frexp(amax.astype(np.float64))   # amax = m 2^k, m in [0.5, 1)
    sig, ex = m * 2, k - 1                      # significand in [1, 2)
    closed = ex - 8 + (sig > 1.75)
    ok = (closed >= -127) & (closed <= 127)
    assert np.array_equal(got[ok].astype(np.int64) - 127, closed[ok])
    assert oracle.e8m0_scale(0.0) == 127        # the page's all-zero rule


def test_e8m0_fp32_amax_bruteforce():
    rng = random.Random(3)
    L = oracle.lib()
    for _ in range(400):
        a = abs(np.float32(rng.lognormvariate(0, 30)))
        if not np.isfinite(a) or a == 0:
            continue
        assert L.orc_e8m0_scale(float(a)) == bf.e8m0_byte(Fraction(float(a)))


# ---------------------------------------------------------------------------------------
# block INT8
# ---------------------------------------------------------------------------------------

def test_i8_worked_examples():
    for rec in goldens.read("i8_worked.txt"):
        x = goldens.padded_block(rec["x"], 128)
        q, s = oracle.quant_i8(x)
        want_scale = np.array([goldens.hexint(rec["scale"][0])], np.uint32).view(np.float32)
        assert s.view(np.uint32)[0] == want_scale.view(np.uint32)[0], rec["name"]
        want_q = np.zeros(128, np.int8)
        want_q[:len(rec["q"])] = [int(t) for t in rec["q"]]
        assert np.array_equal(q, want_q), rec["name"]
        y = oracle.dequant_i8(q, s)
        want_y = np.zeros(128, np.uint16)
        want_y[:len(rec["y"])] = [goldens.hexint(t) for t in rec["y"]]
        assert np.array_equal(y, want_y), rec["name"]


def _bf_quant(x_bits: np.ndarray):
    qs, ss = [], []
    for b in range(x_bits.size // 128):
        xs = [bf.bf16_bits_to_fraction(int(h)) for h in x_bits[b * 128:(b + 1) * 128]]
        q, s = bf.quant_i8_block(xs)
        qs += q
        ss.append(s)
    return np.array(qs, np.int8), ss


def test_i8_quant_bruteforce_tiny():
    rng = np.random.default_rng(7)
    for trial in range(6):
        x = workloads.rows(7 if trial % 2 else 6, trial, 0, 1, 384)[0]
        if trial == 2:     # exact ties: power-of-two scale and half-integer multiples
            x = np.zeros(384, np.uint16)
            vals = np.float32(rng.integers(-254, 255, 384) / 2.0)
            vals[0] = 127.0
            x = (vals.view(np.uint32) >> 16).astype(np.uint16)
        q, s = oracle.quant_i8(x)
        wq, ws = _bf_quant(x)
        assert np.array_equal(q, wq)
        assert [Fraction(float(v)) for v in s] == ws
        y = oracle.dequant_i8(q, s)
        wy = [bf.dequant_i8_value(int(q[i]), ws[i // 128]) for i in range(x.size)]
        assert np.array_equal(y, np.array(wy, np.uint16))


def test_i8_scale_is_correctly_rounded_amax_over_127():
    """scale is the binary32 value nearest amax/127 (checked with exact rationals)."""
    h = all_finite_bf16()
    h = h[(h > 0) & (h < 0x8000)][::7]
    L = oracle.lib()
    for hb in h:
        x = np.zeros(128, np.uint16)
        x[5] = hb
        _, s = oracle.quant_i8(x)
        amax = bf.bf16_bits_to_fraction(int(hb))
        assert Fraction(float(s[0])) == bf.rn32(amax / 127)


def test_i8_invariants_on_cfg1_tensor():
    x = workloads.tensor(1, 0)
    q, s = oracle.quant_i8(x)
    xf = f32(x.reshape(-1)).astype(np.float64).reshape(-1, 128)
    qb = q.astype(np.int64).reshape(-1, 128)
    zero = np.all(xf == 0, axis=1)
    assert 0.01 < zero.mean() < 0.03                      # ~2% zero blocks by construction
    assert np.all(s[zero] == 0) and np.all(qb[zero] == 0)
    assert np.all(s[~zero] > 0)
    assert np.abs(qb).max() <= 127 and not np.any(qb == -128)
    assert np.all(np.abs(qb[~zero]).max(axis=1) == 127)   # the amax element maps to +-127
    # half-quantization-step bound, relative to the stored scale
    err = np.abs(xf - qb * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16))
    # materialized bf16: half step plus half a bf16 ulp
    y = f32(oracle.dequant_i8(q, s)).astype(np.float64).reshape(-1, 128)
    ulp = np.spacing(np.abs(y).astype(np.float32)).astype(np.float64) * 2 ** 16
    assert np.all(np.abs(xf - y) <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16) + ulp / 2)
    # 132-byte layout: n payload bytes plus 4 scale bytes per block
    assert q.nbytes + s.nbytes == 132 * (x.size // 128)


def test_i8_dequant_matches_torch_products():
    """bf16(fl32(q*scale)) for every q and a spread of scales, against torch's IEEE
    product and RNE bf16 conversion."""
    rng = np.random.default_rng(1)
    scales = np.concatenate([rng.lognormal(0, 8, 200).astype(np.float32),
                             np.array([1.0, 2.0 ** -140, 2.0 ** -126, 3.0e36], np.float32)])
    qv = np.arange(-127, 128, dtype=np.int8)
    for sc in scales:
        q = np.resize(qv, 256).astype(np.int8)
        s = np.full(2, sc, np.float32)
        got = oracle.dequant_i8(q, s)
        want = (torch.from_numpy(q.astype(np.float32)) * float(sc)).to(torch.bfloat16)
        assert np.array_equal(got, want.view(torch.int16).numpy().view(np.uint16))


def test_accum_single_source_is_dequant_and_zero_sources_are_neutral():
    x = workloads.rows(7, 0, 0, 2, 1024).reshape(-1)
    q, s = oracle.quant_i8(x)
    assert np.array_equal(oracle.dequant_accum_i8([q], [s]), oracle.dequant_i8(q, s))
    zq, zs = oracle.quant_i8(np.zeros_like(x))
    assert np.array_equal(oracle.dequant_accum_i8([zq, q, zq], [zs, s, zs]), oracle.dequant_i8(q, s))


def test_accum_respects_array_order_and_rounds_each_product():
    """Source order is part of the definition: (a - a) + b differs from a + b - a when b
    is absorbed by a.  And each product is rounded before the add (no FMA)."""
    n = 128
    q = [np.zeros(n, np.int8) for _ in range(3)]
    s = [np.ones(1, np.float32) for _ in range(3)]
    q[0][0], s[0][0] = 127, 2.0 ** 20
    q[1][0], s[1][0] = -127, 2.0 ** 20
    q[2][0], s[2][0] = 1, 2.0 ** -10
    assert oracle.dequant_accum_i8(q, s)[0] == 0x3A80                            # 2^-10
    assert oracle.dequant_accum_i8([q[0], q[2], q[1]], [s[0], s[2], s[1]])[0] == 0  # absorbed
    # product rounding: 3 * (1 + 2^-23) = 3 + 3*2^-23 rounds to 3 + 2^-21 (tie to even),
    # so the sum with -3 is exactly 2^-21 in either order.
    q2 = [np.zeros(n, np.int8), np.zeros(n, np.int8)]
    s2 = [np.array([np.float32(1 + 2.0 ** -23)], np.float32), np.array([1.0], np.float32)]
    q2[0][0], q2[1][0] = 3, -3
    got = oracle.dequant_accum_i8(q2, s2)[0]
    assert got == bf.fraction_to_bf16_bits(Fraction(2) ** -21)
    # With the rounded product second, a fused multiply-add onto acc = -3 would keep the
    # exact 3*2^-23 instead.  Onto acc = +0, as above, fusing rounds like the product.
    got = oracle.dequant_accum_i8(q2[::-1], s2[::-1])[0]
    assert got == bf.fraction_to_bf16_bits(Fraction(2) ** -21)
    assert got != bf.fraction_to_bf16_bits(3 * Fraction(2) ** -23)
    # brute force on random small cases
    rng = np.random.default_rng(4)
    for W in (1, 2, 3):
        xs = [workloads.rows(7, r, 0, 1, 256)[0] for r in range(W)]
        qs, ss = zip(*[oracle.quant_i8(x) for x in xs])
        got = oracle.dequant_accum_i8(list(qs), list(ss))
        for i in rng.integers(0, 256, 40):
            want = bf.accum_value([int(qq[i]) for qq in qs],
                                  [Fraction(float(sv[i // 128])) for sv in ss])
            assert got[i] == want


def test_ring_hop_bruteforce_and_identities():
    for trial in range(3):
        x = workloads.rows(6, trial, 0, 1, 256)[0]
        loc = workloads.rows(7, trial + 10, 0, 1, 256)[0]
        q, s = oracle.quant_i8(x)
        q2, s2 = oracle.ring_hop_i8(q, s, loc)
        for b in range(2):
            wq, ws = bf.hop_block([int(v) for v in q[b * 128:(b + 1) * 128]],
                                  Fraction(float(s[b])),
                                  [int(h) for h in loc[b * 128:(b + 1) * 128]])
            assert list(q2[b * 128:(b + 1) * 128]) == wq
            assert Fraction(float(s2[b])) == ws
    # local == 0, power-of-two scale and max |q| = 127: the hop is the identity
    q = np.random.default_rng(0).integers(-127, 128, 256).astype(np.int8)
    q[3], q[200] = 127, -127
    s = np.array([2.0 ** -3, 2.0 ** 5], np.float32)
    q2, s2 = oracle.ring_hop_i8(q, s, np.zeros(256, np.uint16))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    # local == -dequant(payload) exactly: the block sums to zero -> zero block
    loc = (np.float32(q[:128]) * np.float32(2.0 ** -3)).astype(np.float32)
    negloc = ((-loc).view(np.uint32) >> 16).astype(np.uint16)
    q3, s3 = oracle.ring_hop_i8(q[:128].copy(), s[:1].copy(), negloc)
    assert s3[0] == 0 and not q3.any()


def test_ring_hop_scale_underflow_is_a_zero_block():
    """A binary32 hop sum with 0 < amax < 127 * 2^-150 has a scale that rounds to 0; the
    block is stored as a zero block (scale 0, payload 0), which dequantizes to the same
    zeros as any payload would with that scale."""
    q = np.zeros(128, np.int8)
    q[7] = 1
    s = np.array([2.0 ** -149], np.float32)        # smallest subnormal binary32
    q2, s2 = oracle.ring_hop_i8(q, s, np.zeros(128, np.uint16))
    assert s2[0] == 0 and not q2.any()
    assert bf.rn32(Fraction(2) ** -149 / 127) == 0  # the scale really underflows


def test_ring_hop_clamps_the_quotients_of_few_bit_subnormal_scales():
    """A hop requantizes binary32 sums, whose block amax can be A * 2^-149 for a small
    integer A.  Its scale fl32(amax/127) is then a subnormal with only a few significant
    bits, so x/scale can exceed 127.5: A = 190 gives scale 2^-149 and quotient 190.  The
    block-INT8 range [-127, 127] clamps such quotients.  Every A in 128..16065 against the
    exact-rational brute force: payload [1, -1, 0, ...] with input scale A * 2^-149 and a
    zero local partial, so the sums are +-A * 2^-149 and zeros."""
    As = np.arange(128, 16066)
    nb = As.size
    q = np.zeros((nb, 128), np.int8)
    q[:, 0], q[:, 1] = 1, -1
    s = (As.astype(np.float64) * 2.0 ** -149).astype(np.float32)
    q2, s2 = oracle.ring_hop_i8(q.reshape(-1), s, np.zeros(nb * 128, np.uint16))
    q2 = q2.reshape(nb, 128)
    assert not q2[:, 2:].any()
    binding = 0
    for b, A in enumerate(As.tolist()):
        assert Fraction(float(s[b])) == A * Fraction(2) ** -149         # input scale exact
        wq, ws = bf.hop_block([1, -1, 0], A * Fraction(2) ** -149, [0, 0, 0])
        assert Fraction(float(s2[b])) == ws
        assert [int(q2[b, 0]), int(q2[b, 1]), 0] == wq, A
        binding += bf.rn32(A * Fraction(2) ** -149 / ws) > Fraction(255, 2)
    assert binding > 3000          # the clamp decides thousands of these blocks
    # the two cases worked by hand: scale 2^-149 with quotient 190, and scale 39 * 2^-149
    # with quotient 5000/39 = 128.2; both clamp to +-127
    for A, scale_units in ((190, 1), (5000, 39)):
        b = A - 128
        assert Fraction(float(s2[b])) == scale_units * Fraction(2) ** -149
        assert (int(q2[b, 0]), int(q2[b, 1])) == (127, -127)


def test_ring_allreduce_of_cancelling_partials_clamps_like_the_brute_force():
    """A W = 2 ring whose bf16 partials nearly cancel reaches the clamp through the public
    schedule.  The quantizing rank's block holds the pilot 2^-126 (q = 127 under the scale
    fl32(2^-126/127) = 66052 * 2^-149) and values k * 2^-133 with |k| <= K (q = k); the
    hopping rank holds minus the bf16 rounding of each dequantized value.  The hop sums are
    then -4 * 2^-149 at the pilot and 516 k * 2^-149 elsewhere, so the block amax is
    516 K * 2^-149 and for K <= 7 its scale 4 K * 2^-149 leaves the quotient 129, clamped to
    127.  The final payload and both ranks' outputs are checked against the exact-rational
    brute force of the schedule (chunk c quantized by rank c+1, hopped by rank c)."""
    W, nbc = 2, 9
    m = nbc * 128
    rng = np.random.default_rng(12)
    two = Fraction(2)
    quant_side = np.zeros((W, m), np.uint16)     # partial of the rank that quantizes chunk c
    hop_side = np.zeros((W, m), np.uint16)       # partial of the rank that hops chunk c
    for c in range(W):
        for b in range(nbc):
            K = b + 1 if b < 7 else (31 if b == 7 else 63)
            k = rng.integers(-K, K + 1, 128)
            k[0], k[1 + c], k[5] = 0, K, -K
            vals = [Fraction(int(v)) * two ** -133 for v in k]
            vals[0] = two ** -126
            blk = slice(b * 128, (b + 1) * 128)
            quant_side[c, blk] = [bf.fraction_to_bf16_bits(v) for v in vals]
            wq, ws = bf.quant_i8_block(vals)
            assert ws == 66052 * two ** -149 and wq[0] == 127 and wq[1:] == [int(v) for v in k[1:]]
            hop_side[c, blk] = [bf.fraction_to_bf16_bits(-bf.rn32(qv * ws)) for qv in wq]
    # rank r quantizes chunk (r - 1) mod W and hops chunk r
    partials = [np.zeros(W * m, np.uint16) for _ in range(W)]
    for c in range(W):
        partials[(c + 1) % W][c * m:(c + 1) * m] = quant_side[c]
        partials[c][c * m:(c + 1) * m] = hop_side[c]
    q_fin, s_fin, outs = oracle.ring_allreduce_i8(partials)
    clamped = 0
    for c in range(W):
        for b in range(nbc):
            blk = slice(b * 128, (b + 1) * 128)
            xs = [bf.bf16_bits_to_fraction(int(h)) for h in quant_side[c, blk]]
            q1, s1 = bf.quant_i8_block(xs)
            wq, ws = bf.hop_block(q1, s1, [int(h) for h in hop_side[c, blk]])
            off = c * m + b * 128
            assert Fraction(float(s_fin[off // 128])) == ws
            assert q_fin[off:off + 128].tolist() == wq
            want = [bf.dequant_i8_value(qv, ws) for qv in wq]
            for r in range(W):
                assert outs[r][off:off + 128].tolist() == want
            amax = 516 * (b + 1 if b < 7 else (31 if b == 7 else 63)) * two ** -149
            if bf.rn32(amax / ws) > Fraction(255, 2):
                clamped += 1
                assert wq[1 + c] == 127 and wq[5] == -127
    assert clamped == 2 * 7


def _chain_position(r: int, c: int, W: int) -> int:
    return (r - c - 1) % W


def _exact_ring_partials(W: int, blocks_per_chunk: int, seed: int):
    """Partials whose every ring stage is exact under the chunk schedule (chunk c starts at
    rank c+1 and collects c+2, ...): a pilot element per block makes the running amax
    127 * 2^j at chain position j, and the other elements are small multiples of 2^W so
    that every quantization is exact.  The ring result must equal the exact sum."""
    rng = np.random.default_rng(seed)
    m = blocks_per_chunk * 128
    n = W * m
    parts = []
    for r in range(W):
        v = (rng.integers(-3, 4, n) * 2.0 ** W).astype(np.float64)
        for c in range(W):
            pos = _chain_position(r, c, W)
            pilot = 127.0 if pos == 0 else 127.0 * 2.0 ** (pos - 1)
            v[c * m: (c + 1) * m: 128] = pilot
        parts.append(v)
    return parts


def _to_bf16_exact(v: np.ndarray) -> np.ndarray:
    b = v.astype(np.float32).view(np.uint32)
    assert not np.any(b & 0xFFFF)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_ring_allreduce_exact_sums_and_canonical_payload(W):
    parts = _exact_ring_partials(W, 2, W)
    exact = np.sum(parts, axis=0)
    pb = [_to_bf16_exact(p) for p in parts]
    qf, sf, outs = oracle.ring_allreduce_i8(pb)
    assert np.array_equal(f32(outs[0]).astype(np.float64), exact)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])          # every rank bit-identical
    assert np.array_equal(outs[0], oracle.dequant_i8(qf, sf))   # owner uses the same payload


def test_ring_allreduce_error_bound_and_schedule_on_random_data():
    W = 4
    parts = [workloads.rows(2, r, 0, 4, 512).reshape(-1) for r in range(W)]
    qf, sf, outs = oracle.ring_allreduce_i8(parts)
    exact = np.sum([f32(p).astype(np.float64) for p in parts], axis=0)
    y = f32(outs[0]).astype(np.float64)
    # each of the W quantizations of a block adds at most half its own step; the
    # final step scale is known; bound the earlier steps by the final-amax-based scale
    # of the partial sums computed in float64 (plus slack for fp32 sums and bf16)
    m = exact.size // W
    worst = np.zeros(exact.size // 128)
    for c in range(W):
        run = np.zeros(m)
        order = [(c + 1 + k) % W for k in range(W)]
        for r in order:
            run = run + f32(parts[r][c * m:(c + 1) * m]).astype(np.float64)
            worst[c * m // 128:(c + 1) * m // 128] += np.abs(run).reshape(-1, 128).max(1) / 127 / 2 * 1.05
    bound = np.repeat(worst, 128) + np.abs(y) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(y - exact) <= bound)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    # schedule pin: with W=2, chunk 0 is quantized by rank 1 and hopped by rank 0
    q1, s1 = oracle.quant_i8(parts[1][: parts[1].size // 2])
    qh, sh = oracle.ring_hop_i8(q1, s1, parts[0][: parts[0].size // 2])
    qf2, sf2, _ = oracle.ring_allreduce_i8(parts[:2])
    assert np.array_equal(qf2[: qh.size], qh) and np.array_equal(sf2[: sh.size], sh)


@pytest.mark.parametrize("W", [1, 2, 4])
def test_a2a_allreduce_exact_sums(W):
    """Pilot 127 per block in every source keeps each source scale 1 * 2^0 and the owner
    sum's amax 127 W; other elements are multiples of W, so every step is exact."""
    rng = np.random.default_rng(W)
    n = W * 256
    parts = []
    for r in range(W):
        v = (rng.integers(-2, 3, n) * float(W)).astype(np.float64)
        v[::128] = 127.0
        parts.append(v)
    exact = np.sum(parts, axis=0)
    red, qf, sf, outs = oracle.a2a_allreduce_i8([_to_bf16_exact(p) for p in parts])
    assert np.array_equal(f32(red).astype(np.float64), exact)
    assert np.array_equal(f32(outs[0]).astype(np.float64), exact)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.array_equal(outs[0], oracle.dequant_i8(qf, sf))


def test_a2a_requantizes_the_bf16_sum():
    """The broadcast payload is the block-INT8 quantization of the owner's bf16 sum."""
    W = 4
    parts = [workloads.rows(3, r, 0, 2, 1024).reshape(-1) for r in range(W)]
    red, qf, sf, outs = oracle.a2a_allreduce_i8(parts)
    q, s = oracle.quant_i8(red)
    assert np.array_equal(q, qf) and np.array_equal(s, sf)
    m = parts[0].size // W
    for j in range(W):
        qs, ss = zip(*[oracle.quant_i8(p) for p in parts])
        got = oracle.dequant_accum_i8([qq[j * m:(j + 1) * m] for qq in qs],
                                      [sv[j * m // 128:(j + 1) * m // 128] for sv in ss])
        assert np.array_equal(got, red[j * m:(j + 1) * m])


# ---------------------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------------------

def test_mx_worked_examples():
    for rec in goldens.read("mx_worked.txt"):
        x = goldens.padded_block(rec["x"], 32).reshape(1, 32)
        v, e = oracle.quant_mx(x)
        assert e[0, 0] == int(rec["byte"][0]), rec["name"]
        want = np.zeros(32, np.uint8)
        want[:len(rec["v"])] = [goldens.hexint(t) for t in rec["v"]]
        assert np.array_equal(v[0], want), rec["name"]


def test_mx_quant_bruteforce_rows():
    x = workloads.rows(4, 0, 0, 3, 256)        # gains spread the scales over many octaves
    v, e = oracle.quant_mx(x)
    for r in range(3):
        for g in range(8):
            grp = [bf.bf16_bits_to_fraction(int(h)) for h in x[r, g * 32:(g + 1) * 32]]
            byte = bf.e8m0_byte(max(abs(t) for t in grp))
            assert e[r, g] == byte
            sc = Fraction(2) ** (byte - 127)
            for i, t in enumerate(grp):
                neg0 = t == 0 and (x[r, g * 32 + i] & 0x8000) != 0
                assert v[r, g * 32 + i] == bf.e4m3_nearest(bf.rn32(t / sc), negative_zero=neg0)


def test_mx_never_saturates_and_bounds_error():
    x = workloads.tensor(4, 1, nrows=64)
    v, e = oracle.quant_mx(x)
    dec = torch.from_numpy(v.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    scale = 2.0 ** (e.astype(np.float64) - 127)
    xv = f32(x).astype(np.float64)
    recon = dec * np.repeat(scale, 32, axis=1)
    # E4M3 half-ulp bound: 2^-4 relative for normals, 2^-10 absolute (times scale) below
    err = np.abs(xv - recon)
    tol = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * np.repeat(scale, 32, axis=1))
    assert np.all(err <= tol)
    amax = np.abs(xv).reshape(64, -1, 32).max(2)
    assert np.all(amax / scale <= 448.0)               # the +inf-rounded scale leaves headroom
    assert not np.any((v & 0x7F) == 0x7F)              # no NaN codes


def test_mx_dequant_matches_torch_decode():
    x = workloads.tensor(4, 2, nrows=32)
    v, e = oracle.quant_mx(x)
    y = oracle.dequant_mx(v, e)
    dec = torch.from_numpy(v.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    sc = torch.from_numpy(np.repeat(e, 32, axis=1).astype(np.int32) - 127)
    want = torch.ldexp(dec, sc.to(torch.float32)).to(torch.bfloat16)
    assert np.array_equal(y, want.view(torch.int16).numpy().view(np.uint16))


def test_mx_slices_equal_concatenation_and_leave_the_rest_untouched():
    slices = [workloads.rows(4, j, 0, 8, 384) for j in range(3)]
    cat = np.concatenate(slices, axis=1)
    v_all, e_all = oracle.quant_mx(cat)
    cap, total = 12, 3 * 384
    v = np.full((cap, total), 0xA5, np.uint8)
    e = np.full((cap, total // 32), 0x5A, np.uint8)
    for j, sl in enumerate(slices):
        oracle.quant_mx_slice(sl, 384 * j, v, e)
    assert np.array_equal(v[:8], v_all) and np.array_equal(e[:8], e_all)
    assert np.all(v[8:] == 0xA5) and np.all(e[8:] == 0x5A)


# ---------------------------------------------------------------------------------------
# E4M3 128-block comparison codec
# ---------------------------------------------------------------------------------------

def test_mx_mfma_layout_worked_offsets():
    """Byte offsets of scales in the scaled-MFMA layout, worked by hand from the matrix
    instruction's scale operand (tests/golden/mx_mfma_layout.txt)."""
    cases = [rec["case"] for rec in goldens.read("mx_mfma_layout.txt")]
    cases = [list(map(int, c)) for c in cases]
    assert len(cases) == 14
    for row, group, rb, off in cases:
        assert oracle.mx_mfma_offset(row, group, rb) == off, (row, group, rb)


def test_mx_mfma_layout_is_lane_words_of_k_steps():
    """The layout read the way the GEMM reads it: in tile (512-column group q, row block p),
    the 32-bit word of lane l holds, in byte j, the scale of row 16p + l%16 and 32-column
    group 16q + 4j + l/16 -- the byte lane l supplies at K step j.  Distinct scale bytes
    per (row, group) make every placement visible; whole tiles are covered exactly once."""
    rows, groups, rb = 48, 48, 3
    e = np.zeros((rows, groups), np.uint8)
    ids = {}
    for r in range(rows):
        for g in range(groups):
            ids[(r, g)] = (r * groups + g) % 251
    # pairs with the same id sit far apart; compare through the id table
    for (r, g), v in ids.items():
        e[r, g] = v
    out = np.full(oracle.mx_mfma_bytes(rows, 32 * groups), 0xFF, np.uint8)
    assert out.size == 256 * 3 * 3
    oracle.mx_scales_to_mfma(e, out, rb)
    seen = 0
    for q in range(groups // 16):
        for p in range(rows // 16):
            tile = out[256 * (q * rb + p): 256 * (q * rb + p) + 256]
            for lane in range(64):
                for j in range(4):
                    r, g = 16 * p + lane % 16, 16 * q + 4 * j + lane // 16
                    assert tile[4 * lane + j] == ids[(r, g)], (q, p, lane, j)
                    seen += 1
    assert seen == rows * groups == out.size
    # and the read-back through the offset map is the input
    assert np.array_equal(oracle.mx_scales_from_mfma(out, rows, groups, rb), e)


def test_mx_slices_in_the_mfma_layout_equal_the_concatenation():
    """Six staged slices whose scales go to the MFMA layout equal the one-call quantization
    of the concatenation in that layout; positions no slice covers stay untouched, rows at
    or above the live rows too (slices at 128-column offsets that split 512-column groups)."""
    rows, cap, cols = 40, 48, 384
    xs = [workloads.rows(4, j, 0, rows, cols) for j in range(6)]
    total = 6 * cols
    v1 = np.full((cap, total), 0xEE, np.uint8)
    e1 = np.full(oracle.mx_mfma_bytes(cap, total), 0xEE, np.uint8)
    for j, x in enumerate(xs):
        oracle.quant_mx_slice_mfma(x, j * cols, v1, e1, cap)
    cat = np.concatenate(xs, axis=1)
    v2 = np.full((cap, total), 0xEE, np.uint8)
    e2 = np.full(oracle.mx_mfma_bytes(cap, total), 0xEE, np.uint8)
    oracle.quant_mx_slice_mfma(cat, 0, v2, e2, cap)
    assert np.array_equal(v1, v2) and np.array_equal(e1, e2)
    vr, er = oracle.quant_mx(cat)
    assert np.array_equal(v1[:rows], vr)
    assert np.array_equal(oracle.mx_scales_from_mfma(e1, rows, total // 32, 3), er)
    written = np.zeros(e1.size, bool)
    for r in range(rows):
        for g in range(total // 32):
            written[oracle.mx_mfma_offset(r, g, 3)] = True
    assert np.all(e1[~written] == 0xEE) and np.all(v1[rows:] == 0xEE)


def test_e4m3_b128_worked_examples():
    for rec in goldens.read("e4m3_b128_worked.txt"):
        x = goldens.padded_block(rec["x"], 128)
        v, s = oracle.quant_e4m3_b128(x)
        assert s.view(np.uint32)[0] == goldens.hexint(rec["scale"][0]), rec["name"]
        want = np.zeros(128, np.uint8)
        want[:len(rec["v"])] = [goldens.hexint(t) for t in rec["v"]]
        assert np.array_equal(v, want), rec["name"]


def test_e4m3_b128_bruteforce_and_dequant():
    x = workloads.rows(5, 0, 0, 1, 512)[0]
    v, s = oracle.quant_e4m3_b128(x)
    for b in range(4):
        xs = [bf.bf16_bits_to_fraction(int(h)) for h in x[b * 128:(b + 1) * 128]]
        amax = max(abs(t) for t in xs)
        if amax == 0:
            assert s[b] == 0 and not v[b * 128:(b + 1) * 128].any()
            continue
        sc = bf.rn32(amax / 448)
        assert Fraction(float(s[b])) == sc
        for i, t in enumerate(xs[:64]):
            neg0 = t == 0 and (x[b * 128 + i] & 0x8000) != 0
            assert v[b * 128 + i] == bf.e4m3_nearest(bf.rn32(t / sc), negative_zero=neg0)
    y = oracle.dequant_e4m3_b128(v, s)
    dec = torch.from_numpy(v.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    want = (dec * torch.from_numpy(np.repeat(s, 128))).to(torch.bfloat16)
    assert np.array_equal(y, want.view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------------------------------
# layout figures the pages print
# ---------------------------------------------------------------------------------------

def test_layout_figures_from_the_pages():
    kv = goldens.read_kv("layout.txt")
    n = 128 * 56
    x = workloads.rows(6, 0, 0, 1, n)[0]
    q, s = oracle.quant_i8(x)
    assert (q.nbytes + s.nbytes) // (n // 128) == int(kv["bytes_per_block_i8"])
    v, e = oracle.quant_mx(x.reshape(1, -1))
    assert (v.nbytes + e.nbytes) // (n // 128) == int(kv["bytes_per_128_mx"])
    assert x.nbytes // (n // 128) == int(kv["bytes_per_128_bf16"])
    cut = 100.0 * (1 - int(kv["bytes_per_block_i8"]) / int(kv["bytes_per_128_bf16"]))
    assert round(cut, 1) == float(kv["wire_reduction_percent_1dp"])


def test_a2a_reduce_is_accumulate_then_quantize_then_materialize():
    """The fused owner step is, by definition, A3 -> A1 -> A2 on each owner's shard;
    pinned against the separately pinned steps and against the all-to-all driver."""
    W = 4
    parts = [workloads.rows(3, r, 0, 8, 1024).reshape(-1) for r in range(W)]
    qs, ss = zip(*[oracle.quant_i8(p) for p in parts])
    q, s, ys, red = oracle.a2a_reduce_i8(list(qs), list(ss), W)
    m = parts[0].size // W
    for j in range(W):
        sm = oracle.dequant_accum_i8([qq[j * m:(j + 1) * m] for qq in qs],
                                     [sv[j * m // 128:(j + 1) * m // 128] for sv in ss])
        assert np.array_equal(red[j * m:(j + 1) * m], sm)
        wq, ws = oracle.quant_i8(sm)
        assert np.array_equal(q[j * m:(j + 1) * m], wq)
        assert np.array_equal(s[j * m // 128:(j + 1) * m // 128], ws)
        assert np.array_equal(ys[j], oracle.dequant_i8(wq, ws))
    dred, dq, ds, douts = oracle.a2a_allreduce_i8(parts)
    assert np.array_equal(dred, red) and np.array_equal(dq, q) and np.array_equal(ds, s)
    for j in range(W):
        assert np.array_equal(douts[j][j * m:(j + 1) * m], ys[j])


# ---------------------------------------------------------------------------------------
# MXFP8 on the collective topologies (flat layout: group g = values [32g, 32g+32))
# ---------------------------------------------------------------------------------------

def test_e8m0_quotient_underflow_saturates_to_the_smallest_byte():
    """For 0 < amax below 448 * 2^-150 the binary32 quotient amax/448 is 0; rounding toward
    +infinity with finite saturation then gives the smallest E8M0 value, byte 0.  Swept
    with the brute force over every binary32 octave at five significands each."""
    L = oracle.lib()
    for k in range(-149, 128):
        for sig in (1.0, 1.0 + 2.0 ** -23, 1.75, 1.75 + 2.0 ** -23, 2.0 - 2.0 ** -23):
            a = np.float32(sig * 2.0 ** k) if k > -127 else np.float32(2.0 ** k)
            if not np.isfinite(a) or a == 0:
                continue
            assert L.orc_e8m0_scale(float(a)) == bf.e8m0_byte(Fraction(float(a))), (k, sig)
    assert oracle.e8m0_scale(2.0 ** -149) == 0


def _mx_groups(v, e, g):
    return [int(c) for c in v[g * 32:(g + 1) * 32]], int(e[g])


def test_mx_ring_hop_bruteforce_and_identities():
    for trial in range(3):
        x = workloads.rows(6, trial, 0, 1, 256)[0]
        loc = workloads.rows(7, trial + 10, 0, 1, 256)[0]
        v, e = oracle.quant_mx_flat(x)
        v2, e2 = oracle.ring_hop_mx(v, e, loc)
        for g in range(8):
            codes, byte = _mx_groups(v, e, g)
            wb, wc = bf.mx_hop_group(codes, byte, [int(h) for h in loc[g * 32:(g + 1) * 32]])
            assert e2[g] == wb and list(v2[g * 32:(g + 1) * 32]) == wc, (trial, g)
    # local == +0: the hop re-encodes the payload's own values.  The byte may drop an
    # octave (a group whose largest code is below 256) but every value is unchanged.
    x = workloads.rows(1, 0, 0, 4, 1024).reshape(-1)
    v, e = oracle.quant_mx_flat(x)
    v2, e2 = oracle.ring_hop_mx(v, e, np.zeros_like(x))
    y, y2 = f32(oracle.dequant_mx_flat(v, e)), f32(oracle.dequant_mx_flat(v2, e2))
    assert np.array_equal(y.astype(np.float64), y2.astype(np.float64))
    assert np.all(e2 <= e) and np.any(e2 < e)
    # local == -(payload values), exact in bf16 here: every sum is +0, so every group is
    # the all-zero group (byte 127) with +0 codes.
    dq = torch.from_numpy(v.copy()).view(torch.float8_e4m3fn).double().numpy() * \
        2.0 ** (np.repeat(e, 32).astype(np.float64) - 127)
    yb = oracle.dequant_mx_flat(v, e)
    assert np.array_equal(f32(yb).astype(np.float64), dq)
    v3, e3 = oracle.ring_hop_mx(v, e, yb ^ np.uint16(0x8000))
    assert np.all(e3 == 127) and not v3.any()


def test_mx_hop_signed_zeros():
    """Only -0 + -0 is -0 under round-to-nearest; an E4M3 zero keeps that sign."""
    v = np.zeros(128, np.uint8)
    e = np.full(4, 127, np.uint8)
    loc = np.zeros(128, np.uint16)
    v[0], loc[0] = 0x80, 0x8000
    v[1], loc[1] = 0x80, 0x0000
    v[2], loc[2] = 0x00, 0x8000
    v2, e2 = oracle.ring_hop_mx(v, e, loc)
    assert list(v2[:3]) == [0x80, 0x00, 0x00] and e2[0] == 127


def test_mx_accum_order_and_bruteforce():
    """Sources are summed in array order: 448 - 448 + 2^-29 keeps the small term, while
    448 + 2^-29 - 448 loses it (absorbed below half an ulp of 448)."""
    n = 128
    v = [np.zeros(n, np.uint8) for _ in range(3)]
    e = [np.full(n // 32, 127, np.uint8) for _ in range(3)]
    v[0][0], v[1][0] = 0x7E, 0xFE                  # +448, -448 at scale 2^0
    v[2][0], e[2][0] = 0x38, 127 - 29               # E4M3 1.0 at scale 2^-29
    assert oracle.dequant_accum_mx(v, e)[0] == 0x3100                     # 2^-29
    assert oracle.dequant_accum_mx([v[0], v[2], v[1]], [e[0], e[2], e[1]])[0] == 0
    rng = np.random.default_rng(5)
    for W in (1, 2, 3, 5):
        xs = [workloads.rows(6, r, 0, 1, 256)[0] for r in range(W)]
        vs, es = zip(*[oracle.quant_mx_flat(x) for x in xs])
        got = oracle.dequant_accum_mx(list(vs), list(es))
        for i in rng.integers(0, 256, 48):
            want = bf.mx_accum_value([int(vv[i]) for vv in vs], [int(ee[i // 32]) for ee in es])
            assert got[i] == want, (W, i)


def test_mx_a2a_reduce_is_accumulate_then_quantize_then_materialize():
    W = 4
    parts = [workloads.rows(3, r, 0, 8, 1024).reshape(-1) for r in range(W)]
    vs, es = zip(*[oracle.quant_mx_flat(p) for p in parts])
    v, e, ys, red = oracle.a2a_reduce_mx(list(vs), list(es), W)
    m = parts[0].size // W
    for j in range(W):
        sm = oracle.dequant_accum_mx([vv[j * m:(j + 1) * m] for vv in vs],
                                     [ee[j * m // 32:(j + 1) * m // 32] for ee in es])
        assert np.array_equal(red[j * m:(j + 1) * m], sm)
        wv, we = oracle.quant_mx_flat(sm)
        assert np.array_equal(v[j * m:(j + 1) * m], wv)
        assert np.array_equal(e[j * m // 32:(j + 1) * m // 32], we)
        assert np.array_equal(ys[j], oracle.dequant_mx_flat(wv, we))
    dred, dv, de, douts = oracle.a2a_allreduce_mx(parts)
    assert np.array_equal(dred, red) and np.array_equal(dv, v) and np.array_equal(de, e)
    for j in range(W):
        assert np.array_equal(douts[j][j * m:(j + 1) * m], ys[j])


def _small_int_partials(W: int, n: int, seed: int):
    """Partials in {-2, ..., 2}: every partial sum s has |s| <= 2W <= 16 and at most 4
    significant bits, so every MXFP8 quantization of the ring and the all-to-all is exact
    (the group scale puts the amax in (224, 448], and E4M3 holds 4 significant bits)."""
    rng = np.random.default_rng(seed)
    return [rng.integers(-2, 3, n).astype(np.float64) for _ in range(W)]


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_mx_ring_allreduce_exact_sums_and_canonical_payload(W):
    parts = _small_int_partials(W, W * 256, W)
    exact = np.sum(parts, axis=0)
    vf, ef, outs = oracle.ring_allreduce_mx([_to_bf16_exact(p) for p in parts])
    assert np.array_equal(f32(outs[0]).astype(np.float64), exact)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.array_equal(outs[0], oracle.dequant_mx_flat(vf, ef))
    wv, we = oracle.quant_mx_flat(_to_bf16_exact(exact))    # exact sums requantized
    assert np.array_equal(vf, wv) and np.array_equal(ef, we)


def test_mx_ring_schedule():
    """W=2: chunk 0 is quantized by rank 1 and folded in by rank 0."""
    parts = [workloads.rows(2, r, 0, 2, 512).reshape(-1) for r in range(2)]
    h = parts[0].size // 2
    v1, e1 = oracle.quant_mx_flat(parts[1][:h])
    vh, eh = oracle.ring_hop_mx(v1, e1, parts[0][:h])
    vf, ef, outs = oracle.ring_allreduce_mx(parts)
    assert np.array_equal(vf[:h], vh) and np.array_equal(ef[:h // 32], eh)
    assert np.array_equal(outs[1][:h], oracle.dequant_mx_flat(vh, eh))


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_mx_a2a_allreduce_exact_sums(W):
    parts = _small_int_partials(W, W * 256, 10 + W)
    exact = np.sum(parts, axis=0)
    red, vf, ef, outs = oracle.a2a_allreduce_mx([_to_bf16_exact(p) for p in parts])
    assert np.array_equal(f32(red).astype(np.float64), exact)
    assert np.array_equal(f32(outs[0]).astype(np.float64), exact)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.array_equal(outs[0], oracle.dequant_mx_flat(vf, ef))


# ---------------------------------------------------------------------------------------
# MXFP8 of binary16 slices (the staged quantizer takes BF16 or FP16 slices)
# ---------------------------------------------------------------------------------------

def all_finite_f16() -> np.ndarray:
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return h[((h >> 10) & 0x1F) != 0x1F]


def test_f16_decode_exhaustive_matches_numpy():
    h = all_finite_f16()
    L = oracle.lib()
    got = np.fromiter((L.orc_f16_to_f32(int(v)) for v in h), dtype=np.float32, count=h.size)
    want = h.view(np.float16).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))     # signed zeros too
    for v in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF):
        assert Fraction(float(L.orc_f16_to_f32(v))) == bf.f16_bits_to_fraction(v)


def test_e8m0_over_every_f16_amax():
    """Smallest power of two >= fl32(amax/448) over every positive finite binary16 amax;
    for amax = m 2^k it is k - 8 + [m > 1.75] (no clamping is reached from binary16)."""
    h = all_finite_f16()
    h = h[(h > 0) & (h < 0x8000)]
    amax = h.view(np.float16).astype(np.float32)
    d = (amax / np.float32(448.0)).astype(np.float64)
    e = np.full(d.shape, 200, np.int64)
    for k in range(127, -128, -1):
        e = np.where(2.0 ** k >= d, k, e)
    L = oracle.lib()
    got = np.fromiter((L.orc_e8m0_scale(float(a)) for a in amax), dtype=np.uint8, count=amax.size)
    assert np.array_equal(got.astype(np.int64) - 127, e)
    m, k = np.frexp(amax.astype(np.float64))
    assert np.array_equal(e, (k - 1) - 8 + (m * 2 > 1.75))


def test_mx_f16_quant_bruteforce_rows():
    x = workloads.rows(4, 0, 0, 3, 256, fmt="f16")   # per-row gains: subnormals to hundreds
    v, e = oracle.quant_mx_f16(x)
    for r in range(3):
        for g in range(8):
            grp = [bf.f16_bits_to_fraction(int(h)) for h in x[r, g * 32:(g + 1) * 32]]
            byte = bf.e8m0_byte(max(abs(t) for t in grp))
            assert e[r, g] == byte
            sc = Fraction(2) ** (byte - 127)
            for i, t in enumerate(grp):
                neg0 = t == 0 and (x[r, g * 32 + i] & 0x8000) != 0
                assert v[r, g * 32 + i] == bf.e4m3_nearest(bf.rn32(t / sc), negative_zero=neg0)


def test_mx_f16_equals_bf16_on_values_both_formats_hold():
    """A value with at most 8 significant bits in the binary16 normal range is the same
    number in bf16; the MXFP8 quantization of the two encodings must agree."""
    rng = np.random.default_rng(8)
    sig = rng.integers(128, 256, (16, 512)).astype(np.float64)          # 8-bit significands
    ex = rng.integers(-14 - 7, 15 - 7 + 1, (16, 512))
    vals = sig * 2.0 ** ex * np.where(rng.random((16, 512)) < 0.5, -1, 1)
    vals[:, ::37] = 0.0
    h16 = vals.astype(np.float16)
    assert np.array_equal(h16.astype(np.float64), vals)
    b = vals.astype(np.float32).view(np.uint32)
    assert not np.any(b & 0xFFFF)
    v16, e16 = oracle.quant_mx_f16(h16.view(np.uint16))
    vbf, ebf = oracle.quant_mx((b >> 16).astype(np.uint16))
    assert np.array_equal(v16, vbf) and np.array_equal(e16, ebf)


def test_mx_f16_slices_equal_concatenation_and_leave_the_rest_untouched():
    R, C, S = 8, 256, 3
    xs = [workloads.rows(4, j, 0, R, C, fmt="f16") for j in range(S)]
    cat = np.concatenate(xs, axis=1)
    wv, we = oracle.quant_mx_f16(cat)
    cap = R + 3
    v = np.full((cap, S * C), 0xA5, np.uint8)
    e = np.full((cap, S * C // 32), 0x5A, np.uint8)
    for j in (2, 0, 1):
        oracle.quant_mx_slice_f16(xs[j], j * C, v, e)
    assert np.array_equal(v[:R], wv) and np.array_equal(e[:R], we)
    assert np.all(v[R:] == 0xA5) and np.all(e[R:] == 0x5A)


# ---------------------------------------------------------------------------------------
# the MXFP8 GEMM from staged inputs (the plain definition: Y = X W^T on exact values)
# ---------------------------------------------------------------------------------------

def test_mm_mx_worked_cases():
    """All-ones codes: each output is the sum over groups of 32 * 2^(ex + ew - 254)."""
    M, N, K = 3, 5, 256
    xv = np.full((M, K), 0x38, np.uint8)
    wv = np.full((N, K), 0x38, np.uint8)
    xe = np.full((M, K // 32), 127, np.uint8)
    we = np.full((N, K // 32), 127, np.uint8)
    xe[1, 2], we[4, 2], xe[2, 7] = 130, 120, 0
    Y, S = oracle.mm_mx(xv, xe, wv, we)
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            want[m, n] = sum(32 * 2.0 ** (int(xe[m, g]) + int(we[n, g]) - 254) for g in range(K // 32))
    assert np.array_equal(Y, want) and np.array_equal(S, want)
    xv[0, :] = 0xB8                                                  # -1.0
    Y, S = oracle.mm_mx(xv, xe, wv, we)
    assert np.array_equal(Y[0], -want[0]) and np.array_equal(S[0], want[0])


def test_mm_mx_bruteforce_tiny():
    x = workloads.rows(4, 0, 0, 3, 128)
    w = workloads.rows(7, 1, 0, 2, 128)
    xv, xe = oracle.quant_mx(x)
    wv, we = oracle.quant_mx(w)
    Y, S = oracle.mm_mx(xv, xe, wv, we)
    for m in range(3):
        for n in range(2):
            acc = Fraction(0)
            acs = Fraction(0)
            for k in range(128):
                a = bf.e4m3_value(int(xv[m, k])) * Fraction(2) ** (int(xe[m, k // 32]) - 127)
                b = bf.e4m3_value(int(wv[n, k])) * Fraction(2) ** (int(we[n, k // 32]) - 127)
                acc += a * b
                acs += abs(a * b)
            assert Fraction(Y[m, n]) == acc and Fraction(S[m, n]) == acs


def test_mm_mx_matches_the_pinned_dequantize():
    """Where the bf16 materialization is exact (no value below 2^-133), the GEMM of the
    materialized operands is the same number."""
    x = workloads.rows(6, 2, 0, 8, 512)
    w = workloads.rows(7, 3, 0, 6, 512)
    xv, xe = oracle.quant_mx(x)
    wv, we = oracle.quant_mx(w)
    Y, _ = oracle.mm_mx(xv, xe, wv, we)
    xd = f32(oracle.dequant_mx(xv, xe)).astype(np.float64)
    wd = f32(oracle.dequant_mx(wv, we)).astype(np.float64)
    assert np.array_equal(oracle.mx_values_f64(xv, xe), xd)
    assert np.allclose(Y, xd @ wd.T, rtol=0, atol=1e-12 * np.abs(xd).sum())
