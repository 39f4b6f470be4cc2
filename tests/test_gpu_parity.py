"""GPU parity: every HIP entry point against the CPU oracle, element by element.

Bar (from the codec definitions): INT8 / E4M3 payloads, FP32 and E8M0 scales and every
bf16 output are compared bit for bit -- including the binary32-accumulated A2A sums and
the ring-hop materializations, whose operation order is fixed on both sides.  Inputs
come from the seeded generators in ``workloads`` (never from the GPU path); expected
values come only from ``oracle``.

Sizes: small cases span several tiles and a ragged tail and are compared in full; the
configs at full size are compared in full where the oracle takes seconds, else on
sampled rows (every codec step is local to a 128-value block, so a row's result depends
on that row of each input only), plus properties that hold at any size.
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

COLS = 7168


def f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---- helpers: run one codec on the GPU, return host arrays ------------------------------

def gpu_quant_i8(x: np.ndarray):
    n = x.size
    xd = to_dev(x.reshape(-1))
    q, s = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_quant_i8(xd, q, s, n=n)
    sync()
    return host(q, np.int8), host(s, np.float32)


def gpu_dequant_i8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    n = q.size
    y = empty(n, np.uint16)
    bq.bq_dequant_i8(to_dev(q), to_dev(s), y, n=n)
    sync()
    return host(y, np.uint16)


def assert_same(got, want, what):
    got, want = np.asarray(got).reshape(-1), np.asarray(want).reshape(-1)
    assert got.shape == want.shape, what
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"got {got[bad[:5]]} want {want[bad[:5]]}"


# ---- block INT8: quantize / materialize -------------------------------------------------

def test_i8_roundtrip_cfg1():
    say("i8 roundtrip cfg1 512x7168")
    x = workloads.tensor(1, 0)
    q, s = gpu_quant_i8(x)
    wq, ws = oracle.quant_i8(x)
    assert_same(q, wq, "payload")
    assert_same(s, ws, "scales")
    y = gpu_dequant_i8(q, s)
    assert_same(y, oracle.dequant_i8(wq, ws), "materialized bf16")
    xf = f32(x).astype(np.float64).reshape(-1, 128)
    err = np.abs(xf - q.astype(np.float64).reshape(-1, 128) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16))


@pytest.mark.parametrize("blocks", [1, 3, 4, 15, 17, 63, 64, 65, 255, 257, 1031])
def test_i8_ragged_sizes(blocks):
    say(f"i8 ragged blocks={blocks}")
    x = workloads.rows(6, blocks, 0, 1, 128 * blocks)[0]
    q, s = gpu_quant_i8(x)
    wq, ws = oracle.quant_i8(x)
    assert_same(q, wq, "payload")
    assert_same(s, ws, "scales")
    assert_same(gpu_dequant_i8(q, s), oracle.dequant_i8(wq, ws), "bf16")


def test_empty_inputs_launch_nothing():
    say("empty inputs")
    z = torch.empty(0, device="cuda")
    bq.bq_quant_i8(z, z, z, n=0)
    bq.bq_dequant_i8(z, z, z, n=0)
    bq.bq_ring_hop_i8(z, z, z, z, z, n=0)
    bq.bq_quant_e4m3_b128(z, z, z, n=0)
    sync()


def _every_amax_blocks(rng, lo_frac=-1.0):
    """One block per positive finite bf16 amax, alternating its sign; the other 127 values
    are bf16 values drawn uniformly in [-amax, amax] (truncated toward zero)."""
    h = np.arange(1, 0x7F80, dtype=np.uint32)            # positive finite bf16
    amax = (h << 16).view(np.float32)
    u = rng.uniform(lo_frac, 1.0, (h.size, 127)).astype(np.float32)
    vals = (u * amax[:, None]).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)   # truncation keeps |x| <= amax
    first = h.astype(np.uint16) | np.where(np.arange(h.size) % 2 == 1, 0x8000, 0).astype(np.uint16)
    blocks = np.concatenate([first[:, None], bits], axis=1)
    perm = rng.permuted(np.tile(np.arange(128), (h.size, 1)), axis=1)
    return np.take_along_axis(blocks, perm, axis=1).reshape(-1)


def test_i8_every_bf16_amax():
    say("i8 every bf16 amax")
    x = _every_amax_blocks(np.random.default_rng(1))
    q, s = gpu_quant_i8(x)
    wq, ws = oracle.quant_i8(x)
    assert_same(s, ws, "scales over every bf16 amax")
    assert_same(q, wq, "payload over every bf16 amax")
    assert_same(gpu_dequant_i8(q, s), oracle.dequant_i8(wq, ws), "bf16")


def test_i8_exact_ties_take_the_exact_path():
    """amax = 127 * 2^k gives a power-of-two scale; half-integer multiples of it are exact
    ties, which the kernel must round half-to-even exactly like the oracle."""
    say("i8 exact ties")
    rng = np.random.default_rng(2)
    nb = 4096
    k = rng.integers(-20, 20, nb)
    scale = np.ldexp(1.0, k)
    vals = rng.integers(-254, 255, (nb, 128)) / 2.0 * scale[:, None]
    vals[:, 0] = 127 * scale * np.where(rng.random(nb) < 0.5, 1, -1)
    x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).reshape(-1)
    assert np.array_equal(f32(x).astype(np.float64), vals.reshape(-1))
    q, s = gpu_quant_i8(x)
    wq, ws = oracle.quant_i8(x)
    assert_same(s, ws, "scales")
    assert_same(q, wq, "payload")


def test_i8_metric_shape_3072x7168():
    say("i8 quant+dequant 3072x7168 (cfg2 rank0)")
    x = workloads.tensor(2, 0)
    q, s = gpu_quant_i8(x)
    wq, ws = oracle.quant_i8(x)
    assert_same(q, wq, "payload")
    assert_same(s, ws, "scales")
    assert_same(gpu_dequant_i8(q, s), oracle.dequant_i8(wq, ws), "bf16")


def test_dequant_bf16_rounding_sweep():
    """With q = 1 the materialization is bf16_rne(scale): every bf16 upper half with the
    lower halves that decide rounding (exact, tie, both sides of the tie)."""
    say("dequant bf16 rounding sweep")
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    hi = np.arange(0x7F7F, dtype=np.uint32)       # positive, finite, rounding stays finite
    sc = ((hi[:, None] << 16) | lows[None, :]).reshape(-1).view(np.float32)
    sc = np.concatenate([sc, -sc]).astype(np.float32)
    q = np.ones(sc.size * 128, np.int8)
    q[1::128] = -1
    y = gpu_dequant_i8(q, sc)
    assert_same(y, oracle.dequant_i8(q, sc), "bf16 rounding of q*scale")


# ---- ring hop and the ring all-reduce ----------------------------------------------------

def test_ring_hop_matches_oracle_and_in_place():
    say("ring hop 768x7168, out of place and in place")
    x = workloads.rows(2, 1, 0, 768, COLS).reshape(-1)
    loc = workloads.rows(2, 2, 0, 768, COLS).reshape(-1)
    wq, ws = oracle.quant_i8(x)
    hq, hs = oracle.ring_hop_i8(wq, ws, loc)
    n = x.size
    qi, si, ld = to_dev(wq), to_dev(ws), to_dev(loc)
    qo, so = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_ring_hop_i8(qi, si, ld, qo, so, n=n)
    sync()
    assert_same(host(qo, np.int8), hq, "hop payload")
    assert_same(host(so, np.float32), hs, "hop scales")
    bq.bq_ring_hop_i8(qi, si, ld, qi, si, n=n)           # exact in-place form
    sync()
    assert_same(host(qi, np.int8), hq, "in-place hop payload")
    assert_same(host(si, np.float32), hs, "in-place hop scales")


def test_ring_hop_scale_underflow_zero_block():
    say("ring hop scale underflow")
    q = np.zeros(256, np.int8)
    q[7] = 1
    q[200] = -3
    s = np.array([2.0 ** -149, 1.0], np.float32)
    loc = np.zeros(256, np.uint16)
    wq, ws = oracle.ring_hop_i8(q, s, loc)
    qo, so = empty(256, np.int8), empty(2, np.float32)
    bq.bq_ring_hop_i8(to_dev(q), to_dev(s), to_dev(loc), qo, so, n=256)
    sync()
    assert_same(host(qo, np.int8), wq, "payload")
    assert_same(host(so, np.float32), ws, "scales")
    assert ws[0] == 0


def test_ring_hop_clamps_few_bit_subnormal_scales():
    """Hop blocks whose binary32 sums have amax A * 2^-149 for every A in 1..2^20: the scale
    fl32(amax/127) is subnormal with few significant bits, the quotient can exceed 127.5
    (A = 190: scale 2^-149, quotient 190) and the [-127, 127] clamp decides the byte.
    Payload [1, -1, 0, ...] with input scale A * 2^-149 and a zero local partial; out of
    place and in place, bit for bit."""
    say("ring hop clamp: amax A*2^-149, A = 1..2^20")
    A = np.arange(1, 2 ** 20 + 1, dtype=np.float64)
    nb = A.size
    n = nb * 128
    q = np.zeros((nb, 128), np.int8)
    q[:, 0], q[:, 1] = 1, -1
    q = q.reshape(-1)
    s = (A * 2.0 ** -149).astype(np.float32)
    assert np.array_equal(s.astype(np.float64) * 2.0 ** 149, A)
    loc = np.zeros(n, np.uint16)
    wq, ws = oracle.ring_hop_i8(q, s, loc)
    # the clamp binds on thousands of these blocks
    nz = ws > 0
    assert np.count_nonzero(s[nz].astype(np.float64) / ws[nz] > 127.5) > 3900
    qi, si, ld = to_dev(q), to_dev(s), to_dev(loc)
    qo, so = empty(n, np.int8), empty(nb, np.float32)
    bq.bq_ring_hop_i8(qi, si, ld, qo, so, n=n)
    sync()
    assert_same(host(qo, np.int8), wq, "hop payload")
    assert_same(host(so, np.float32), ws, "hop scales")
    bq.bq_ring_hop_i8(qi, si, ld, qi, si, n=n)
    sync()
    assert_same(host(qi, np.int8), wq, "in-place hop payload")
    assert_same(host(si, np.float32), ws, "in-place hop scales")


def _cancelling_ring_partials(W: int, blocks: int, seed: int):
    """Partials of a W-rank ring whose hop sums nearly cancel near 2^-126.  The rank that
    quantizes chunk c at step 0 holds, per block, a pilot (128 + j) * 2^-133 (a bf16 normal
    just above 2^-126) and values k * 2^-133 with |k| <= K; the next rank holds minus the
    bf16 materialization of that payload (from the oracle), every later rank zeros.  The
    first hop's binary32 sums are then the few-bit residues of the scale's rounding."""
    rng = np.random.default_rng(seed)
    m = blocks * 128
    n = W * m
    parts = [np.zeros(n, np.uint16) for _ in range(W)]
    for c in range(W):
        K = np.where(rng.random(blocks) < 0.5, rng.integers(1, 8, blocks),
                     rng.integers(1, 64, blocks))
        k = rng.integers(-63, 64, (blocks, 128))
        k = np.clip(k, -K[:, None], K[:, None])
        k[:, 1], k[:, 2] = K, -K
        mag = np.abs(k).astype(np.uint32)
        bits = np.where(k < 0, 0x8000, 0).astype(np.uint32) | mag   # k * 2^-133: bf16 subnormal
        pilot = (128 + rng.integers(0, 128, blocks)).astype(np.uint32)   # (128+j) * 2^-133
        bits[:, 0] = (1 << 7) | (pilot - 128)                           # exponent field 1
        quant_side = bits.astype(np.uint16).reshape(-1)
        qq, ss = oracle.quant_i8(quant_side)
        hop_side = oracle.dequant_i8(qq, ss) ^ np.uint16(0x8000)
        parts[(c + 1) % W][c * m:(c + 1) * m] = quant_side
        parts[(c + 2) % W][c * m:(c + 1) * m] = hop_side
    return parts


@pytest.mark.parametrize("W", [2, 4])
def test_ring_allreduce_cancelling_partials(W):
    """The clamp reached through the public ring driver: partials that cancel to few-bit
    binary32 residues at the first hop, compared bit for bit with the oracle (final
    payload, scales, every rank's output)."""
    say(f"ring allreduce W={W}, cancelling partials near 2^-126")
    blocks = 4096
    parts = _cancelling_ring_partials(W, blocks, 40 + W)
    # the first hop of chunk 0 reaches the clamp on many blocks
    m = blocks * 128
    q1, s1 = oracle.quant_i8(parts[1 % W][:m])
    sums = (q1.astype(np.float64).reshape(-1, 128) * s1.astype(np.float64)[:, None]
            + f32(parts[2 % W][:m]).astype(np.float64).reshape(-1, 128))
    _, s2 = oracle.ring_hop_i8(q1, s1, parts[2 % W][:m])
    nz = s2 > 0
    assert np.count_nonzero(np.abs(sums).max(1)[nz] / s2[nz] > 127.5) > 100
    wq, ws, wouts = oracle.ring_allreduce_i8(parts)
    _, qw, sw, outs = gpu_ring(parts)
    assert_same(host(qw, np.int8), wq, "final payloads")
    assert_same(host(sw, np.float32), ws, "final scales")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


def gpu_ring(partials: list[np.ndarray]):
    W, n = len(partials), partials[0].size
    pd = [to_dev(p.reshape(-1)) for p in partials]
    qw, sw = empty(n, np.int8), empty(n // 128, np.float32)
    outs = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_ring_allreduce_i8(pd, qw, sw, outs, n=n)
    sync()
    return pd, qw, sw, outs


@pytest.mark.parametrize("W,rows", [(1, 4), (2, 6), (3, 9), (4, 12), (8, 16)])
def test_ring_allreduce_small(W, rows):
    say(f"ring allreduce W={W} rows={rows}")
    parts = [workloads.rows(2, r, 0, rows, 1024).reshape(-1) for r in range(W)]
    wq, ws, wouts = oracle.ring_allreduce_i8(parts)
    _, qw, sw, outs = gpu_ring(parts)
    assert_same(host(qw, np.int8), wq, "final payloads")
    assert_same(host(sw, np.float32), ws, "final scales")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


def test_ring_allreduce_cfg2_full():
    """The metric workload: 4 simulated ranks x 3072x7168, compared in full."""
    say("ring allreduce cfg2 4x3072x7168 (full compare)")
    parts = [workloads.tensor(2, r).reshape(-1) for r in range(4)]
    wq, ws, wouts = oracle.ring_allreduce_i8(parts)
    _, qw, sw, outs = gpu_ring(parts)
    assert_same(host(qw, np.int8), wq, "final payloads")
    assert_same(host(sw, np.float32), ws, "final scales")
    for r in range(4):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


def test_ring_allreduce_cfg5_prefill_full():
    """Prefill size: 4 ranks x 16384x7168 (t3, zero blocks, spikes): the final payloads and
    scales and every rank's output against the oracle in full (the oracle takes about ten
    seconds), and every rank's output bit-identical on the GPU."""
    W = 4
    say("ring allreduce cfg5 4x16384x7168 (full compare)")
    parts = [workloads.tensor(5, r).reshape(-1) for r in range(W)]
    pd, qw, sw, outs = gpu_ring(parts)
    for r in range(1, W):
        assert torch.equal(outs[r], outs[0]), f"rank {r} differs from rank 0"
    wq, ws, wouts = oracle.ring_allreduce_i8(parts)
    assert_same(host(qw, np.int8), wq, "final payloads")
    assert_same(host(sw, np.float32), ws, "final scales")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


# ---- A2A: multi-source accumulate and the all-to-all reduce -------------------------------

@pytest.mark.parametrize("nsrc", [1, 2, 3, 8, 9, 16, 64])
def test_accum_sources(nsrc):
    say(f"accumulate nsrc={nsrc}")
    n = 128 * 77
    xs = [workloads.rows(7, s, 0, 1, n)[0] for s in range(nsrc)]
    qs, ss = zip(*[oracle.quant_i8(x) for x in xs])
    want = oracle.dequant_accum_i8(list(qs), list(ss))
    qd, sd = [to_dev(q) for q in qs], [to_dev(s) for s in ss]
    y = empty(n, np.uint16)
    bq.bq_dequant_accum_i8(qd, sd, y, n=n)
    sync()
    assert_same(host(y, np.uint16), want, "accumulated bf16")


def gpu_a2a(partials):
    W, n = len(partials), partials[0].size
    pd = [to_dev(p.reshape(-1)) for p in partials]
    qs = [empty(n, np.int8) for _ in range(W)]
    ss = [empty(n // 128, np.float32) for _ in range(W)]
    red, qb, sb = empty(n, np.uint16), empty(n, np.int8), empty(n // 128, np.float32)
    outs = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_a2a_allreduce_i8(pd, qs, ss, red, qb, sb, outs, n=n)
    sync()
    return red, qb, sb, outs


def test_a2a_cfg3_w4_full():
    say("a2a cfg3 W=4 4x3072x7168 (full compare)")
    parts = [workloads.tensor(3, r).reshape(-1) for r in range(4)]
    wred, wq, ws, wouts = oracle.a2a_allreduce_i8(parts)
    red, qb, sb, outs = gpu_a2a(parts)
    assert_same(host(red, np.uint16), wred, "owner bf16 sums")
    assert_same(host(qb, np.int8), wq, "broadcast payload")
    assert_same(host(sb, np.float32), ws, "broadcast scales")
    for r in range(4):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


def test_a2a_cfg3_w16_full():
    W = 16
    say("a2a cfg3 W=16 16x3072x7168 (full compare; the oracle takes about half a minute)")
    parts = [workloads.tensor(3, r).reshape(-1) for r in range(W)]
    red, qb, sb, outs = gpu_a2a(parts)
    for r in range(1, W):
        assert torch.equal(outs[r], outs[0]), f"rank {r} differs from rank 0"
    wred, wq, ws, wouts = oracle.a2a_allreduce_i8(parts)
    assert_same(host(red, np.uint16), wred, "owner bf16 sums")
    assert_same(host(qb, np.int8), wq, "broadcast payload")
    assert_same(host(sb, np.float32), ws, "broadcast scales")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


@pytest.mark.parametrize("nseg,nsrc,rows", [(4, 4, 48), (2, 3, 6), (16, 16, 32), (1, 1, 3)])
def test_a2a_reduce_fused_matches_oracle(nseg, nsrc, rows):
    say(f"fused a2a owner step nseg={nseg} nsrc={nsrc} rows={rows}")
    parts = [workloads.rows(3, r, 0, rows, 1024).reshape(-1) for r in range(nsrc)]
    qs, ss = zip(*[oracle.quant_i8(p) for p in parts])
    wq, ws, wys, wred = oracle.a2a_reduce_i8(list(qs), list(ss), nseg)
    n = parts[0].size
    m = n // nseg
    qd, sd = [to_dev(q) for q in qs], [to_dev(v) for v in ss]
    qo, so, red = empty(n, np.int8), empty(n // 128, np.float32), empty(n, np.uint16)
    ys = [empty(m, np.uint16) for _ in range(nseg)]
    bq.bq_a2a_reduce_i8(nseg, qd, sd, qo, so, ys, red)
    qo2, so2 = empty(n, np.int8), empty(n // 128, np.float32)
    bq.bq_a2a_reduce_i8(nseg, qd, sd, qo2, so2)          # payload only
    sync()
    assert_same(host(qo, np.int8), wq, "payload")
    assert_same(host(so, np.float32), ws, "scales")
    assert_same(host(red, np.uint16), wred, "bf16 sums")
    for j in range(nseg):
        assert_same(host(ys[j], np.uint16), wys[j], f"owner {j} materialization")
    assert_same(host(qo2, np.int8), wq, "payload without optional outputs")
    assert_same(host(so2, np.float32), ws, "scales without optional outputs")


def test_allgather_dequant_skip_own_leaves_the_owner_shard():
    say("all-gather materialization with and without skip_own")
    W, rows = 4, 16
    x = workloads.rows(6, 0, 0, rows, COLS).reshape(-1)
    q, s = oracle.quant_i8(x)
    want = oracle.dequant_i8(q, s)
    n, m = x.size, x.size // W
    qd, sd = to_dev(q), to_dev(s)
    outs = [filled(n, np.uint16, 0x7B) for _ in range(W)]
    bq.bq_allgather_dequant_i8(qd, sd, outs, skip_own=True)
    full = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_allgather_dequant_i8(qd, sd, full)
    sync()
    for r in range(W):
        got = host(outs[r], np.uint16)
        own = np.zeros(n, bool)
        own[r * m:(r + 1) * m] = True
        assert np.all(got[own] == 0x7B7B), f"rank {r} own shard was written"
        assert_same(got[~own], want[~own], f"rank {r} other shards")
        assert_same(host(full[r], np.uint16), want, f"rank {r} full")


def test_a2a_driver_without_red():
    say("a2a driver, red = NULL")
    W = 4
    parts = [workloads.rows(3, r, 0, 96, COLS).reshape(-1) for r in range(W)]
    wred, wq, ws, wouts = oracle.a2a_allreduce_i8(parts)
    n = parts[0].size
    pd = [to_dev(p) for p in parts]
    qs = [empty(n, np.int8) for _ in range(W)]
    ss = [empty(n // 128, np.float32) for _ in range(W)]
    qb, sb = empty(n, np.int8), empty(n // 128, np.float32)
    outs = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_a2a_allreduce_i8(pd, qs, ss, None, qb, sb, outs, n=n)
    sync()
    assert_same(host(qb, np.int8), wq, "payload")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


# ---- MXFP8 ---------------------------------------------------------------------------------

def gpu_quant_mx(x: np.ndarray, ldv_pad: int = 0, lds_pad: int = 0):
    rows, cols = x.shape
    v = empty((rows, cols + ldv_pad), np.uint8)
    e = empty((rows, cols // 32 + lds_pad), np.uint8)
    bq.bq_quant_mx(to_dev(x), v, e, rows=rows, cols=cols)
    sync()
    return host(v, np.uint8)[:, :cols], host(e, np.uint8)[:, :cols // 32]


@pytest.mark.parametrize("rows,cols,pad", [(1, 128, 0), (3, 384, 16), (7, 640, 0), (33, 1152, 32),
                                           (64, 7168, 0)])
def test_mx_small_shapes(rows, cols, pad):
    say(f"mx quant/dequant {rows}x{cols} pad={pad}")
    x = workloads.rows(4, 9, 0, rows, cols)
    v, e = gpu_quant_mx(x, ldv_pad=pad, lds_pad=4 if pad else 0)
    wv, we = oracle.quant_mx(x)
    assert_same(e, we, "E8M0 scales")
    assert_same(v, wv, "E4M3 values")
    y = empty((rows, cols + pad), np.uint16)
    bq.bq_dequant_mx(to_dev(wv), to_dev(we), y, rows=rows, cols=cols, ldv=cols, lds=cols // 32)
    sync()
    assert_same(host(y, np.uint16)[:, :cols], oracle.dequant_mx(wv, we), "bf16")


def test_mx_every_bf16_amax_and_every_value():
    """Groups with every positive bf16 amax (the E8M0 rule over its whole domain) and
    groups with amax 448 holding every bf16 value up to 448 (the E4M3 encoder)."""
    say("mx every amax / every value")
    rng = np.random.default_rng(4)
    h = np.arange(1, 0x7F80, dtype=np.uint32)
    amax_bits = (h << 16).view(np.float32)
    u = rng.uniform(-1, 1, (h.size, 31)).astype(np.float32)
    other = ((u * amax_bits[:, None]).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    groups = np.concatenate([h.astype(np.uint16)[:, None], other], axis=1)
    # every bf16 value with |x| <= 448, 31 per group next to a 448 pilot
    allv = np.arange(65536, dtype=np.uint32)
    mag = (allv & 0x7FFF) << 16
    allv = allv[mag.view(np.float32) <= 448.0].astype(np.uint16)
    pad = (-allv.size) % 31
    allv = np.concatenate([allv, np.zeros(pad, np.uint16)]).reshape(-1, 31)
    pilot = np.full((allv.shape[0], 1), 0x43E0, np.uint16)          # 448
    groups = np.concatenate([groups, np.concatenate([pilot, allv], axis=1)])
    pad_g = (-groups.shape[0]) % 4
    groups = np.concatenate([groups, np.zeros((pad_g, 32), np.uint16)])
    x = groups.reshape(-1, 128)
    v, e = gpu_quant_mx(x)
    wv, we = oracle.quant_mx(x)
    assert_same(e, we, "E8M0 over every bf16 amax")
    assert_same(v, wv, "E4M3 values")
    y = empty(x.shape, np.uint16)
    bq.bq_dequant_mx(to_dev(wv), to_dev(we), y)
    sync()
    assert_same(host(y, np.uint16), oracle.dequant_mx(wv, we), "bf16")


def test_mx_dequant_every_code_and_scale():
    """Dequantize every E4M3 code under every E8M0 byte 0..254 (subnormal products too)."""
    say("mx dequant every code x byte")
    codes = np.arange(256, dtype=np.uint8)
    codes = np.concatenate([codes[(codes & 0x7F) != 0x7F], np.zeros(2, np.uint8)])
    v = np.tile(codes, (255, 1))                               # 255 rows of all 254 codes
    e = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 8, axis=1)
    y = empty(v.shape, np.uint16)
    bq.bq_dequant_mx(to_dev(v), to_dev(e), y)
    sync()
    assert_same(host(y, np.uint16), oracle.dequant_mx(v, e), "bf16")


def test_mx_staged_slices_cfg4():
    """Six 4096x7168 slices at 128-aligned offsets of a 4096x43008 staging buffer: equal
    bit for bit to the one-call quantization of the concatenation and, in full, to the
    oracle's (about ten seconds of oracle work); a 4608-row capacity keeps rows 4096..
    untouched; the dequantize of the whole buffer against the oracle."""
    R, K, J = 4096, 7168, 6
    say("mx staged slices cfg4 6x4096x7168 -> 4096x43008")
    slices = [workloads.tensor(4, j) for j in range(J)]
    sd = [to_dev(s) for s in slices]
    cap = 4608
    v = filled((cap, K * J), np.uint8, 0xA5)
    e = filled((cap, K * J // 32), np.uint8, 0x5A)
    for j in range(J):
        bq.bq_quant_mx_slice(sd[j], K * j, v, e, capacity_rows=cap)
    cat = torch.cat(sd, dim=1)
    v1, e1 = empty((R, K * J), np.uint8), empty((R, K * J // 32), np.uint8)
    bq.bq_quant_mx(cat, v1, e1)
    sync()
    assert torch.equal(v[:R], v1) and torch.equal(e[:R], e1), "staged != concatenated"
    assert bool((v[R:] == 0xA5).all()) and bool((e[R:] == 0x5A).all()), "rows past live touched"
    wv, we = oracle.quant_mx(np.concatenate(slices, axis=1))
    assert_same(host(v, np.uint8)[:R], wv, "E4M3 values")
    assert_same(host(e, np.uint8)[:R], we, "E8M0 scales")
    y = empty((R, K * J), np.uint16)
    bq.bq_dequant_mx(v1, e1, y)
    sync()
    assert_same(host(y, np.uint16), oracle.dequant_mx(wv, we), "bf16")


# ---- E4M3 128-block codec --------------------------------------------------------------------

def gpu_e4m3(x: np.ndarray):
    n = x.size
    v, s = empty(n, np.uint8), empty(n // 128, np.float32)
    bq.bq_quant_e4m3_b128(to_dev(x.reshape(-1)), v, s, n=n)
    y = empty(n, np.uint16)
    bq.bq_dequant_e4m3_b128(v, s, y, n=n)
    sync()
    return host(v, np.uint8), host(s, np.float32), host(y, np.uint16)


def test_e4m3_b128_every_amax_and_ragged():
    say("e4m3 b128 every amax")
    x = _every_amax_blocks(np.random.default_rng(6))
    v, s, y = gpu_e4m3(x)
    wv, ws = oracle.quant_e4m3_b128(x)
    assert_same(s, ws, "scales")
    assert_same(v, wv, "E4M3 values")
    assert_same(y, oracle.dequant_e4m3_b128(wv, ws), "bf16")
    for blocks in (1, 5, 67):
        xr = workloads.rows(5, 3, 0, 1, 128 * blocks)[0]
        v, s, y = gpu_e4m3(xr)
        wv, ws = oracle.quant_e4m3_b128(xr)
        assert_same(v, wv, f"values ({blocks} blocks)")
        assert_same(s, ws, f"scales ({blocks} blocks)")
        assert_same(y, oracle.dequant_e4m3_b128(wv, ws), f"bf16 ({blocks} blocks)")


def test_e4m3_b128_cfg5_full():
    say("e4m3 b128 cfg5 16384x7168 (full compare)")
    x = workloads.tensor(5, 0)
    v, s, y = gpu_e4m3(x)
    wv, ws = oracle.quant_e4m3_b128(x)
    assert_same(v, wv, "values")
    assert_same(s, ws, "scales")
    assert_same(y, oracle.dequant_e4m3_b128(wv, ws), "bf16")


# ---- graphs, repeatability, errors ---------------------------------------------------------

def test_graph_replay_matches_eager():
    say("ring allreduce in a HIP graph vs eager")
    W, rows = 4, 64
    parts = [workloads.rows(2, r, 0, rows, COLS).reshape(-1) for r in range(W)]
    n = parts[0].size
    pd = [to_dev(p) for p in parts]
    qw, sw = empty(n, np.int8), empty(n // 128, np.float32)
    outs = [empty(n, np.uint16) for _ in range(W)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bq.bq_ring_allreduce_i8(pd, qw, sw, outs, n=n, stream=s)
    s.synchronize()
    eager = [o.clone() for o in outs]
    eager_q = qw.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bq.bq_ring_allreduce_i8(pd, qw, sw, outs, n=n, stream=s)
    for rep in range(3):
        for o in outs:
            o.zero_()
        qw.zero_()
        sync()
        g.replay()
        sync()
        for r in range(W):
            assert torch.equal(outs[r], eager[r]), f"replay {rep} rank {r}"
        assert torch.equal(qw, eager_q), f"replay {rep} payload"
        _ = torch.randn(1024, device="cuda").sum().item()     # eager work between replays


def test_repeat_runs_are_bit_identical():
    say("repeatability")
    parts = [workloads.rows(3, r, 0, 96, COLS).reshape(-1) for r in range(4)]
    a = gpu_a2a(parts)
    b = gpu_a2a(parts)
    for t1, t2 in zip(a[:3], b[:3]):
        assert torch.equal(t1, t2)
    for o1, o2 in zip(a[3], b[3]):
        assert torch.equal(o1, o2)


def test_invalid_calls_write_nothing():
    say("invalid calls leave outputs untouched")
    n = 4096
    x = to_dev(workloads.rows(6, 0, 0, 1, n)[0])
    q = filled(n + 16, np.int8, 0x3C)
    s = filled(n // 128, np.float32, 0x3C)
    with pytest.raises(bq.BlockqError) as e:
        bq.bq_quant_i8(x, q[8:], s, n=n)                  # misaligned payload pointer
    assert e.value.name == "BQ_ERR_ALIGN"
    with pytest.raises(bq.BlockqError):
        bq.bq_quant_i8(x, q, s, n=n + 64)                 # not a multiple of 128
    sync()
    assert bool((q.view(torch.uint8) == 0x3C).all()) and bool((s.view(torch.uint8) == 0x3C).all())
