"""GPU parity of the MXFP8 collective entry points (flat layout) against the CPU oracle.

Bar: E4M3 codes, E8M0 bytes and every bf16 output bit for bit.  Inputs come from the
seeded generators in ``workloads`` or are built here from the codec's fields; expected
values come only from ``oracle``.
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


def assert_same(got, want, what):
    got, want = np.asarray(got).reshape(-1), np.asarray(want).reshape(-1)
    assert got.shape == want.shape, what
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"got {got[bad[:5]]} want {want[bad[:5]]}"


# ---- flat quantize / dequantize -----------------------------------------------------------

@pytest.mark.parametrize("blocks", [1, 3, 5, 17, 64, 257])
def test_mx_flat_batch_matches_oracle(blocks):
    say(f"mx flat quant/dequant batch of 3, {blocks} blocks each")
    n = 128 * blocks
    xs = [workloads.rows(4, s, 0, 1, n)[0] for s in range(3)]
    xd = [to_dev(x) for x in xs]
    vs = [empty(n, np.uint8) for _ in xs]
    es = [empty(n // 32, np.uint8) for _ in xs]
    bq.bq_quant_mx_batch(xd, vs, es, n=n)
    ys = [empty(n, np.uint16) for _ in xs]
    bq.bq_dequant_mx_batch(vs, es, ys, n=n)
    sync()
    for i, x in enumerate(xs):
        wv, we = oracle.quant_mx_flat(x)
        assert_same(host(vs[i], np.uint8), wv, f"codes {i}")
        assert_same(host(es[i], np.uint8), we, f"bytes {i}")
        assert_same(host(ys[i], np.uint16), oracle.dequant_mx_flat(wv, we), f"values {i}")


# ---- the mx_ring hop ----------------------------------------------------------------------

def gpu_hop(v, e, loc, in_place=False):
    n = v.size
    vi, ei, ld = to_dev(v), to_dev(e), to_dev(loc)
    if in_place:
        bq.bq_ring_hop_mx(vi, ei, ld, vi, ei, n=n)
        sync()
        return host(vi, np.uint8), host(ei, np.uint8)
    vo, eo = empty(n, np.uint8), empty(n // 32, np.uint8)
    bq.bq_ring_hop_mx(vi, ei, ld, vo, eo, n=n)
    sync()
    return host(vo, np.uint8), host(eo, np.uint8)


def test_mx_ring_hop_matches_oracle_and_in_place():
    say("mx ring hop 768x7168, out of place and in place")
    x = workloads.rows(2, 1, 0, 768, COLS).reshape(-1)
    loc = workloads.rows(2, 2, 0, 768, COLS).reshape(-1)
    wv, we = oracle.quant_mx_flat(x)
    hv, he = oracle.ring_hop_mx(wv, we, loc)
    gv, ge = gpu_hop(wv, we, loc)
    assert_same(gv, hv, "hop codes")
    assert_same(ge, he, "hop bytes")
    gv, ge = gpu_hop(wv, we, loc, in_place=True)
    assert_same(gv, hv, "in-place hop codes")
    assert_same(ge, he, "in-place hop bytes")


def _bf16_pow2(k: int) -> int:
    """bf16 bits of 2^k (normal or subnormal); k >= -133."""
    if k >= -126:
        return (k + 127) << 7
    return 1 << (k + 133)


def test_mx_ring_hop_scale_byte_boundaries():
    """Group amax exactly 448 * 2^(b-127), one bf16 step above and below it, for every
    byte b a finite payload can carry -- the E8M0 rule's octave boundaries from a binary32
    amax, including the range where fl32(amax/448) is subnormal (b <= 1) -- plus signed
    zeros and all-zero groups."""
    say("mx ring hop E8M0 boundaries from binary32 sums")
    groups_v, groups_e, groups_l = [], [], []
    for b in range(0, 247):
        for d in (0, 1, -1):
            v = np.zeros(32, np.uint8)
            loc = np.zeros(32, np.uint16)
            v[0] = 0x7E                                  # 448 * 2^(b-127)
            v[5] = 0x80                                  # -0 payload value
            loc[5] = 0x8000 if b % 2 else 0             # -0 + -0 = -0 on odd b
            if d:
                k = max(b - 127 - 15, -133)              # a bf16 step the fp32 sum keeps
                loc[0] = _bf16_pow2(k) | (0x8000 if d < 0 else 0)
            v[9] = 0x38 | (0x80 if b % 3 == 0 else 0)    # +-1.0 * 2^(b-127)
            groups_v.append(v)
            groups_e.append(b)
            groups_l.append(loc)
    zero_v, zero_l = np.zeros(32, np.uint8), np.zeros(32, np.uint16)
    zero_v[3], zero_l[3] = 0x80, 0x8000
    for b in (0, 127, 246):
        groups_v.append(zero_v.copy())
        groups_e.append(b)
        groups_l.append(zero_l.copy())
    while len(groups_v) % 4:
        groups_v.append(np.zeros(32, np.uint8))
        groups_e.append(127)
        groups_l.append(np.zeros(32, np.uint16))
    v = np.concatenate(groups_v)
    e = np.array(groups_e, np.uint8)
    loc = np.concatenate(groups_l)
    hv, he = oracle.ring_hop_mx(v, e, loc)
    gv, ge = gpu_hop(v, e, loc)
    assert_same(ge, he, "bytes")
    assert_same(gv, hv, "codes")
    assert len(set(he.tolist())) > 200


def test_mx_ring_hop_random_fields():
    """Random codes (NaN codes excluded), random bytes over [0, 240] and bf16 locals
    within +-24 octaves of each group's scale."""
    say("mx ring hop random fields")
    rng = np.random.default_rng(11)
    ng = 4 * 2048
    e = rng.integers(0, 241, ng).astype(np.uint8)
    v = rng.integers(0, 256, ng * 32).astype(np.uint8)
    v[(v & 0x7F) == 0x7F] = 0x7E
    k = np.repeat(e.astype(np.int64) - 127, 32) + rng.integers(-24, 9, ng * 32)
    k = np.clip(k, -133, 127)
    mag = np.where(k >= -126, ((k + 127) << 7) | rng.integers(0, 128, k.size),
                   1 << np.clip(k + 133, 0, 6))
    loc = (mag | (rng.integers(0, 2, k.size) << 15)).astype(np.uint16)
    loc[rng.random(k.size) < 0.1] = 0
    hv, he = oracle.ring_hop_mx(v, e, loc)
    gv, ge = gpu_hop(v, e, loc)
    assert_same(ge, he, "bytes")
    assert_same(gv, hv, "codes")


# ---- the mx_a2a accumulate and owner step ---------------------------------------------------

@pytest.mark.parametrize("nsrc", [1, 2, 3, 5, 9, 64])
def test_mx_accum_sources(nsrc):
    say(f"mx accumulate nsrc={nsrc}")
    n = 128 * 77
    xs = [workloads.rows(7, s, 0, 1, n)[0] for s in range(nsrc)]
    vs, es = zip(*[oracle.quant_mx_flat(x) for x in xs])
    want = oracle.dequant_accum_mx(list(vs), list(es))
    y = empty(n, np.uint16)
    bq.bq_dequant_accum_mx([to_dev(v) for v in vs], [to_dev(e) for e in es], y, n=n)
    sync()
    assert_same(host(y, np.uint16), want, "accumulated bf16")


@pytest.mark.parametrize("nseg,nsrc,rows", [(4, 4, 48), (2, 3, 6), (16, 16, 32), (1, 1, 3)])
def test_mx_a2a_reduce_fused_matches_oracle(nseg, nsrc, rows):
    say(f"mx fused a2a owner step nseg={nseg} nsrc={nsrc} rows={rows}")
    n = rows * 1024
    parts = [workloads.rows(3, r, 0, rows, 1024).reshape(-1) for r in range(nsrc)]
    vs, es = zip(*[oracle.quant_mx_flat(p) for p in parts])
    wv, we, wys, wred = oracle.a2a_reduce_mx(list(vs), list(es), nseg)
    m = n // nseg
    vo, eo, red = empty(n, np.uint8), empty(n // 32, np.uint8), empty(n, np.uint16)
    ys = [filled(m, np.uint16, 0x5A) for _ in range(nseg)]
    bq.bq_a2a_reduce_mx(nseg, [to_dev(v) for v in vs], [to_dev(e) for e in es], vo, eo,
                        y_out=ys, red=red, seg_n=m)
    sync()
    assert_same(host(vo, np.uint8), wv, "payload")
    assert_same(host(eo, np.uint8), we, "bytes")
    assert_same(host(red, np.uint16), wred, "owner sums")
    for j in range(nseg):
        assert_same(host(ys[j], np.uint16), wys[j], f"owner {j} materialization")


def test_mx_allgather_skip_own_leaves_the_owner_shard():
    say("mx all-gather dequant, skip own shard")
    W, n = 4, 4 * 2048
    x = workloads.rows(1, 0, 0, 8, 1024).reshape(-1)
    wv, we = oracle.quant_mx_flat(x)
    y = oracle.dequant_mx_flat(wv, we)
    outs = [filled(n, np.uint16, 0x77) for _ in range(W)]
    bq.bq_allgather_dequant_mx(to_dev(wv), to_dev(we), outs, skip_own=True, n=n)
    sync()
    m = n // W
    for r in range(W):
        got = host(outs[r], np.uint16)
        for j in range(W):
            seg = got[j * m:(j + 1) * m]
            if j == r:
                assert np.all(seg == 0x7777), f"rank {r} wrote its own shard"
            else:
                assert_same(seg, y[j * m:(j + 1) * m], f"rank {r} shard {j}")


# ---- the drivers ------------------------------------------------------------------------------

def gpu_mx_ring(partials):
    W, n = len(partials), partials[0].size
    pd = [to_dev(p.reshape(-1)) for p in partials]
    vw, ew = empty(n, np.uint8), empty(n // 32, np.uint8)
    outs = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_ring_allreduce_mx(pd, vw, ew, outs, n=n)
    sync()
    return vw, ew, outs


def gpu_mx_a2a(partials, with_red=True):
    W, n = len(partials), partials[0].size
    pd = [to_dev(p.reshape(-1)) for p in partials]
    vs = [empty(n, np.uint8) for _ in range(W)]
    es = [empty(n // 32, np.uint8) for _ in range(W)]
    red = empty(n, np.uint16) if with_red else None
    vb, eb = empty(n, np.uint8), empty(n // 32, np.uint8)
    outs = [empty(n, np.uint16) for _ in range(W)]
    bq.bq_a2a_allreduce_mx(pd, vs, es, red, vb, eb, outs, n=n)
    sync()
    return red, vb, eb, outs


@pytest.mark.parametrize("W,rows", [(1, 4), (2, 6), (3, 9), (4, 12), (8, 16)])
def test_mx_ring_allreduce_small(W, rows):
    say(f"mx ring allreduce W={W} rows={rows}")
    parts = [workloads.rows(2, r, 0, rows, 1024).reshape(-1) for r in range(W)]
    wv, we, wouts = oracle.ring_allreduce_mx(parts)
    vw, ew, outs = gpu_mx_ring(parts)
    assert_same(host(vw, np.uint8), wv, "final codes")
    assert_same(host(ew, np.uint8), we, "final bytes")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


def test_mx_ring_allreduce_cfg2_full():
    """4 simulated ranks x 3072x7168 with the MXFP8 codec, compared in full."""
    say("mx ring allreduce 4x3072x7168 (full compare)")
    parts = [workloads.tensor(2, r).reshape(-1) for r in range(4)]
    wv, we, wouts = oracle.ring_allreduce_mx(parts)
    vw, ew, outs = gpu_mx_ring(parts)
    assert_same(host(vw, np.uint8), wv, "final codes")
    assert_same(host(ew, np.uint8), we, "final bytes")
    for r in range(4):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


@pytest.mark.parametrize("W,rows", [(1, 4), (2, 6), (4, 12), (8, 16)])
def test_mx_a2a_allreduce_small(W, rows):
    say(f"mx a2a allreduce W={W} rows={rows}")
    parts = [workloads.rows(3, r, 0, rows, 1024).reshape(-1) for r in range(W)]
    wred, wv, we, wouts = oracle.a2a_allreduce_mx(parts)
    red, vb, eb, outs = gpu_mx_a2a(parts)
    assert_same(host(red, np.uint16), wred, "owner sums")
    assert_same(host(vb, np.uint8), wv, "broadcast codes")
    assert_same(host(eb, np.uint8), we, "broadcast bytes")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


@pytest.mark.parametrize("W", [4, 16])
def test_mx_a2a_cfg3_full(W):
    """4 and 16 ranks x 3072x7168: the broadcast payload and every rank's output against
    the oracle in full (the 16-rank oracle takes about half a minute), every rank's output
    bit-identical on the GPU; driver run without red."""
    say(f"mx a2a W={W} {W}x3072x7168 (full compare)")
    parts = [workloads.tensor(3, r).reshape(-1) for r in range(W)]
    _, vb, eb, outs = gpu_mx_a2a(parts, with_red=False)
    for r in range(1, W):
        assert torch.equal(outs[r], outs[0]), f"rank {r} differs from rank 0"
    _, wv, we, wouts = oracle.a2a_allreduce_mx(parts)
    assert_same(host(vb, np.uint8), wv, "codes")
    assert_same(host(eb, np.uint8), we, "bytes")
    for r in range(W):
        assert_same(host(outs[r], np.uint16), wouts[r], f"rank {r} output")


def test_mx_ring_graph_replay_matches_eager():
    """The mx_ring driver captured in a HIP graph, replayed three times with eager work
    and synchronizations between replays: every replay equals the eager result."""
    say("mx ring allreduce graph replay")
    W, rows = 4, 16
    parts = [workloads.rows(2, r, 0, rows, 1024).reshape(-1) for r in range(W)]
    n = parts[0].size
    pd = [to_dev(p) for p in parts]
    vw, ew = empty(n, np.uint8), empty(n // 32, np.uint8)
    outs = [empty(n, np.uint16) for _ in range(W)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        bq.bq_ring_allreduce_mx(pd, vw, ew, outs, n=n, stream=stream)
    stream.synchronize()
    want = [host(o, np.uint16).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        bq.bq_ring_allreduce_mx(pd, vw, ew, outs, n=n, stream=stream)
    for rep in range(3):
        for o in outs:
            o.zero_()
        vw.zero_()
        sync()
        g.replay()
        sync()
        for r in range(W):
            assert_same(host(outs[r], np.uint16), want[r], f"replay {rep} rank {r}")
        _ = torch.randn(1024, device="cuda").sum().item()     # eager work between replays


@pytest.mark.parametrize("codec", ["i8", "mx"])
def test_a2a_graph_replay_matches_eager(codec):
    """The i8_a2a / mx_a2a driver captured in a HIP graph, replayed three times with eager
    work and synchronizations between replays: every replay equals the eager result, the
    owner sums and the broadcast payload included."""
    say(f"{codec} a2a allreduce graph replay")
    W, rows = 4, 16
    parts = [workloads.rows(3, r, 0, rows, 1024).reshape(-1) for r in range(W)]
    n = parts[0].size
    pd = [to_dev(p) for p in parts]
    if codec == "i8":
        send = ([empty(n, np.int8) for _ in range(W)], [empty(n // 128, np.float32) for _ in range(W)])
        bcast = (empty(n, np.int8), empty(n // 128, np.float32))
        run = bq.bq_a2a_allreduce_i8
    else:
        send = ([empty(n, np.uint8) for _ in range(W)], [empty(n // 32, np.uint8) for _ in range(W)])
        bcast = (empty(n, np.uint8), empty(n // 32, np.uint8))
        run = bq.bq_a2a_allreduce_mx
    red = empty(n, np.uint16)
    outs = [empty(n, np.uint16) for _ in range(W)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(pd, send[0], send[1], red, bcast[0], bcast[1], outs, n=n, stream=stream)
    stream.synchronize()
    want = [o.clone() for o in outs] + [red.clone(), bcast[0].clone(), bcast[1].clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run(pd, send[0], send[1], red, bcast[0], bcast[1], outs, n=n, stream=stream)
    for rep in range(3):
        for t in outs + [red, bcast[0], bcast[1]] + send[0] + send[1]:
            t.zero_()
        sync()
        g.replay()
        sync()
        got = outs + [red, bcast[0], bcast[1]]
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"
        _ = torch.randn(1024, device="cuda").sum().item()     # eager work between replays
