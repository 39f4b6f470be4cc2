#!/usr/bin/env python3
"""Benchmark of the block-quantized wire codec path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: four
simulated ranks, each holding a 3072x7168 bf16 partial (N(0, 0.5)), go through
  * the i8_ring all-reduce: block-INT8 quantize, three fused ring-hop steps, and
    every rank's materialization from the final payloads;
  * the i8_a2a all-reduce: quantize once, then per owner one fused pass (4-source
    FP32 accumulate, bf16 rounding, requantize, the owner's own materialization),
    then the other ranks' materialization of every shard;
  * MXFP8: the four partials staged as 128-aligned slices of a 3072x28672 buffer,
    then dequantized;
  * the E4M3 128-block codec on rank 0's partial, quantize and dequantize.

`value` is the metric itself: the block-INT8 quantize of the ring's step-0 chunks
(4 ranks x 768x7168, 3072x7168 values in one launch) followed by the three 4-rank
fused ring-hop steps, timed as a region of its own (K passes back to back), as
algorithmic bytes (each kernel's inputs read once, outputs written once) over time,
in GB/s against the 8 TB/s HBM peak.  The whole step is reported beside it
(`step`), and so is every distinct kernel of the step alone (`kernels`), one TP4
rank's own quantize and hop as single-segment launches (`share_kernels`), each of
the five workload configurations at full size (`configs`) and the staged MXFP8
GEMM (`gemm`).  Inputs are resident in HBM.  Sixteen complete buffer sets (inputs,
intermediates, outputs; about 1.5 GB each) rotate pass by pass -- and launch by launch
when a kernel is timed alone -- so inputs are cold in the 256 MB last-level cache while
what a kernel consumes from the previous kernel of the same pass may be served by it,
as in any pipeline on one GPU.

Every timed region starts behind a 2 GiB read queued on the same stream, so the host has
enqueued the region's launches before the GPU reaches them: the events then bracket GPU
work only, with no gap waiting for the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --sweep             (quantize, hop and copy from 8 MB to 1 GB)
       python bench.py --gemm              (the staged MXFP8 GEMM alone)
       python bench.py --summarize-trace CSV   (rocprofv3 kernel trace -> table)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) for i8 quant + ring-hop at 3072×7168 bf16"
W = 4
ROWS, COLS = 3072, 7168
N = ROWS * COLS
NB = N // 128
M = N // W                 # values per ring chunk / A2A shard
SETS = 16                  # rotating buffer sets, each a full step's inputs and outputs (~1.5 GB)
DRAWS = 4                  # distinct input draws; set k holds draw k % DRAWS at its own addresses
SAMPLES = 5                # timed samples per region (median reported)
REPS = 30                  # back-to-back launches per sample when a kernel is timed alone
CONFIG_PASSES = 10         # passes per sample of each workload configuration

# algorithmic bytes per 128 values of each kernel (inputs read once, outputs written once)
B_QUANT = 256 + 132        # bf16 in; int8 + fp32 scale out
B_DEQUANT = 132 + 256
B_DEQUANT_SHARED = lambda w: 132 + 256 * w   # w ranks materialize from one shared payload
B_HOP = 132 + 256 + 132    # payload + local bf16 in; payload out
B_ACCUM = lambda w: 132 * w + 256
B_A2A_REDUCE = lambda w: 132 * w + 132 + 256   # w sources in; payload + owner's bf16 out
B_ALLGATHER_SKIP = lambda w: 132 + 256 * (w - 1)   # shared payload once; w-1 ranks write
B_MX = 256 + 128 + 4       # bf16 in; E4M3 + 4 E8M0 bytes out (per 128 values)
# the flat MXFP8 payload has the INT8 payload's 132 bytes per 128 values, so the MXFP8
# collectives move the same bytes as their INT8 counterparts (B_HOP, B_A2A_REDUCE, ...)
B_E4M3 = 256 + 132


def code_only(text: str) -> str:
    """Source text without // comments, trailing blanks and blank lines (the device sources
    hold no // inside string literals)."""
    lines = (line.split("//", 1)[0].rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_digest() -> str:
    """Digest of the device code of the metric's kernels -- the INT8 kernels' source and the
    headers it includes, comments left out: the HBM counters in profiles/ stay valid while it
    is unchanged; host-side validation, comments and other kernel families may change."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_wire_amd", "csrc")
    for name in ("bq_device.h", "bq_i8.hip", "bq_launch.h"):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + code_only(f.read()).encode())
    return h.hexdigest()[:16]


class Step:
    """All buffers of one step and its launches as (name, algorithmic bytes, fn, args).

    `calls` is the step as a user runs it: the two collective drivers, the MXFP8 slice
    and dequantize calls and the E4M3 codec calls.  `kernels` is the same work as the
    primitive calls the drivers make, one kernel launch each, for per-kernel timing.
    """

    def __init__(self, torch, bq, sets: int):
        import workloads
        self.torch, self.bq = torch, bq
        L = self.L = bq.lib
        dev = "cuda"
        i16, i8, u8, f32 = torch.int16, torch.int8, torch.uint8, torch.float32
        e = lambda n, dt: torch.empty(n, dtype=dt, device=dev)
        self.sets = []
        for k in range(sets):
            if k < DRAWS:
                parts = [torch.from_numpy(workloads.rows(2, r + 16 * k, 0, ROWS, COLS)
                                          .view(np.int16)).to(dev) for r in range(W)]
            else:
                parts = [t.clone() for t in self.sets[k % DRAWS]["parts"]]
            b = {"parts": parts}
            b["q_wire"], b["s_wire"] = e(N, i8), e(NB, f32)
            b["ring_out"] = [e(N, i16) for _ in range(W)]
            b["q_send"] = [e(N, i8) for _ in range(W)]
            b["s_send"] = [e(NB, f32) for _ in range(W)]
            b["red"], b["q_bc"], b["s_bc"] = e(N, i16), e(N, i8), e(NB, f32)
            b["a2a_out"] = [e(N, i16) for _ in range(W)]
            b["mx_v"] = torch.empty((ROWS, W * COLS), dtype=u8, device=dev)
            b["mx_e"] = torch.empty((ROWS, W * COLS // 32), dtype=u8, device=dev)
            b["mx_y"] = torch.empty((ROWS, W * COLS), dtype=i16, device=dev)
            b["e4_v"], b["e4_s"], b["e4_y"] = e(N, u8), e(NB, f32), e(N, i16)
            # the MXFP8 collectives (not part of the step; timed beside it)
            b["mxw_v"], b["mxw_e"] = e(N, u8), e(N // 32, u8)
            b["mxr_out"] = [e(N, i16) for _ in range(W)]
            b["mx_send_v"] = [e(N, u8) for _ in range(W)]
            b["mx_send_e"] = [e(N // 32, u8) for _ in range(W)]
            b["mx_bc_v"], b["mx_bc_e"] = e(N, u8), e(N // 32, u8)
            b["mxa_out"] = [e(N, i16) for _ in range(W)]
            self.sets.append(b)
        self.stream = torch.cuda.current_stream()
        sp = ctypes.c_void_p(self.stream.cuda_stream)
        A = lambda ptrs: (ctypes.c_void_p * len(ptrs))(*ptrs)
        P = lambda t: t.data_ptr()
        MB = M // 128
        self.calls, self.kernels, self.next_kernels, self.metric = [], [], [], []
        self.share_kernels = []
        for b in self.sets:
            parts = b["parts"]
            calls, kern, nxt = [], [], []
            xs = A([P(t) for t in parts])
            # i8_ring driver; and its kernels: rank r starts with chunk r-1 and at step k
            # folds chunk r-1-k into the payload it received
            ring_bytes = NB * B_QUANT + (W - 1) * NB * B_HOP + NB * B_DEQUANT_SHARED(W)
            calls.append(("i8_ring_allreduce", ring_bytes,
                          L.bq_ring_allreduce_i8, (W, N, xs, P(b["q_wire"]), P(b["s_wire"]),
                                                   A([P(t) for t in b["ring_out"]]), sp)))
            chunk = lambda r, k: (r - 1 - k) % W
            x0 = A([P(parts[r]) + 2 * M * chunk(r, 0) for r in range(W)])
            q0 = A([P(b["q_wire"]) + M * chunk(r, 0) for r in range(W)])
            s0 = A([P(b["s_wire"]) + 4 * MB * chunk(r, 0) for r in range(W)])
            kern.append(("quant_i8 x4", NB * B_QUANT, L.bq_quant_i8_batch, (W, x0, M, q0, s0, sp)))
            for k in range(1, W):
                lk = A([P(parts[r]) + 2 * M * chunk(r, k) for r in range(W)])
                qk = A([P(b["q_wire"]) + M * chunk(r, k) for r in range(W)])
                sk = A([P(b["s_wire"]) + 4 * MB * chunk(r, k) for r in range(W)])
                kern.append(("ring_hop_i8 x4", NB * B_HOP, L.bq_ring_hop_i8_batch,
                             (W, qk, sk, lk, M, qk, sk, sp)))
            kern.append(("allgather_dequant_i8 x4", NB * B_DEQUANT_SHARED(W),
                         L.bq_allgather_dequant_i8,
                         (W, P(b["q_wire"]), P(b["s_wire"]), N, A([P(t) for t in b["ring_out"]]),
                          0, sp)))
            # i8_a2a driver and its kernels: quantize once, fused owner step (payload and
            # the owner's own shard), the other ranks' materialization of each shard
            a2a_bytes = (W * NB * B_QUANT + NB * B_A2A_REDUCE(W) + NB * B_ALLGATHER_SKIP(W))
            qsend, ssend = A([P(t) for t in b["q_send"]]), A([P(t) for t in b["s_send"]])
            outs = A([P(t) for t in b["a2a_out"]])
            calls.append(("i8_a2a_allreduce", a2a_bytes,
                          L.bq_a2a_allreduce_i8, (W, N, xs, qsend, ssend, None, P(b["q_bc"]),
                                                  P(b["s_bc"]), outs, sp)))
            kern.append(("quant_i8 x4", W * NB * B_QUANT, L.bq_quant_i8_batch,
                         (W, xs, N, qsend, ssend, sp)))
            own = A([P(b["a2a_out"][j]) + 2 * M * j for j in range(W)])
            kern.append(("a2a_reduce_i8 4src x4 owners", NB * B_A2A_REDUCE(W), L.bq_a2a_reduce_i8,
                         (W, W, qsend, ssend, M, P(b["q_bc"]), P(b["s_bc"]), own, None, sp)))
            kern.append(("allgather_dequant_i8 x4 skip own", NB * B_ALLGATHER_SKIP(W),
                         L.bq_allgather_dequant_i8, (W, P(b["q_bc"]), P(b["s_bc"]), N, outs, 1, sp)))
            # MXFP8: the four partials as 128-aligned slices of the staging buffer
            for r in range(W):
                c = ("quant_mx_slice", NB * B_MX, L.bq_quant_mx_slice,
                     (P(parts[r]), ROWS, COLS, COLS, COLS * r, P(b["mx_v"]), W * COLS,
                      P(b["mx_e"]), W * COLS // 32, ROWS, sp))
                calls.append(c)
                kern.append(c)
            c = ("dequant_mx", W * NB * B_MX, L.bq_dequant_mx,
                 (P(b["mx_v"]), W * COLS, P(b["mx_e"]), W * COLS // 32, ROWS, W * COLS,
                  P(b["mx_y"]), W * COLS, sp))
            calls.append(c)
            kern.append(c)
            # E4M3 128-block codec on rank 0
            for c in (("quant_e4m3_b128", NB * B_E4M3, L.bq_quant_e4m3_b128,
                       (P(parts[0]), N, P(b["e4_v"]), P(b["e4_s"]), sp)),
                      ("dequant_e4m3_b128", NB * B_E4M3, L.bq_dequant_e4m3_b128,
                       (P(b["e4_v"]), P(b["e4_s"]), N, P(b["e4_y"]), sp))):
                calls.append(c)
                kern.append(c)
            # MXFP8 ring and all-to-all (the mx_ring / mx_a2a modes) at the same shapes
            v0 = A([P(b["mxw_v"]) + M * chunk(r, 0) for r in range(W)])
            e0 = A([P(b["mxw_e"]) + (M // 32) * chunk(r, 0) for r in range(W)])
            nxt.append(("quant_mx_flat x4", NB * B_MX, L.bq_quant_mx_batch, (W, x0, M, v0, e0, sp)))
            for k in range(1, W):
                lk = A([P(parts[r]) + 2 * M * chunk(r, k) for r in range(W)])
                vk = A([P(b["mxw_v"]) + M * chunk(r, k) for r in range(W)])
                ek = A([P(b["mxw_e"]) + (M // 32) * chunk(r, k) for r in range(W)])
                nxt.append(("ring_hop_mx x4", NB * B_HOP, L.bq_ring_hop_mx_batch,
                            (W, vk, ek, lk, M, vk, ek, sp)))
            nxt.append(("allgather_dequant_mx x4", NB * B_DEQUANT_SHARED(W),
                        L.bq_allgather_dequant_mx,
                        (W, P(b["mxw_v"]), P(b["mxw_e"]), N, A([P(t) for t in b["mxr_out"]]), 0,
                         sp)))
            vsend, esend = A([P(t) for t in b["mx_send_v"]]), A([P(t) for t in b["mx_send_e"]])
            mouts = A([P(t) for t in b["mxa_out"]])
            nxt.append(("quant_mx_flat x4", W * NB * B_MX, L.bq_quant_mx_batch,
                        (W, xs, N, vsend, esend, sp)))
            mown = A([P(b["mxa_out"][j]) + 2 * M * j for j in range(W)])
            nxt.append(("a2a_reduce_mx 4src x4 owners", NB * B_A2A_REDUCE(W), L.bq_a2a_reduce_mx,
                        (W, W, vsend, esend, M, P(b["mx_bc_v"]), P(b["mx_bc_e"]), mown, None, sp)))
            nxt.append(("allgather_dequant_mx x4 skip own", NB * B_ALLGATHER_SKIP(W),
                        L.bq_allgather_dequant_mx,
                        (W, P(b["mx_bc_v"]), P(b["mx_bc_e"]), N, mouts, 1, sp)))
            # one TP4 rank's share as its own single-segment launches: rank 0's step-0
            # quantize of its 768x7168 chunk and its hop of the next chunk, in place
            c1 = chunk(0, 1)
            share = [("quant_i8 one rank", MB * B_QUANT, L.bq_quant_i8,
                      (P(parts[0]) + 2 * M * chunk(0, 0), M, P(b["q_wire"]) + M * chunk(0, 0),
                       P(b["s_wire"]) + 4 * MB * chunk(0, 0), sp)),
                     ("ring_hop_i8 one rank", MB * B_HOP, L.bq_ring_hop_i8,
                      (P(b["q_wire"]) + M * c1, P(b["s_wire"]) + 4 * MB * c1,
                       P(parts[0]) + 2 * M * c1, M, P(b["q_wire"]) + M * c1,
                       P(b["s_wire"]) + 4 * MB * c1, sp))]
            self.calls.append(calls)
            self.kernels.append(kern)
            self.next_kernels.append(nxt)
            self.share_kernels.append(share)
            # the metric: the ring's step-0 quantize and its three hop steps
            self.metric.append(kern[:W])
        assert sum(c[1] for c in self.calls[0]) == sum(k[1] for k in self.kernels[0])
        assert [k[0] for k in self.metric[0]] == ["quant_i8 x4"] + ["ring_hop_i8 x4"] * (W - 1)

    @property
    def step_bytes(self) -> int:
        return sum(c[1] for c in self.calls[0])

    @property
    def metric_bytes(self) -> int:
        return sum(c[1] for c in self.metric[0])

    def run(self, i: int) -> None:
        run_calls(self.calls[i % len(self.calls)])

    def run_metric(self, i: int) -> None:
        run_calls(self.metric[i % len(self.metric)])


def run_calls(calls) -> None:
    """Launch a list of pre-marshalled (name, bytes, C function, args) calls."""
    for name, _, fn, args in calls:
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{name}: status {st}")


class Region:
    """Timing of launches on one stream between two HIP events.  A read of 2 GiB (a sum) is
    queued first, on the same stream: it keeps the GPU busy for about half a millisecond
    while the host enqueues the region's launches, so the GPU never waits for the host
    inside the region and the events bracket GPU work only.  Being a read, it also leaves
    the 256 MB last-level cache holding only clean lines of its own -- the region's first
    inputs are cold and no earlier write is still waiting to be written back (a copy
    there instead measurably slowed the first launches of each region)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.src = torch.zeros(1 << 29, dtype=torch.float32, device="cuda")

    def time_us(self, launch) -> float:
        """Microseconds from the first to the last of the launches `launch()` enqueues."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            self.total = self.src.sum()
        e0.record(self.stream)
        launch()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3


def time_kernels(region: Region, seqs, reps: int, samples: int) -> dict:
    """Each distinct kernel of `seqs` (a list, one per buffer set, of call lists) alone:
    `reps` back-to-back launches rotating over the buffer sets (consecutive launches share
    no buffer, so inputs are cold in the last-level cache) between one pair of events, in
    `samples` samples taken round-robin over the kernels; the median is reported."""
    kinds = {}
    for k, (name, nbytes, _, _) in enumerate(seqs[0]):
        kinds.setdefault((name, nbytes), []).append(k)
    got = {key: [] for key in kinds}
    for smp in range(samples):
        for key, idx in kinds.items():
            def launch(smp=smp, idx=idx):
                for i in range(smp * reps, (smp + 1) * reps):
                    run_calls([seqs[i % len(seqs)][idx[i % len(idx)]]])
            got[key].append(region.time_us(launch) / reps)
    out = {}
    for (name, nbytes), idx in kinds.items():
        us = statistics.median(got[(name, nbytes)])
        gbs = nbytes / (us * 1e-6) / 1e9
        out[f"{name} ({nbytes} B)"] = {"bytes_per_launch": nbytes, "launches_per_pass": len(idx),
                                       "us_per_launch": round(us, 2), "gbs": round(gbs, 1),
                                       "frac": round(gbs / HBM_PEAK_GBS, 4),
                                       "us_per_pass": us * len(idx),
                                       "samples_us": [round(t, 2) for t in got[(name, nbytes)]]}
    return out


def rate(nbytes: int, values: int, us: float) -> dict:
    """A pass's throughput as GB/s and as values per second, each against the HBM peak
    (the values-per-second bound is the peak over the pass's bytes per value)."""
    gbs = nbytes / (us * 1e-6) / 1e9
    vps = values / (us * 1e-6)
    bound = HBM_PEAK_GBS * 1e9 / (nbytes / values)
    return {"us_per_pass": round(us, 2), "bytes_per_pass": nbytes, "gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "values_per_pass": values,
            "elements_per_s": round(vps, -6), "bytes_per_element": round(nbytes / values, 4),
            "elements_frac": round(vps / bound, 4)}


class ConfigRun:
    """One workload configuration at full size: per buffer set, the pass as a user runs it
    (`calls`, the public entry points) and as its kernel launches (`kernels`, for the
    per-kernel table); `values` counts the values a pass delivers."""

    def __init__(self, name, values, calls, kernels, keep):
        self.name, self.values, self.calls, self.kernels = name, values, calls, kernels
        self.keep = keep     # the device buffers, held while the config runs
        self.nbytes = sum(c[1] for c in calls[0])
        assert self.nbytes == sum(k[1] for k in kernels[0])


def _dev_sets(torch, host_arrays, sets):
    """`sets` device copies of each host array (bf16 bits as int16): the buffer sets hold
    the same values at different addresses."""
    base = [torch.from_numpy(a.reshape(-1).view(np.int16)).to("cuda") for a in host_arrays]
    return [base] + [[t.clone() for t in base] for _ in range(sets - 1)]


def build_configs(torch, bq, stream, which):
    """The five workload configurations, seeded synthetic inputs at full size."""
    import workloads
    L = bq.lib
    sp = ctypes.c_void_p(stream.cuda_stream)
    A = lambda ptrs: (ctypes.c_void_p * len(ptrs))(*ptrs)
    P = lambda t: t.data_ptr()
    e = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
    i16, i8, u8, f32 = torch.int16, torch.int8, torch.uint8, torch.float32
    for cfg in which:
        if cfg == "cfg1":
            # block-INT8 round trip of one 512x7168 tensor; 56 buffer sets (~1 GB)
            R1, n = 512, 512 * COLS
            nb = n // 128
            sets = 56
            xs = _dev_sets(torch, [workloads.rows(1, 0, 0, R1, COLS)], sets)
            calls, kern, keep = [], [], []
            for (x,) in xs:
                q, sc, y = e(n, i8), e(nb, f32), e(n, i16)
                keep += [x, q, sc, y]
                c = [("quant_i8", nb * B_QUANT, L.bq_quant_i8, (P(x), n, P(q), P(sc), sp)),
                     ("dequant_i8", nb * B_DEQUANT, L.bq_dequant_i8, (P(q), P(sc), n, P(y), sp))]
                calls.append(c)
                kern.append(c)
            yield ConfigRun("cfg1: block-INT8 quantize + dequantize round trip, 512x7168 bf16",
                            n, calls, kern, keep)
        elif cfg in ("cfg3_w4", "cfg3_w16"):
            Wc = 4 if cfg == "cfg3_w4" else 16
            n, nb = N, NB
            m, mb = n // Wc, NB // Wc
            host = [workloads.rows(3, r, 0, ROWS, COLS) for r in range(Wc)]
            sets = 2
            calls, kern, keep = [], [], []
            for parts in _dev_sets(torch, host, sets):
                qs = [e(n, i8) for _ in range(Wc)]
                ss = [e(nb, f32) for _ in range(Wc)]
                qb, sb = e(n, i8), e(nb, f32)
                outs = [e(n, i16) for _ in range(Wc)]
                keep += parts + qs + ss + [qb, sb] + outs
                xa, qa, sa, oa = (A([P(t) for t in v]) for v in (parts, qs, ss, outs))
                own = A([P(outs[j]) + 2 * m * j for j in range(Wc)])
                b_q, b_r, b_g = Wc * nb * B_QUANT, nb * B_A2A_REDUCE(Wc), nb * B_ALLGATHER_SKIP(Wc)
                calls.append([("i8_a2a_allreduce", b_q + b_r + b_g, L.bq_a2a_allreduce_i8,
                               (Wc, n, xa, qa, sa, None, P(qb), P(sb), oa, sp))])
                kern.append([(f"quant_i8 x{Wc}", b_q, L.bq_quant_i8_batch, (Wc, xa, n, qa, sa, sp)),
                             (f"a2a_reduce_i8 {Wc}src x{Wc} owners", b_r, L.bq_a2a_reduce_i8,
                              (Wc, Wc, qa, sa, m, P(qb), P(sb), own, None, sp)),
                             (f"allgather_dequant_i8 x{Wc} skip own", b_g,
                              L.bq_allgather_dequant_i8, (Wc, P(qb), P(sb), n, oa, 1, sp))])
            yield ConfigRun(f"cfg3: i8_a2a all-reduce, {Wc} ranks x 3072x7168 bf16 "
                            f"(shards {ROWS // Wc}x7168), 0.3*t(4)", n, calls, kern, keep)
        elif cfg == "cfg4":
            MR, K6 = 4096, 6
            ldv, lds = K6 * COLS, K6 * COLS // 32
            host = [workloads.rows(4, j, 0, MR, COLS) for j in range(K6)]
            nb_slice = MR * COLS // 128
            calls, kern, keep = [], [], []
            for sl in _dev_sets(torch, host, 2):
                v = torch.empty((MR, ldv), dtype=u8, device="cuda")
                es = torch.empty((MR, lds), dtype=u8, device="cuda")
                y = torch.empty((MR, ldv), dtype=i16, device="cuda")
                keep += sl + [v, es, y]
                c = [("quant_mx_slice 4096x7168", nb_slice * B_MX, L.bq_quant_mx_slice,
                      (P(sl[j]), MR, COLS, COLS, COLS * j, P(v), ldv, P(es), lds, MR, sp))
                     for j in range(K6)]
                c.append(("dequant_mx 4096x43008", K6 * nb_slice * B_MX, L.bq_dequant_mx,
                          (P(v), ldv, P(es), lds, MR, ldv, P(y), ldv, sp)))
                calls.append(c)
                kern.append(c)
            yield ConfigRun("cfg4: six 4096x7168 bf16 slices staged as MXFP8 into 4096x43008, "
                            "then dequantized", MR * ldv, calls, kern, keep)
        elif cfg == "cfg5":
            R5 = 16384
            n = R5 * COLS
            nb, m = n // 128, n // W
            mb = m // 128
            host = [workloads.rows(5, r, 0, R5, COLS) for r in range(W)]
            calls, kern, keep = [], [], []
            chunk = lambda r, k: (r - 1 - k) % W
            for parts in _dev_sets(torch, host, 2):
                qw, sw = e(n, i8), e(nb, f32)
                outs = [e(n, i16) for _ in range(W)]
                ev, es, ey = e(n, u8), e(nb, f32), e(n, i16)
                keep += parts + [qw, sw, ev, es, ey] + outs
                xa, oa = A([P(t) for t in parts]), A([P(t) for t in outs])
                ring_b = nb * B_QUANT + (W - 1) * nb * B_HOP + nb * B_DEQUANT_SHARED(W)
                e4 = [("quant_e4m3_b128 16384x7168", nb * B_E4M3, L.bq_quant_e4m3_b128,
                       (P(parts[0]), n, P(ev), P(es), sp)),
                      ("dequant_e4m3_b128 16384x7168", nb * B_E4M3, L.bq_dequant_e4m3_b128,
                       (P(ev), P(es), n, P(ey), sp))]
                calls.append([("i8_ring_allreduce", ring_b, L.bq_ring_allreduce_i8,
                               (W, n, xa, P(qw), P(sw), oa, sp))] + e4)
                k = [("quant_i8 x4 4096x7168", nb * B_QUANT, L.bq_quant_i8_batch,
                      (W, A([P(parts[r]) + 2 * m * chunk(r, 0) for r in range(W)]), m,
                       A([P(qw) + m * chunk(r, 0) for r in range(W)]),
                       A([P(sw) + 4 * mb * chunk(r, 0) for r in range(W)]), sp))]
                for s_ in range(1, W):
                    qk = A([P(qw) + m * chunk(r, s_) for r in range(W)])
                    sk = A([P(sw) + 4 * mb * chunk(r, s_) for r in range(W)])
                    lk = A([P(parts[r]) + 2 * m * chunk(r, s_) for r in range(W)])
                    k.append(("ring_hop_i8 x4 4096x7168", nb * B_HOP, L.bq_ring_hop_i8_batch,
                              (W, qk, sk, lk, m, qk, sk, sp)))
                k.append(("allgather_dequant_i8 x4 16384x7168", nb * B_DEQUANT_SHARED(W),
                          L.bq_allgather_dequant_i8, (W, P(qw), P(sw), n, oa, 0, sp)))
                kern.append(k + e4)
            yield ConfigRun("cfg5: i8_ring all-reduce of 4 ranks x 16384x7168 bf16 partials "
                            "(12 hops of 4096x7168), t(3) with zero blocks and spikes, plus the "
                            "E4M3 128-block codec on 16384x7168", n, calls, kern, keep)


CONFIGS = ["cfg1", "cfg3_w4", "cfg3_w16", "cfg4", "cfg5"]


def config_bench(torch, bq, region: Region, stream, passes: int, reps: int,
                 which=CONFIGS) -> dict:
    """Every configuration at full size: `passes` passes back to back (rotating buffer sets)
    as one timed region, and each of its kernels alone."""
    out = {}
    for cr in build_configs(torch, bq, stream, which):
        for i in range(2 * len(cr.calls)):          # warm-up pass over every buffer set
            run_calls(cr.calls[i % len(cr.calls)])
        samples = []
        for _ in range(3):
            us = region.time_us(lambda: [run_calls(cr.calls[i % len(cr.calls)])
                                         for i in range(passes)]) / passes
            samples.append(us)
        r = rate(cr.nbytes, cr.values, statistics.median(samples))
        r["samples_us"] = [round(t, 2) for t in samples]
        r["kernels"] = {k: {kk: v[kk] for kk in ("bytes_per_launch", "launches_per_pass",
                                                  "us_per_launch", "gbs", "frac")}
                        for k, v in time_kernels(region, cr.kernels, reps, 3).items()}
        out[cr.name] = r
        del cr
        torch.cuda.empty_cache()
    return out


MM_M, MM_N, MM_SLICES = 4096, 7168, 6      # staged projection: six 4096 x 7168 slices, N = 7168
MFMA_FP8_PEAK_TFLOPS = 5000.0               # MI355X dense fp8 matrix-core peak


def gemm_bench(torch, bq, region: Region, reps: int, warmup: int = 20) -> dict:
    """The dense MXFP8 GEMM from a staged buffer (not part of the step): six bf16 slices of
    4096 x 7168 quantized into a 4096 x 43008 staging buffer, times 7168 x 43008 MXFP8
    weights, into bf16.  Synthetic N(0, 1) inputs drawn on the GPU with a fixed seed.  Two
    scale layouts are timed on the same values: row-major E8M0 rows (bq_mm_mx) and the
    scaled-MFMA layout (bq_mm_mx_mfma), each at K = 43008 and at K = 42880, a K that is not
    a multiple of 512; samples are taken round-robin over the four, after `warmup` launches
    of each.  The headline figure is the staged layout the slice quantizer writes for the
    GEMM, the MFMA layout, at K = 43008."""
    K = MM_SLICES * COLS
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    xv = torch.empty((MM_M, K), dtype=torch.uint8, device="cuda")
    xe = torch.empty((MM_M, K // 32), dtype=torch.uint8, device="cuda")
    xl = torch.empty(bq.bq_mx_scale_mfma_bytes(MM_M, K), dtype=torch.uint8, device="cuda")
    for j in range(MM_SLICES):
        xs = torch.randn((MM_M, COLS), generator=g, device="cuda").to(torch.bfloat16)
        bq.bq_quant_mx_slice(xs, j * COLS, xv, xe)
        bq.bq_quant_mx_slice_mfma(xs, j * COLS, xv, xl)
    w = torch.randn((MM_N, K), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.empty((MM_N, K), dtype=torch.uint8, device="cuda")
    we = torch.empty((MM_N, K // 32), dtype=torch.uint8, device="cuda")
    wl = torch.empty(bq.bq_mx_scale_mfma_bytes(MM_N, K), dtype=torch.uint8, device="cuda")
    bq.bq_quant_mx(w, wv, we)
    bq.bq_quant_mx_slice_mfma(w, 0, wv, wl)
    del w
    y = torch.empty((MM_M, MM_N), dtype=torch.bfloat16, device="cuda")
    runs = {
        ("row-major", K): lambda: bq.bq_mm_mx(xv, xe, wv, we, y, K=K),
        ("mfma", K): lambda: bq.bq_mm_mx_mfma(xv, xl, wv, wl, y, K=K),
        ("row-major", K - 128): lambda: bq.bq_mm_mx(xv, xe, wv, we, y, K=K - 128),
        ("mfma", K - 128): lambda: bq.bq_mm_mx_mfma(xv, xl, wv, wl, y, K=K - 128),
    }
    for fn in runs.values():
        for _ in range(warmup):
            fn()
    samples = {key: [] for key in runs}
    for _ in range(SAMPLES):
        for key, fn in runs.items():
            samples[key].append(region.time_us(lambda fn=fn: [fn() for _ in range(reps)]) / reps)
    out = {}
    for (layout, k), ss in samples.items():
        us = statistics.median(ss)
        flops = 2.0 * MM_M * MM_N * k
        tflops = flops / (us * 1e-6) / 1e12
        out[f"{layout} K={k}"] = {"us_per_launch": round(us, 1), "achieved": round(tflops, 1),
                                  "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4),
                                  "flops_per_launch": flops,
                                  "samples_us": [round(t, 1) for t in ss]}
    head = out[f"mfma K={K}"]
    return {"workload": f"staged MXFP8 GEMM {MM_M}x{MM_N}x{K} (six 4096x7168 slices), bf16 out, "
                        "scales in the scaled-MFMA layout",
            "bound": "mfma", "us_per_launch": head["us_per_launch"], "achieved": head["achieved"],
            "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": head["frac"],
            "flops_per_launch": head["flops_per_launch"], "samples_us": head["samples_us"],
            "layouts": out}


def copy_reference(torch, region: Region, total_bytes: int, reps: int) -> dict:
    """A plain device-to-device copy (torch's) moving total_bytes per launch, half read and half
    written: the rate a kernel of that many algorithmic bytes could reach if it did nothing but
    stream them.  Timed like the step's kernels: reps back-to-back launches on the same stream
    between one pair of HIP events, sources and destinations rotating over at least 1 GiB each,
    so both are cold in the last-level cache (as the kernels' inputs and outputs are)."""
    half = total_bytes // 2
    nsrc = max(2, (1 << 30) // half + 1)
    src = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsrc)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsrc)]
    with torch.cuda.stream(region.stream):
        for i in range(3):
            dst[i % nsrc].copy_(src[i % nsrc])

        def launch():
            for i in range(reps):
                dst[(i + 3) % nsrc].copy_(src[(i + 3) % nsrc])
        us = statistics.median(region.time_us(launch) / reps for _ in range(3))
    del src, dst
    return {"bytes_per_launch": 2 * half, "us_per_launch": round(us, 2),
            "gbs": round(2 * half / (us * 1e-6) / 1e9, 1)}


def receipt(torch, bq) -> dict:
    """What the figures were measured on: software versions and the device."""
    props = torch.cuda.get_device_properties(0)
    out = {"torch": torch.__version__, "hip": torch.version.hip, "library": bq.bq_version(),
           "device": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count,
           "memory_gib": round(props.total_memory / 2 ** 30, 1)}
    uuid = getattr(props, "uuid", None)
    if uuid is not None:
        out["uuid"] = str(uuid)
    out["clocks"] = gpu_clock_levels(props)
    # the device code measured (the .hip sources and their headers, comments left out)
    out["source_digest"] = kernel_source_digest()
    return out


def gpu_clock_levels(props) -> dict | None:
    """The device's shader and memory clock levels as sysfs lists them (the level in use when
    read is marked with *), or None where they cannot be read."""
    try:
        bdf = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    except (AttributeError, TypeError, ValueError):
        return None
    out = {}
    for key in ("pp_dpm_sclk", "pp_dpm_mclk"):
        try:
            with open(f"/sys/bus/pci/devices/{bdf}/{key}") as f:
                out[key] = [line.strip() for line in f if line.strip()]
        except OSError:
            pass
    return out or None


def cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_worker(kind, bounds, repeat, barrier, out) -> None:
    """One worker of the CPU baseline: the oracle on rows [a, b) of every ring chunk /
    all-to-all shard of every rank -- the same slice of each chunk, so every block's result
    is the one the full run computes.  kind "metric": the ring's step-0 quantize and its
    three hop steps; kind "step": the whole step.  The work runs `repeat` times and the time
    per pass is reported.  Inputs are generated before the clock starts; all workers start at
    a barrier."""
    os.environ["OMP_NUM_THREADS"] = "1"
    import oracle
    import workloads
    a, b = bounds
    ch = ROWS // W
    parts = [np.concatenate([workloads.rows(2, r, c * ch + a, b - a, COLS) for c in range(W)])
             for r in range(W)]
    R = parts[0].shape[0]
    m = (b - a) * COLS
    v = np.empty((R, W * COLS), np.uint8)
    e = np.empty((R, W * COLS // 32), np.uint8)
    barrier.wait(timeout=600)
    t0 = time.perf_counter()
    for _ in range(repeat):
        _oracle_pass(kind, parts, m, v, e)
    out.put((time.perf_counter() - t0) / repeat)


def _oracle_pass(kind, parts, m, v, e) -> None:
    import oracle
    if kind == "metric":
        flat = [p.reshape(-1) for p in parts]
        wire = {}
        for r in range(W):
            c = (r - 1) % W
            wire[c] = oracle.quant_i8(flat[r][c * m:(c + 1) * m])
        for k in range(1, W):
            for r in range(W):
                c = (r - 1 - k) % W
                wire[c] = oracle.ring_hop_i8(wire[c][0], wire[c][1], flat[r][c * m:(c + 1) * m])
    else:
        oracle.ring_allreduce_i8([p.reshape(-1) for p in parts])
        oracle.a2a_allreduce_i8([p.reshape(-1) for p in parts])
        for r in range(W):
            oracle.quant_mx_slice(parts[r], COLS * r, v, e)
        oracle.dequant_mx(v, e)
        ev, es = oracle.quant_e4m3_b128(parts[0])
        oracle.dequant_e4m3_b128(ev, es)


def cpu_baseline_workers(kind: str, workers: int, repeat: int = 1) -> dict:
    """The unmodified oracle on `workers` processes (spawned children that never touch the
    GPU), the rows of each chunk split statically among them, one slice per process, the
    work repeated `repeat` times; the time per pass is the slowest worker's."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    ch = ROWS // W
    edges = [round(i * ch / workers) for i in range(workers + 1)]
    bounds = [(edges[i], edges[i + 1]) for i in range(workers) if edges[i + 1] > edges[i]]
    barrier = ctx.Barrier(len(bounds))
    out = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(kind, bd, repeat, barrier, out))
             for bd in bounds]
    for pr in procs:
        pr.start()
    times = [out.get(timeout=900) for _ in procs]
    for pr in procs:
        pr.join(timeout=60)
    return {"seconds": max(times), "workers": len(bounds), "repeat": repeat}


def host_cpu_share() -> dict:
    """Cores the CPU baseline may use: those in this process's affinity mask, at most 16 --
    a GPU host gives each of its GPUs a share of 16 cores, whatever it has online."""
    online = os.sysconf("SC_NPROCESSORS_ONLN")
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = online
    return {"online": online, "allowed": allowed, "used": max(1, min(16, allowed))}


def sweep(torch, bq, region: Region, reps: int = 20, samples: int = 3) -> list:
    """The INT8 quantize, the ring hop (single segment, out of place) and torch's device
    copy at 8 MB .. 1 GB of algorithmic bytes per launch, each timed like the step's kernels:
    `reps` back-to-back launches rotating over buffer sets of at least 1.2 GB in all, in
    `samples` samples (median).  Separates a launch's fixed cost from its streaming rate."""
    L = bq.lib
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: t.data_ptr()
    e = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
    rows = []
    for kind in ("quant_i8", "ring_hop_i8", "copy"):
        for mb in (8, 16, 32, 64, 128, 256, 512, 1024):
            per_block = {"quant_i8": B_QUANT, "ring_hop_i8": B_HOP, "copy": 512}[kind]
            nb = int(mb * 1e6 // per_block)
            n = nb * 128
            nbytes = nb * per_block
            nsets = max(2, -(-int(1.2e9) // nbytes))
            calls = []
            keep = []
            for _ in range(nsets):
                if kind == "quant_i8":
                    x = torch.randn(n, device="cuda", dtype=torch.bfloat16).view(torch.int16)
                    q, sc = e(n, torch.int8), e(nb, torch.float32)
                    keep += [x, q, sc]
                    calls.append(("quant_i8", nbytes, L.bq_quant_i8, (P(x), n, P(q), P(sc), sp)))
                elif kind == "ring_hop_i8":
                    qi = torch.randint(-127, 128, (n,), device="cuda", dtype=torch.int8)
                    si = torch.rand(nb, device="cuda", dtype=torch.float32) + 0.5
                    loc = torch.randn(n, device="cuda", dtype=torch.bfloat16).view(torch.int16)
                    qo, so = e(n, torch.int8), e(nb, torch.float32)
                    keep += [qi, si, loc, qo, so]
                    calls.append(("ring_hop_i8", nbytes, L.bq_ring_hop_i8,
                                  (P(qi), P(si), P(loc), n, P(qo), P(so), sp)))
                else:
                    src, dst = e(nbytes // 2, torch.uint8), e(nbytes // 2, torch.uint8)
                    keep += [src, dst]
                    calls.append(("copy", nbytes, None, (dst, src)))

            def launch_one(c):
                if c[2] is None:
                    c[3][0].copy_(c[3][1])
                else:
                    run_calls([c])
            for c in calls:
                launch_one(c)
            got = []
            for smp in range(samples):
                got.append(region.time_us(lambda: [launch_one(calls[i % nsets])
                                                   for i in range(reps)]) / reps)
            us = statistics.median(got)
            gbs = nbytes / (us * 1e-6) / 1e9
            row = {"kernel": kind, "bytes_per_launch": nbytes, "us_per_launch": round(us, 2),
                   "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                   "samples_us": [round(t, 2) for t in got]}
            print(json.dumps(row), flush=True)
            rows.append(row)
            del calls, keep
            torch.cuda.empty_cache()
    return rows


def summarize_trace(path: str) -> str:
    """A rocprofv3 kernel trace (CSV) as markdown: one row per kernel and launch shape
    (workgroups x segments) with its dispatch count, average / min / max duration and the
    average over its back-to-back runs (10 or more consecutive dispatches of that kernel and
    shape: the per-kernel samples); then the metric's passes (the INT8 quantize of 1344 x 4
    workgroups followed by three ring hops of the same shape) with the average duration of
    each of the four launches."""
    import csv
    import re
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            m = re.search(r"(k_\w+<[^>]*>)", name)
            short = m.group(1) if m else name[:40]
            wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                         (short, wg, int(r["Grid_Size_Y"]))))
    rows.sort()
    keys = [k for _, _, k in rows]
    dur = [(e - s) / 1e3 for s, e, _ in rows]
    groups, runs = {}, {}
    for k, d in zip(keys, dur):
        groups.setdefault(k, []).append(d)
    i = 0
    while i < len(keys):
        j = i
        while j + 1 < len(keys) and keys[j + 1] == keys[i]:
            j += 1
        if j - i + 1 >= 10:
            runs.setdefault(keys[i], []).extend(dur[i:j + 1])
        i = j + 1
    total = sum(dur)
    lines = ["| kernel | workgroups x segments | dispatches | avg us | min us | max us | "
             "back-to-back avg us | share of GPU time |", "|---|---|---|---|---|---|---|---|"]
    for k, ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        b2b = f"{statistics.mean(runs[k]):.2f}" if k in runs else ""
        lines.append(f"| `{k[0]}` | {k[1]} x {k[2]} | {len(ds)} | {statistics.mean(ds):.2f} | "
                     f"{min(ds):.2f} | {max(ds):.2f} | {b2b} | {100 * sum(ds) / total:.1f}% |")
    def is_quant(k):
        return k[0].startswith("k_quant_i8<") and k[1:] == (1344, 4)
    h = ("k_ring_hop_i8<1>", 1344, 4)
    pos = [[], [], [], []]
    for i in range(len(keys) - 3):
        if is_quant(keys[i]) and keys[i + 1] == h and keys[i + 2] == h and keys[i + 3] == h:
            for p in range(4):
                pos[p].append(dur[i + p])
    if pos[0]:
        lines += ["", f"Metric passes (quantize, hop 1, hop 2, hop 3): {len(pos[0])}; average us "
                      f"{', '.join(f'{statistics.mean(p):.2f}' for p in pos)}; hop average "
                      f"{statistics.mean(pos[1] + pos[2] + pos[3]):.2f}; pass "
                      f"{sum(statistics.mean(p) for p in pos):.2f}"]
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the five workload configurations at full size")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the quantize, the hop and a copy from 8 MB to 1 GB per launch")
    ap.add_argument("--gemm", action="store_true",
                    help="only time the staged MXFP8 GEMM (--steps launches per sample, at most 4; "
                         "--warmup launches of each layout first)")
    ap.add_argument("--config", choices=CONFIGS,
                    help="only time one workload configuration at full size")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print a rocprofv3 kernel trace as a table and exit (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not "
              "supported (a simulated rank is a separate HBM buffer on the one GPU)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30}))
        return 0

    import block_quantized_wire_amd as bq
    region = Region(torch, torch.cuda.current_stream())
    if args.sweep:
        sweep(torch, bq, region)
        return 0
    if args.gemm:
        print(json.dumps({"gemm": gemm_bench(torch, bq, region, reps=max(1, min(4, args.steps)),
                                             warmup=args.warmup)}), flush=True)
        return 0
    if args.config:
        print(json.dumps({"configs": config_bench(torch, bq, region, torch.cuda.current_stream(),
                                                  CONFIG_PASSES, REPS, [args.config])}), flush=True)
        return 0
    step = Step(torch, bq, SETS)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step.run(i)
        step.run_metric(i)
    torch.cuda.synchronize()
    K = args.steps

    # timed region 1: K whole steps
    ms = region.time_us(lambda: [step.run(i) for i in range(K)]) / 1e3 / K
    step_gbs = step.step_bytes / (ms * 1e-3) / 1e9

    # the metric's own region: K passes of the ring's step-0 quantize and three hop steps,
    # in SAMPLES samples (median)
    metric_us = [region.time_us(lambda: [step.run_metric(i) for i in range(K)]) / K
                 for _ in range(SAMPLES)]
    metric = rate(step.metric_bytes, W * N, statistics.median(metric_us))

    # each distinct kernel of the step alone: REPS back-to-back launches per sample
    per = time_kernels(region, step.kernels, REPS, SAMPLES)
    for seq in step.next_kernels:           # the MXFP8 ring / all-to-all primitives
        run_calls(seq)
    per_next = time_kernels(region, step.next_kernels, REPS, SAMPLES)
    per_share = time_kernels(region, step.share_kernels, REPS, SAMPLES)
    # the roofline's kernel: the metric pass's kernel with the most time per pass, timed
    # alone with every input cold (events between launches inside the metric's region
    # would add about 2.7 us per launch, a sixth of a hop)
    metric_kernels = {f"{n} ({b} B)" for n, b, _, _ in step.metric[0]}
    dom_name = max(metric_kernels, key=lambda k: per[k]["us_per_pass"])
    dom = per[dom_name]
    copy_ref = copy_reference(torch, region, dom["bytes_per_launch"], REPS)

    # accuracy on input set 0, outside the timed regions: the all-reduce outputs against
    # the exact (fp64) sum of the bf16 partials, the codec round trips against their input
    step.run(0)
    torch.cuda.synchronize()
    f64 = lambda t: t.view(torch.bfloat16).double().reshape(-1)
    b0 = step.sets[0]
    exact = sum(f64(p) for p in b0["parts"])

    def err(got, ref):
        d = (got - ref).abs()
        return {"max_abs": float(d.max()), "rms": float(d.pow(2).mean().sqrt())}

    mx_in = torch.cat([p.view(ROWS, COLS) for p in b0["parts"]], dim=1)
    bq.bq_ring_allreduce_mx(b0["parts"], b0["mxw_v"], b0["mxw_e"], b0["mxr_out"], n=N)
    bq.bq_a2a_allreduce_mx(b0["parts"], b0["mx_send_v"], b0["mx_send_e"], None, b0["mx_bc_v"],
                           b0["mx_bc_e"], b0["mxa_out"], n=N)
    torch.cuda.synchronize()
    accuracy = {
        "i8_ring_vs_fp64_sum": err(f64(b0["ring_out"][0]), exact),
        "i8_a2a_vs_fp64_sum": err(f64(b0["a2a_out"][0]), exact),
        "mx_ring_vs_fp64_sum": err(f64(b0["mxr_out"][0]), exact),
        "mx_a2a_vs_fp64_sum": err(f64(b0["mxa_out"][0]), exact),
        "mxfp8_roundtrip": err(f64(b0["mx_y"].contiguous()), f64(mx_in.contiguous())),
        "e4m3_b128_roundtrip": err(f64(b0["e4_y"]), f64(b0["parts"][0])),
        "ranks_bit_identical": all(torch.equal(b0["ring_out"][0], o) for o in b0["ring_out"]) and
        all(torch.equal(b0["a2a_out"][0], o) for o in b0["a2a_out"]) and
        all(torch.equal(b0["mxr_out"][0], o) for o in b0["mxr_out"]) and
        all(torch.equal(b0["mxa_out"][0], o) for o in b0["mxa_out"]),
    }
    del exact, mx_in

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        if t.get("source_digest") == kernel_source_digest() and dom_name in t.get("kernels", {}):
            traffic = t["kernels"][dom_name]

    line = {
        "metric": METRIC,
        "value": metric["gbs"],
        "unit": "GB/s",
        "pct_of_peak": round(100 * metric["frac"], 2),
        "elements_per_s": metric["elements_per_s"],
        "elements_pct_of_peak": round(100 * metric["elements_frac"], 2),
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "i8 quant + ring hop at 3072x7168 bf16: the block-INT8 quantize "
                               "of the ring's step-0 chunks (4 ranks x 768x7168, one launch) "
                               "then the three 4-rank fused ring-hop steps (4 x 768x7168 each), "
                               "over 4 simulated ranks' N(0,0.5) partials of 3072x7168",
                   "ranks": W, "rows": ROWS, "cols": COLS, "input_sets": SETS},
        # `value`: K passes of the metric's kernels back to back, SAMPLES samples (median)
        "value_region": dict(metric, passes_per_sample=K,
                             samples_us=[round(t, 2) for t in metric_us],
                             values_counted="3072x7168 values quantized + 3 x 3072x7168 values "
                                            "hopped per pass"),
        # the whole step (every row of the hot path), timed region 1
        "step": {"workload": "4 simulated ranks x 3072x7168 bf16 partials, N(0,0.5): i8_ring + "
                             "i8_a2a all-reduce, MXFP8 staged slices + dequant, E4M3-b128 codec",
                 "ms": round(ms, 4), "bytes": step.step_bytes, "gbs": round(step_gbs, 1),
                 "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": dom["gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom["frac"],
                     "bytes_per_launch": dom["bytes_per_launch"],
                     "us_per_launch": dom["us_per_launch"],
                     "launches_per_pass": dom["launches_per_pass"],
                     "timed": "the kernel alone: REPS back-to-back launches over 16 buffer sets "
                              "(every input cold), SAMPLES samples, median",
                     "traffic": traffic,
                     # a plain device copy of the same bytes per launch, timed the same way
                     "copy_same_bytes": dict(copy_ref, kernel_over_copy=round(
                         dom["gbs"] / copy_ref["gbs"], 3))},
        "kernels": {k: {kk: v[kk] for kk in ("bytes_per_launch", "launches_per_pass",
                                             "us_per_launch", "gbs", "frac", "samples_us")}
                    for k, v in per.items()},
        # the MXFP8 ring / all-to-all primitives at the same shapes, timed the same way;
        # not part of the step and not in `value`
        "next_kernels": {k: {kk: v[kk] for kk in ("bytes_per_launch", "launches_per_pass",
                                                  "us_per_launch", "gbs", "frac", "samples_us")}
                         for k, v in per_next.items()},
        # one TP4 rank's share, 768x7168, as single-segment launches timed the same way
        # (context: a launch this small pays its fixed start-up cost on 22 MB)
        "share_kernels": {k: {kk: v[kk] for kk in ("bytes_per_launch", "us_per_launch", "gbs",
                                                   "frac", "samples_us")}
                          for k, v in per_share.items()},
    }
    line["accuracy"] = accuracy
    line["receipt"] = receipt(torch, bq)
    step_bytes = step.step_bytes
    del step
    torch.cuda.empty_cache()
    if not args.no_configs:
        line["configs"] = config_bench(torch, bq, region, torch.cuda.current_stream(),
                                       CONFIG_PASSES, REPS)
    line["gemm"] = gemm_bench(torch, bq, region, reps=4)
    if not args.no_cpu_baseline:
        share = host_cpu_share()
        # repeats sized for about 10-20 s of CPU work in each of the three samples
        ca = cpu_baseline_workers("metric", share["used"], repeat=20)
        c1 = cpu_baseline_workers("metric", 1, repeat=15)
        cs = cpu_baseline_workers("step", share["used"])
        mb = line["value_region"]["bytes_per_pass"]
        line["cpu_baseline"] = {
            "value": round(mb / ca["seconds"] / 1e9, 4), "unit": "GB/s", "cores": ca["workers"],
            "kind": "oracle", "cpu": cpu_model(), "host_cores": share,
            "sample": f"the metric's whole pass (the step-0 quantize and three hop steps, all "
                      f"{ROWS} rows of every rank), the rows of each chunk split over "
                      f"{ca['workers']} processes, {ca['repeat']} passes "
                      f"({ca['seconds']:.3f} s per pass)",
            "one_core": {"value": round(mb / c1["seconds"] / 1e9, 4), "cores": 1,
                         "sample": f"the same pass in one process, {c1['repeat']} passes "
                                   f"({c1['seconds']:.2f} s per pass)"},
            "step": {"value": round(step_bytes / cs["seconds"] / 1e9, 4),
                     "cores": cs["workers"],
                     "sample": f"the whole step, rows split over {cs['workers']} processes "
                               f"({cs['seconds']:.2f} s)"}}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
