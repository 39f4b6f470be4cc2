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
`value` is the algorithmic bytes of the step (each kernel's inputs read once and
outputs written once; the four ranks' materialization reads its one shared payload
once) over the step time, in GB/s; HBM peak is 8 TB/s.  Inputs are resident in HBM.
Four complete buffer sets (inputs, intermediates, outputs; about 1 GB each) rotate
step by step, so a step's inputs are cold in the 256 MB last-level cache while what
a kernel consumes from the previous kernel of the same step may be served by it, as
in any pipeline on one GPU.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
SETS = 4                   # rotating buffer sets, each a full step's inputs and outputs (~1 GB)
SAMPLES = 5                # timed samples per kernel in timed region 2 (median reported)

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
    """Digest of the device code (the .hip sources and the headers they include, comments
    left out): the HBM counters in profiles/ stay valid while it is unchanged; host-side
    validation and comments may change."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_wire_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h")):
            continue
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
            b = {"parts": [torch.from_numpy(workloads.rows(2, r + 16 * k, 0, ROWS, COLS)
                                            .view(np.int16)).to(dev) for r in range(W)]}
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
        self.calls, self.kernels, self.next_kernels = [], [], []
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
            self.calls.append(calls)
            self.kernels.append(kern)
            self.next_kernels.append(nxt)
        assert sum(c[1] for c in self.calls[0]) == sum(k[1] for k in self.kernels[0])

    @property
    def step_bytes(self) -> int:
        return sum(c[1] for c in self.calls[0])

    def run(self, i: int) -> None:
        for name, _, fn, args in self.calls[i % len(self.calls)]:
            st = fn(*args)
            if st != 0:
                raise RuntimeError(f"{name}: status {st} ({self.bq.bq_status_str(st)})")

    def run_kernels(self, i: int, events) -> None:
        for k, (name, _, fn, args) in enumerate(self.kernels[i % len(self.kernels)]):
            events[k][0].record(self.stream)
            st = fn(*args)
            events[k][1].record(self.stream)
            if st != 0:
                raise RuntimeError(f"{name}: status {st} ({self.bq.bq_status_str(st)})")


MM_M, MM_N, MM_SLICES = 4096, 7168, 6      # staged projection: six 4096 x 7168 slices, N = 7168
MFMA_FP8_PEAK_TFLOPS = 5000.0               # MI355X dense fp8 matrix-core peak


def gemm_bench(torch, bq, reps: int, warmup: int = 2) -> dict:
    """The dense MXFP8 GEMM from a staged buffer (not part of the step): six bf16 slices
    of 4096 x 7168 quantized into a 4096 x 43008 staging buffer, times 7168 x 43008 MXFP8
    weights, into bf16.  Synthetic N(0, 1) inputs drawn on the GPU with a fixed seed."""
    K = MM_SLICES * COLS
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    xv = torch.empty((MM_M, K), dtype=torch.uint8, device="cuda")
    xe = torch.empty((MM_M, K // 32), dtype=torch.uint8, device="cuda")
    for j in range(MM_SLICES):
        xs = torch.randn((MM_M, COLS), generator=g, device="cuda").to(torch.bfloat16)
        bq.bq_quant_mx_slice(xs, j * COLS, xv, xe)
    w = torch.randn((MM_N, K), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.empty((MM_N, K), dtype=torch.uint8, device="cuda")
    we = torch.empty((MM_N, K // 32), dtype=torch.uint8, device="cuda")
    bq.bq_quant_mx(w, wv, we)
    del w
    y = torch.empty((MM_M, MM_N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        bq.bq_mm_mx(xv, xe, wv, we, y)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    samples = []
    for _ in range(SAMPLES):
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            bq.bq_mm_mx(xv, xe, wv, we, y)
        e1.record(stream)
        torch.cuda.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e3 / reps)
    us = statistics.median(samples)
    flops = 2.0 * MM_M * MM_N * K
    tflops = flops / (us * 1e-6) / 1e12
    return {"workload": f"staged MXFP8 GEMM {MM_M}x{MM_N}x{K} (six 4096x7168 slices), bf16 out",
            "bound": "mfma", "us_per_launch": round(us, 1), "achieved": round(tflops, 1),
            "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4),
            "flops_per_launch": flops, "samples_us": [round(t, 1) for t in samples]}


def copy_reference(torch, stream, total_bytes: int, reps: int) -> dict:
    """A plain device-to-device copy (torch's) moving total_bytes per launch, half read and half
    written: the rate a kernel of that many algorithmic bytes could reach if it did nothing but
    stream them.  Timed like the step's kernels: reps back-to-back launches on the same stream
    between one pair of HIP events, the sources rotating over at least 1 GiB so they are cold in
    the last-level cache."""
    half = total_bytes // 2
    nsrc = max(2, (1 << 30) // half + 1)
    src = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsrc)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(2)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(3):
            dst[i % 2].copy_(src[i % nsrc])
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            dst[i % 2].copy_(src[(i + 3) % nsrc])
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
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


def cpu_baseline(rows_per_rank: int) -> dict:
    """The oracle, single-threaded, on the first `rows_per_rank` rows of every rank."""
    import oracle
    import workloads
    R = rows_per_rank
    parts = [workloads.rows(2, r, 0, R, COLS) for r in range(W)]
    t0 = time.perf_counter()
    oracle.ring_allreduce_i8([p.reshape(-1) for p in parts])
    oracle.a2a_allreduce_i8([p.reshape(-1) for p in parts])
    v = np.empty((R, W * COLS), np.uint8)
    e = np.empty((R, W * COLS // 32), np.uint8)
    for r in range(W):
        oracle.quant_mx_slice(parts[r], COLS * r, v, e)
    oracle.dequant_mx(v, e)
    ev, es = oracle.quant_e4m3_b128(parts[0])
    oracle.dequant_e4m3_b128(ev, es)
    dt = time.perf_counter() - t0
    frac = R / ROWS
    return {"seconds": dt, "frac": frac}


def _oracle_slice(bounds, barrier, out) -> None:
    """One worker of the all-core CPU baseline: the step's oracle work on rows
    [a, b) of every ring chunk / all-to-all shard of every rank -- the same slice of each
    chunk, so every block's result is the one the full run computes.  Inputs are
    generated before the clock starts; all workers start at a barrier."""
    os.environ["OMP_NUM_THREADS"] = "1"
    import oracle
    import workloads
    a, b = bounds
    ch = ROWS // W
    parts = [np.concatenate([workloads.rows(2, r, c * ch + a, b - a, COLS) for c in range(W)])
             for r in range(W)]
    R = parts[0].shape[0]
    v = np.empty((R, W * COLS), np.uint8)
    e = np.empty((R, W * COLS // 32), np.uint8)
    barrier.wait(timeout=600)
    t0 = time.perf_counter()
    oracle.ring_allreduce_i8([p.reshape(-1) for p in parts])
    oracle.a2a_allreduce_i8([p.reshape(-1) for p in parts])
    for r in range(W):
        oracle.quant_mx_slice(parts[r], COLS * r, v, e)
    oracle.dequant_mx(v, e)
    ev, es = oracle.quant_e4m3_b128(parts[0])
    oracle.dequant_e4m3_b128(ev, es)
    out.put(time.perf_counter() - t0)


def cpu_baseline_all_cores(workers: int) -> dict:
    """The unmodified oracle on `workers` processes (spawned children that never touch the
    GPU), the rows of each chunk split statically among them, one slice per process."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    ch = ROWS // W
    edges = [round(i * ch / workers) for i in range(workers + 1)]
    bounds = [(edges[i], edges[i + 1]) for i in range(workers) if edges[i + 1] > edges[i]]
    barrier = ctx.Barrier(len(bounds))
    out = ctx.Queue()
    procs = [ctx.Process(target=_oracle_slice, args=(bd, barrier, out)) for bd in bounds]
    for pr in procs:
        pr.start()
    times = [out.get(timeout=900) for _ in procs]
    for pr in procs:
        pr.join(timeout=60)
    return {"seconds": max(times), "workers": len(bounds)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3072,
                    help="rows per rank of the CPU-baseline sample (multiple of 4)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
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
    step = Step(torch, bq, SETS)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step.run(i)
    torch.cuda.synchronize()

    # timed region 1: the whole step, eager launches, no per-kernel events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(step.stream)
    for i in range(args.steps):
        step.run(i)
    t1.record(step.stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    step_gbs = step.step_bytes / (ms * 1e-3) / 1e9

    # timed region 2: each distinct kernel of the step alone, R back-to-back launches
    # rotating over the buffer sets (inputs and outputs: consecutive launches share no
    # buffer, so inputs are cold in the last-level cache) between one pair of HIP events
    # on the launch stream -- no event sits between two launches, so the average is
    # the kernel's own duration as a trace shows it.  SAMPLES such samples per kernel,
    # taken round-robin over the kernels; the figure is their median.
    reps = max(10, args.steps // 4)

    def time_kinds(seqs):
        kinds = {}
        for k, (name, nbytes, _, _) in enumerate(seqs[0]):
            kinds.setdefault((name, nbytes), []).append(k)
        samples = {key: [] for key in kinds}
        for smp in range(SAMPLES):
            for (name, nbytes), idx in kinds.items():
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(step.stream)
                for i in range(smp * reps, (smp + 1) * reps):
                    _, _, fn, fargs = seqs[i % len(seqs)][idx[i % len(idx)]]
                    st = fn(*fargs)
                    if st != 0:
                        raise RuntimeError(f"{name}: status {st}")
                e1.record(step.stream)
                torch.cuda.synchronize()
                samples[(name, nbytes)].append(e0.elapsed_time(e1) * 1e3 / reps)
        out = {}
        for (name, nbytes), idx in kinds.items():
            us = statistics.median(samples[(name, nbytes)])
            gbs = nbytes / (us * 1e-6) / 1e9
            out[f"{name} ({nbytes} B)"] = {"bytes_per_launch": nbytes, "launches_per_step": len(idx),
                                           "us_per_launch": us, "gbs": gbs,
                                           "frac": gbs / HBM_PEAK_GBS, "us_per_step": us * len(idx),
                                           "samples_us": [round(t, 2) for t in samples[(name, nbytes)]]}
        return out

    per = time_kinds(step.kernels)
    # the MXFP8 ring and all-to-all primitives (not part of the step), after a warmup pass
    for seq in step.next_kernels:
        for name, _, fn, fargs in seq:
            if fn(*fargs) != 0:
                raise RuntimeError(f"{name}: warmup failed")
    per_next = time_kinds(step.next_kernels)
    dom_name = max(per, key=lambda k: per[k]["us_per_step"])
    dom = per[dom_name]
    copy_ref = copy_reference(torch, step.stream, dom["bytes_per_launch"], max(reps, 20))

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
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "4 simulated ranks x 3072x7168 bf16 partials, N(0,0.5): i8_ring "
                               "+ i8_a2a all-reduce, MXFP8 staged slices + dequant, E4M3-b128 codec",
                   "ranks": W, "rows": ROWS, "cols": COLS, "input_sets": SETS,
                   "step_bytes": step.step_bytes},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom["gbs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom["frac"], 4),
                     "bytes_per_launch": dom["bytes_per_launch"],
                     "us_per_launch": round(dom["us_per_launch"], 2),
                     "traffic": traffic,
                     # a plain device copy of the same bytes per launch, timed the same way
                     "copy_same_bytes": dict(copy_ref, kernel_over_copy=round(
                         dom["gbs"] / copy_ref["gbs"], 3))},
        "kernels": {k: {"bytes_per_launch": v["bytes_per_launch"],
                        "launches_per_step": v["launches_per_step"],
                        "us_per_launch": round(v["us_per_launch"], 2), "gbs": round(v["gbs"], 1),
                        "frac": round(v["frac"], 4), "samples_us": v["samples_us"]}
                    for k, v in per.items()},
        # the MXFP8 ring / all-to-all primitives at the same shapes, timed the same way;
        # not part of the step and not in `value`
        "next_kernels": {k: {"bytes_per_launch": v["bytes_per_launch"],
                             "launches_per_pass": v["launches_per_step"],
                             "us_per_launch": round(v["us_per_launch"], 2),
                             "gbs": round(v["gbs"], 1), "frac": round(v["frac"], 4),
                             "samples_us": v["samples_us"]}
                         for k, v in per_next.items()},
    }
    line["accuracy"] = accuracy
    line["receipt"] = receipt(torch, bq)
    line["gemm"] = gemm_bench(torch, bq, reps=4, warmup=20)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args.cpu_rows)
        cpu_gbs = step.step_bytes * cb["frac"] / cb["seconds"] / 1e9
        nw = max(1, min(16, os.cpu_count() or 1))
        ca = cpu_baseline_all_cores(nw)
        all_gbs = step.step_bytes / ca["seconds"] / 1e9
        line["cpu_baseline"] = {"value": round(all_gbs, 4), "unit": "GB/s", "cores": ca["workers"],
                                "kind": "oracle", "cpu": cpu_model(),
                                "sample": f"the whole step (all {ROWS} rows of every rank), the rows "
                                          f"of each chunk split over {ca['workers']} processes "
                                          f"({ca['seconds']:.2f} s)",
                                "one_core": {"value": round(cpu_gbs, 4), "cores": 1,
                                             "sample": f"the same step on the first {args.cpu_rows} "
                                                       f"of {ROWS} rows of every rank, one process "
                                                       f"({cb['seconds']:.1f} s)"}}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
