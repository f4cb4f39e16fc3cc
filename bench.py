#!/usr/bin/env python3
"""Benchmark of the VSA hot path on one MI355X.

A step is one pass of the whole path over the Wan2.2-A14B-shaped input
(q, k, v (1, 39936, 40, 128) bf16 after tiling; grid 21x30x52; 624 cubes):
  tile(q), tile(k), tile(v) -> select (pool, scores, top-78) -> fwd -> untile(out).
Inputs are resident in HBM before timing. Each kernel group is bracketed by
events on the stream the library launches on (torch's current stream).

The headline figure is the fine forward (vsa_fwd): kernel-only, warmed,
effective TFLOP/s = 4 * D * 64 * sum over (b, h, query cube) of the real
tokens of the selected cubes, divided by its mean launch time. The same
kernel is also timed at topk = all (dense) and over the sparsity sweep
topk in {624, 312, 187, 78, 31}. Further legs on the same tensors: the
lookup-table path (cumulative-mass selector + vsa_fwd_lut with its row
statistics), the two-stage path (coarse output, gated combine), the fine
kernel in Hilbert cube order, and the block mask -> LUT compaction; then the
whole path on the 720p HunyuanVideo-like workload. The Wan step is also
timed back to back, eagerly and replayed as one captured HIP graph. Context
measured in the same run: the engine clock during the timed vsa_fwd loop (a
shader-cycle meter on a second stream, in a repeat of the loop), and two bf16
ceilings of this part, a bounded MFMA-only loop on random operands and a
large hipBLASLt GEMM. The CPU oracle is timed on a bounded sample of the same
workload, in one process per core, as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-hy720] [--no-cpu]
       python bench.py --fwd-only [--fwd-workload wan|hy720] ...   (profiler mode: vsa_fwd
           launches, a 1 GiB copy that calibrates the HBM counters, LDS conflict controls)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, AMD's published figure
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
CPU_PROCS_MAX = 16          # host cores a one-GPU share of the box provides


def code_digest(path: str) -> str:
    """SHA-256 of a C++/HIP source with its comments removed and every run of
    whitespace folded to one space: it changes with the code, not with the
    comments."""
    import hashlib
    import re

    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def profiled_traffic() -> float | None:
    """HBM bytes per vsa_fwd launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated against a 1 GiB copy), or None when the
    fine kernel's code has changed since those counters were taken."""
    prof = os.path.join(ROOT, "profiles", "fwd_kernel_wan.md")
    src = os.path.join(ROOT, "video_dit_block_amd", "csrc", "fwd.hip")
    try:
        fields = dict(line.split(": ", 1) for line in open(prof).read().splitlines()
                      if line.split(": ", 1)[0] in ("fwd_code_sha256", "fetch_bytes_per_launch",
                                                    "write_bytes_per_launch"))
        digest = code_digest(src)
    except (OSError, ValueError):
        return None
    if fields.get("fwd_code_sha256") != digest:
        return None
    return float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"])


def fwd_flops(topk_idx: np.ndarray, vbs: np.ndarray, D: int) -> float:
    """4 * D * (64 query rows) * (real selected KV tokens), summed over units."""
    sel_tokens = vbs[topk_idx].astype(np.int64).sum()
    return 4.0 * D * 64.0 * float(sel_tokens)


def fwd_flops_real_q(topk_idx: np.ndarray, vbs: np.ndarray, D: int) -> float:
    """The stricter count: only the real rows of each query cube,
    4 * D * vbs[c] * (real selected KV tokens), summed over units (Nq = Nkv)."""
    sel = vbs[topk_idx].astype(np.int64).sum(axis=-1)          # (B, NH, Nq)
    return 4.0 * D * float((sel * vbs[None, None, :].astype(np.int64)).sum())


def lut_flops(kv_block_idx: np.ndarray, counts: np.ndarray, vbs: np.ndarray, D: int) -> float:
    """fwd_flops over the first counts[b, h, c] ids of each row."""
    used = np.arange(kv_block_idx.shape[-1]) < counts[..., None]
    sel_tokens = (vbs[kv_block_idx].astype(np.int64) * used).sum()
    return 4.0 * D * 64.0 * float(sel_tokens)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--fwd-reps", type=int, default=50,
                    help="extra back-to-back vsa_fwd launches timed for the kernel figure")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the topk sweep {624, 312, 187, 78, 31}")
    ap.add_argument("--no-hy720", action="store_true",
                    help="skip the whole path on the 720p HunyuanVideo-like workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cdf-tau", type=float, default=0.9,
                    help="threshold of the cumulative-mass selector leg")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="fine-stage oracle seconds per CPU worker process")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time only vsa_fwd launches (for profiler runs)")
    ap.add_argument("--fwd-workload", choices=("wan", "hy720"), default="wan",
                    help="workload of the --fwd-only launches")
    return ap.parse_args()


_CPU_CASE = None  # the workload, inherited by the forked CPU workers


def _cpu_worker(job):
    """One CPU worker (one BLAS thread): tile head h with the oracle, time the
    oracle's selector on it, then the oracle's fine stage over the head's
    query cubes in order until `seconds` of fine-stage time."""
    import threadpoolctl

    import oracle

    h, seconds = job
    case = _CPU_CASE
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        tiled = [oracle.tile(x[:, :, h:h + 1], case.T, case.H, case.W) for x in (case.q, case.k,
                                                                               case.v)]
        vbs = tiled[0][1]
        q64, k64, v64 = (oracle.decode_bf16(t[0]) for t in tiled)
        t1 = time.perf_counter()
        idx, _ = oracle.select(q64, k64, vbs, case.topk)
        t2 = time.perf_counter()
        units, flops = 0, 0.0
        while units < vbs.size and time.perf_counter() - t2 < seconds:
            oracle.fwd_unit(q64, k64, v64, idx, vbs, 0, 0, units)
            flops += fwd_flops(idx[0, 0, units:units + 1], vbs, case.D)
            units += 1
        t3 = time.perf_counter()
    return {"head": h, "tile_s": t1 - t0, "select_s": t2 - t1, "fwd_s": t3 - t2,
            "units": units, "flops": flops, "head_flops": fwd_flops(idx, vbs, case.D)}


def cpu_baseline(case, seconds: float) -> dict:
    """The CPU oracle (as it stands, never tuned) on a bounded sample of the
    workload: one worker process per host core (at most CPU_PROCS_MAX), one
    BLAS thread each, each on its own head: the oracle's selector on the whole
    head, then the oracle's fine stage over that head's first query cubes for
    `seconds`. Reported in the metric's unit (effective TFLOP/s of the fine
    stage, all workers together), with the single-process rate, the
    whole-workload times extrapolated from the sample, and the CPU model.
    Runs before anything touches the GPU (the workers are forked)."""
    import multiprocessing as mp

    global _CPU_CASE
    _CPU_CASE = case
    procs = max(1, min(CPU_PROCS_MAX, len(os.sched_getaffinity(0)), case.NH))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(procs) as pool:
        res = pool.map(_cpu_worker, [(h, seconds) for h in range(procs)])
    wall = time.perf_counter() - t0
    model = "unknown"
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                     if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    rate_each = [r["flops"] / r["fwd_s"] for r in res]      # FLOP/s per process
    agg = float(sum(rate_each))
    whole_flops = float(np.mean([r["head_flops"] for r in res])) * case.NH
    sel_head = float(np.mean([r["select_s"] for r in res]))
    n_cubes = -(-case.T // 4) * -(-case.H // 4) * -(-case.W // 4)
    lo, hi = min(r["units"] for r in res), max(r["units"] for r in res)
    units_label = (f"all {n_cubes} query cubes of each head" if lo == hi == n_cubes
                   else f"{lo} to {hi} of the head's {n_cubes} query cubes")
    return {
        "value": agg / 1e12,
        "unit": "TFLOP/s",
        "cores": procs,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle: {procs} worker processes (1 BLAS thread each) on "
                   f"heads 0..{procs - 1} of the Wan workload; per worker the oracle selector "
                   f"(top-{case.topk}) on its whole head, then the fine stage on its query "
                   f"cubes in order for at most {seconds:.0f} s ({units_label}); "
                   f"{sum(r['units'] for r in res)} of {case.NH * n_cubes} units in all, "
                   f"{sum(r['fwd_s'] for r in res):.1f} s of fine-stage CPU time, "
                   f"{wall:.1f} s wall"),
        "cpu_model": model,
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "blas_threads_per_process": 1,
        "single_process_tflops": round(float(np.median(rate_each)) / 1e12, 5),
        "fwd_whole_workload_s_extrapolated": {
            "single_process": round(whole_flops / float(np.median(rate_each)), 1),
            f"{procs}_processes": round(whole_flops / agg, 1)},
        "selector_s_per_head": round(sel_head, 3),
        "selector_whole_workload_s_extrapolated": {
            "single_process": round(sel_head * case.NH, 2),
            f"{procs}_processes": round(sel_head * case.NH / procs, 2)},
    }


class ClockMeter:
    """The engine clock while a loop runs: libvsa_probe.so's meter, one
    one-wave workgroup per XCD on a second stream (default priority) for a
    fixed span of the 100 MHz real-time counter, counting shader cycles
    (s_memtime) meanwhile. Started just before the loop, with a span that
    ends within it. The meter's waves hold a few slots of 8 CUs, so each loop
    is timed without it and then repeated once with it for the clock."""

    def __init__(self, torch, dev):
        import ctypes

        self.torch = torch
        self.lib = ctypes.CDLL(os.path.join(ROOT, "video_dit_block_amd", "libvsa_probe.so"))
        self.lib.vsa_probe_clock.restype = ctypes.c_int32
        self.lib.vsa_probe_clock.argtypes = [ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p,
                                             ctypes.c_void_p]
        self.slots = 8
        self.buf = torch.zeros(2 * self.slots, dtype=torch.int64, device=dev)
        self.stream = torch.cuda.Stream(device=dev)

    def start(self, span_ms: float):
        self.span_ms = span_ms
        self.stream.wait_stream(self.torch.cuda.current_stream())
        st = self.lib.vsa_probe_clock(self.slots, int(span_ms * 1e5), self.buf.data_ptr(),
                                      self.stream.cuda_stream)
        assert st == 0, st

    def stop(self) -> dict:
        self.torch.cuda.synchronize()
        v = self.buf.cpu().numpy().reshape(self.slots, 2).astype(np.float64)
        mhz = v[:, 0] / v[:, 1] * 100.0
        return {"source": "shader cycle counter (s_memtime) over the 100 MHz real-time counter, "
                          f"one one-wave workgroup per XCD on a second stream, {self.span_ms:.0f} "
                          "ms inside a repeat of the timed loop",
                "mean_mhz": round(float(mhz.mean()), 1), "min_mhz": round(float(mhz.min()), 1),
                "max_mhz": round(float(mhz.max()), 1)}


def bf16_ceilings(torch, dev, clock) -> dict:
    """Measured bf16 rates of this part, context for the fine kernel's: a
    bounded MFMA-only loop on random operands (libvsa_probe.so, about 0.5 s),
    the same loop carrying the fine kernel's vector work at its occupancy, and
    torch.matmul bf16 at 16384^3 (hipBLASLt), each timed with events after a
    warm-up long enough for the clock to settle."""
    import ctypes

    out = {}
    lib = ctypes.CDLL(os.path.join(ROOT, "video_dit_block_amd", "libvsa_probe.so"))
    lib.vsa_probe_mfma.restype = ctypes.c_int32
    lib.vsa_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.vsa_probe_mfma_flop.restype = ctypes.c_double
    lib.vsa_probe_mfma_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    slots, blocks, iters = 64, 1024, 4000
    gen = torch.Generator(device=dev).manual_seed(11)
    src = torch.randn((slots, 16384), generator=gen, device=dev).to(torch.bfloat16)
    res = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    run = lambda: lib.vsa_probe_mfma(src.data_ptr(), slots, blocks, iters, res.data_ptr(),
                                     stream)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(8):                     # about 0.1 s: the clock settles
        assert run() == 0
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(20):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 20
    clock.start(span_ms=100.0)            # the same loop again, for its clock only
    for _ in range(20):
        run()
    out["mfma_loop_clock"] = clock.stop()
    out["mfma_loop_tflops"] = round(lib.vsa_probe_mfma_flop(blocks, iters) / ms / 1e9, 1)
    out["mfma_loop"] = ("v_mfma_f32_32x32x16_bf16 on random bf16 operands read from LDS, "
                        "4 waves per workgroup, 4 workgroups per CU, 1024 workgroups")
    # the same MFMAs with the fine kernel's vector work and occupancy
    lib.vsa_probe_mfma_mix.restype = ctypes.c_int32
    lib.vsa_probe_mfma_mix.argtypes = lib.vsa_probe_mfma.argtypes
    lib.vsa_probe_mfma_mix_flop.restype = ctypes.c_double
    lib.vsa_probe_mfma_mix_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    mblocks = 2048
    mres = torch.empty(mblocks * 128, dtype=torch.float32, device=dev)
    mrun = lambda: lib.vsa_probe_mfma_mix(src.data_ptr(), slots, mblocks, iters, mres.data_ptr(),
                                          stream)
    for _ in range(8):
        assert mrun() == 0
    e0.record()
    for _ in range(20):
        mrun()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 20
    clock.start(span_ms=100.0)
    for _ in range(20):
        mrun()
    out["mfma_vector_loop_clock"] = clock.stop()
    out["mfma_vector_loop_tflops"] = round(lib.vsa_probe_mfma_mix_flop(mblocks, iters) / ms / 1e9,
                                           1)
    out["mfma_vector_loop"] = ("the MFMA loop plus 16 exp2 and 48 FMAs per 16 MFMAs on "
                               "independent registers (a fine-kernel wave-step's vector work), "
                               "2 waves per workgroup, 4 workgroups and 2 waves per SIMD as in "
                               "the fine kernel, 2048 workgroups")
    n = 16384
    a = torch.randn((n, n), generator=gen, device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), generator=gen, device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0.record()
    for _ in range(8):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 8
    clock.start(span_ms=30.0)             # the same loop again, for its clock only
    for _ in range(8):
        torch.matmul(a, b, out=c)
    out["gemm_clock"] = clock.stop()
    out["gemm_bf16_16384_tflops"] = round(2.0 * n ** 3 / ms / 1e9, 1)
    del a, b, c, src, res
    return out


def time_pipeline(case, vsa, torch, reps: int) -> dict:
    """Event-timed tile x3 -> select -> fwd -> untile on another workload
    (inputs resident in HBM, buffers allocated once)."""
    dev = torch.device("cuda:0")
    T, H, W, NH, D, B, topk = case.T, case.H, case.W, case.NH, case.D, case.B, case.topk
    to_gpu = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to_gpu(case.q), to_gpu(case.k), to_gpu(case.v)
    Nc = vsa.num_cubes(T, H, W)
    S = Nc * 64
    qt, kt, vt = (torch.empty((B, S, NH, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    vbs = torch.empty(Nc, dtype=torch.int32, device=dev)
    ws = torch.empty(vsa.select_workspace_bytes(B, NH, Nc, D), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device=dev)
    wsf = torch.empty(vsa.fwd_workspace_bytes(B, Nc, Nc, NH, D, topk), dtype=torch.uint8,
                      device=dev)
    out = torch.empty_like(qt)
    out_nat = torch.empty_like(q)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def step(record):
        if record:
            marks[0].record()
        for x, xt in ((q, qt), (k, kt), (v, vt)):
            vsa.tile(x, T, H, W, out=xt, vbs=vbs)
        if record:
            marks[1].record()
        vsa.select(qt, kt, vbs, topk, workspace=ws, out=idx)
        if record:
            marks[2].record()
        vsa.fwd(qt, kt, vt, idx, vbs, out=out, workspace=wsf)
        if record:
            marks[3].record()
        vsa.untile(out, T, H, W, out=out_nat)
        if record:
            marks[4].record()

    step(False)
    torch.cuda.synchronize()
    parts = np.zeros(4)
    for _ in range(reps):
        step(True)
        torch.cuda.synchronize()
        parts += [marks[i].elapsed_time(marks[i + 1]) for i in range(4)]
    parts /= reps
    flops = fwd_flops(idx.cpu().numpy(), vbs.cpu().numpy(), D)
    return {
        "workload": f"{case.name}: grid {T}x{H}x{W} ({T * H * W} tokens) -> {Nc} cubes, "
                    f"{NH} heads, D {D}, topk {topk}",
        "ms_per_step": round(float(parts.sum()), 4),
        "step_breakdown_ms": {"tile_qkv": round(parts[0], 4), "select": round(parts[1], 4),
                              "fwd": round(parts[2], 4), "untile": round(parts[3], 4)},
        "fwd_tflop": round(flops / 1e12, 4),
        "fwd_tflops": round(flops / (parts[2] * 1e-3) / 1e12, 1),
        "fwd_finite": bool(torch.isfinite(out.float()).all()),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the VSA path runs on a single MI355X; "
              "multi-GPU runs are not supported (see the sharding notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    import video_dit_block_amd as vsa

    if args.fwd_only and args.fwd_workload == "hy720":
        print("[bench] generating the 720p input", file=sys.stderr, flush=True)
        case = synth.hy720()
    else:
        print("[bench] generating the Wan-shaped input (seed 2)", file=sys.stderr, flush=True)
        case = synth.wan()
    cpu = None
    if not args.no_cpu and not args.fwd_only:
        # before any GPU call: the CPU workers are forked from this process
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, args.cpu_seconds)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    T, H, W, NH, D, B, topk = case.T, case.H, case.W, case.NH, case.D, case.B, case.topk
    to_gpu = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to_gpu(case.q), to_gpu(case.k), to_gpu(case.v)
    Nc = vsa.num_cubes(T, H, W)
    S = Nc * 64
    qt, kt, vt = (torch.empty((B, S, NH, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    vbs = torch.empty(Nc, dtype=torch.int32, device=dev)
    ws = torch.empty(vsa.select_workspace_bytes(B, NH, Nc, D), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device=dev)
    # one workspace for every fine-stage call of the run: the largest of the
    # sizes needed by its index-row lengths (with key-range splits the size
    # is not monotone in the row length)
    row_lens = {topk, Nc, Nc // 2, *synth.SWEEP_TOPK}
    wsf = torch.empty(max(vsa.fwd_workspace_bytes(B, Nc, Nc, NH, D, t) for t in row_lens
                          if t <= Nc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(qt)
    out_nat = torch.empty_like(q)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [ev() for _ in range(5)]

    def step(record: bool):
        if record:
            marks[0].record()
        vsa.tile(q, T, H, W, out=qt, vbs=vbs)
        vsa.tile(k, T, H, W, out=kt, vbs=vbs)
        vsa.tile(v, T, H, W, out=vt, vbs=vbs)
        if record:
            marks[1].record()
        vsa.select(qt, kt, vbs, topk, workspace=ws, out=idx)
        if record:
            marks[2].record()
        vsa.fwd(qt, kt, vt, idx, vbs, out=out, workspace=wsf)
        if record:
            marks[3].record()
        vsa.untile(out, T, H, W, out=out_nat)
        if record:
            marks[4].record()

    if args.fwd_only:
        # profiler mode: one full step, then only vsa_fwd launches, then one
        # plain 1 GiB device copy whose byte counts calibrate HBM counters
        step(False)
        torch.cuda.synchronize()
        for _ in range(args.warmup + args.steps):
            vsa.fwd(qt, kt, vt, idx, vbs, out=out, workspace=wsf)
        torch.cuda.synchronize()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        # controls for the LDS bank-conflict counter: the same reads laid out
        # conflict-free (stride 1) and on few banks (stride 8), 4- and 16-byte
        lib = ctypes.CDLL(os.path.join(ROOT, "video_dit_block_amd", "libvsa_probe.so"))
        lib.vsa_probe_lds.restype = ctypes.c_int32
        lib.vsa_probe_lds.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
        res = torch.empty(1024 * 64, dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        for width in (4, 16):
            for stride in (1, 8):
                st = lib.vsa_probe_lds(width, stride, 1024, 1024, res.data_ptr(), stream)
                if st != 0:
                    raise RuntimeError(f"vsa_probe_lds failed: {st}")
        torch.cuda.synchronize()
        print(json.dumps({"fwd_only": True, "workload": case.name,
                          "launches": args.warmup + args.steps,
                          "calibration_copy_bytes": 1 << 30,
                          "lds_controls": "width 4/16 x stride 1/8, 1024 x 1024 reads"}))
        return

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    parts = np.zeros(4)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        parts += [marks[i].elapsed_time(marks[i + 1]) for i in range(4)]
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    parts /= args.steps
    step_ms = float(parts.sum())

    # the step back to back, eagerly and as one captured HIP graph (no entry
    # point allocates, sets memory or synchronises, so a step captures whole)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(args.steps):
        step(False)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(False)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / args.steps
    del graph

    # the fine forward alone, back to back (kernel-only, warmed), with the
    # engine clock sampled while it runs
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(args.fwd_reps):
        vsa.fwd(qt, kt, vt, idx, vbs, out=out, workspace=wsf)
    e1.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / args.fwd_reps
    # the same loop again with the clock meter beside it (its figure only)
    clock = ClockMeter(torch, dev)
    clock.start(span_ms=0.7 * args.fwd_reps * fwd_ms)
    for _ in range(args.fwd_reps):
        vsa.fwd(qt, kt, vt, idx, vbs, out=out, workspace=wsf)
    clock_fwd = clock.stop()
    # the same calls one at a time, each between its own pair of events
    pairs = [(ev(), ev()) for _ in range(args.fwd_reps)]
    for a, b in pairs:
        a.record()
        vsa.fwd(qt, kt, vt, idx, vbs, out=out, workspace=wsf)
        b.record()
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in pairs])

    vbs_h = vbs.cpu().numpy()
    idx_h = idx.cpu().numpy()
    flops = fwd_flops(idx_h, vbs_h, D)
    flops_real_q = fwd_flops_real_q(idx_h, vbs_h, D)
    tflops = flops / (fwd_ms * 1e-3) / 1e12
    finite = bool(torch.isfinite(out.float()).all())

    # same kernel, topk = all cubes (dense)
    idx_all = torch.empty((B, NH, Nc, Nc), dtype=torch.int32, device=dev)
    vsa.select(qt, kt, vbs, Nc, workspace=ws, out=idx_all)
    out_d = torch.empty_like(qt)
    vsa.fwd(qt, kt, vt, idx_all, vbs, out=out_d, workspace=wsf)
    torch.cuda.synchronize()
    reps_d = max(3, args.fwd_reps // 10)
    e0.record()
    for _ in range(reps_d):
        vsa.fwd(qt, kt, vt, idx_all, vbs, out=out_d, workspace=wsf)
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1) / reps_d
    dense_flops = fwd_flops(idx_all.cpu().numpy(), vbs_h, D)

    sweep = None
    if not args.no_sweep:
        sweep = {}
        for kk in synth.SWEEP_TOPK:
            ik = idx_all[..., :kk].contiguous()
            vsa.fwd(qt, kt, vt, ik, vbs, out=out_d, workspace=wsf)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps_d):
                vsa.fwd(qt, kt, vt, ik, vbs, out=out_d, workspace=wsf)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps_d
            fl = fwd_flops(ik.cpu().numpy(), vbs_h, D)
            sweep[str(kk)] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                              "speedup_vs_dense": round(dense_ms / ms, 3)}
        del ik
    del idx_all

    # lookup-table leg: the cumulative-mass selector (tau, at most half of the
    # cubes) and vsa_fwd_lut on its table, with and without the row statistics
    max_k = Nc // 2
    lidx, lcnt = vsa.select_cdf(qt, kt, vbs, max_k, args.cdf_tau, workspace=ws)
    lse = torch.empty((B, NH, S), dtype=torch.float32, device=dev)
    mp = torch.empty_like(lse)
    lib = vsa._lib.load()
    ptrs = lambda o, st: (qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), lidx.data_ptr(),
                          lcnt.data_ptr(), vbs.data_ptr(), o.data_ptr(),
                          lse.data_ptr() if st else None, mp.data_ptr() if st else None,
                          B, Nc, Nc, NH, D, max_k, 0.0, wsf.data_ptr(), wsf.numel(),
                          torch.cuda.current_stream().cuda_stream)
    timed = {}
    for name, fn in (("select_cdf", lambda: vsa.select_cdf(qt, kt, vbs, max_k, args.cdf_tau,
                                                           workspace=ws)),
                     ("fwd_lut", lambda: lib.vsa_fwd_lut(*ptrs(out_d, False))),
                     ("fwd_lut_stats", lambda: lib.vsa_fwd_lut(*ptrs(out_d, True)))):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps_d):
            fn()
        e1.record()
        torch.cuda.synchronize()
        timed[name] = e0.elapsed_time(e1) / reps_d
    lcnt_h = lcnt.cpu().numpy()
    lfl = lut_flops(lidx.cpu().numpy(), lcnt_h, vbs_h, D)
    lut = {"tau": args.cdf_tau, "max_k": max_k, "mean_count": round(float(lcnt_h.mean()), 2),
           "sparsity": round(1 - float(lcnt_h.mean()) / Nc, 4),
           "select_cdf_ms": round(timed["select_cdf"], 4),
           "fwd_lut_ms": round(timed["fwd_lut"], 4), "fwd_lut_tflop": round(lfl / 1e12, 4),
           "fwd_lut_tflops": round(lfl / timed["fwd_lut"] / 1e9, 1),
           "fwd_lut_with_lse_max_prob_ms": round(timed["fwd_lut_stats"], 4),
           "stats_finite": bool(torch.isfinite(lse).all() and torch.isfinite(mp).all())}
    del out_d, lidx, lcnt, lse, mp

    # two-stage leg: the coarse stage's own output (pooled q, k, v, cube scores,
    # softmax over cubes times pooled v), with and without the top-k ids taken
    # from the same scores, and the gated combine with seeded uniform gates
    wsc = torch.empty(vsa.coarse_workspace_bytes(B, NH, Nc, D), dtype=torch.uint8, device=dev)
    oc = torch.empty((B, NH, Nc, D), dtype=torch.float32, device=dev)
    idx2 = torch.empty_like(idx)
    gen = torch.Generator(device=dev).manual_seed(7)
    gc = torch.rand(tuple(qt.shape), device=dev, generator=gen).to(torch.bfloat16)
    gf = torch.rand(tuple(qt.shape), device=dev, generator=gen).to(torch.bfloat16)
    comb = torch.empty_like(qt)
    stream = torch.cuda.current_stream().cuda_stream
    cargs = lambda ids: (qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), vbs.data_ptr(), B, Nc, NH,
                         D, topk, ids, 0.0, oc.data_ptr(), wsc.data_ptr(), wsc.numel(), stream)
    for name, fn in (("coarse", lambda: lib.vsa_coarse(*cargs(None))),
                     ("coarse_topk", lambda: lib.vsa_coarse(*cargs(idx2.data_ptr()))),
                     ("combine", lambda: lib.vsa_gate_combine(out.data_ptr(), oc.data_ptr(),
                                                              gc.data_ptr(), gf.data_ptr(),
                                                              comb.data_ptr(), B, Nc, NH, D,
                                                              stream))):
        assert fn() == 0, name
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps_d):
            fn()
        e1.record()
        torch.cuda.synchronize()
        timed[name] = e0.elapsed_time(e1) / reps_d
    comb_bytes = 4 * S * NH * D * 2 + oc.numel() * 4
    two_stage = {
        "coarse_ms": round(timed["coarse"], 4),
        "coarse_with_topk_ms": round(timed["coarse_topk"], 4),
        "topk_equal_to_select": bool(torch.equal(idx2, idx)),
        "gate_combine_ms": round(timed["combine"], 4),
        "gate_combine_gbs": round(comb_bytes / (timed["combine"] * 1e-3) / 1e9, 1),
        "o_coarse_finite": bool(torch.isfinite(oc).all()),
        "step_ms": round(parts[0] + timed["coarse_topk"] + parts[2] + timed["combine"] + parts[3],
                         4),
    }
    del wsc, oc, idx2, gc, gf, comb

    # cube order and mask legs: the fine kernel on the same tensors tiled in
    # 3D Hilbert cube order (selector rerun on them), and the compaction of
    # the top-k selection written as a dense block mask into the LUT
    order = vsa.cube_order(T, H, W, "hilbert").to(dev)
    qh, kh, vh = (torch.empty_like(qt) for _ in range(3))
    vbs_hil = torch.empty_like(vbs)
    for src, dst in ((q, qh), (k, kh), (v, vh)):
        vsa.tile(src, T, H, W, out=dst, vbs=vbs_hil, order=order)
    idx_hil = vsa.select(qh, kh, vbs_hil, topk, workspace=ws)
    out_h = torch.empty_like(qt)
    mask = torch.zeros((B, NH, Nc, Nc), dtype=torch.uint8, device=dev)
    mask.scatter_(3, idx.long(), 1)
    lut_ids = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device=dev)
    lut_cnt = torch.empty((B, NH, Nc), dtype=torch.int32, device=dev)
    for name, fn in (("fwd_hilbert", lambda: vsa.fwd(qh, kh, vh, idx_hil, vbs_hil, out=out_h,
                                                     workspace=wsf)),
                     ("mask_to_lut", lambda: lib.vsa_mask_to_lut(mask.data_ptr(), B, NH, Nc, Nc,
                                                                 topk, lut_ids.data_ptr(),
                                                                 lut_cnt.data_ptr(), None,
                                                                 stream))):
        fn()
        torch.cuda.synchronize()
        reps_o = max(reps_d, 10)
        e0.record()
        for _ in range(reps_o):
            fn()
        e1.record()
        torch.cuda.synchronize()
        timed[name] = e0.elapsed_time(e1) / reps_o
    hfl = fwd_flops(idx_hil.cpu().numpy(), vbs_hil.cpu().numpy(), D)
    mask_bytes = mask.numel() + lut_ids.numel() * 4 + lut_cnt.numel() * 4
    order_mask = {
        "hilbert_fwd_ms": round(timed["fwd_hilbert"], 4),
        "hilbert_fwd_tflops": round(hfl / timed["fwd_hilbert"] / 1e9, 1),
        "row_major_fwd_ms": round(fwd_ms, 4),
        "mask_to_lut_ms": round(timed["mask_to_lut"], 4),
        "mask_to_lut_gbs": round(mask_bytes / (timed["mask_to_lut"] * 1e-3) / 1e9, 1),
        "lut_equals_sorted_topk": bool(torch.equal(lut_ids, torch.sort(idx, dim=-1).values)),
    }
    del qh, kh, vh, out_h, mask, lut_ids, lut_cnt, idx_hil

    # tiling traffic: read real rows, write all rows, per tensor
    tile_bytes = 3 * (T * H * W + S) * NH * D * 2
    print("[bench] bf16 ceilings", file=sys.stderr, flush=True)
    ceilings = bf16_ceilings(torch, dev, clock)

    line = {
        "metric": "fine VSA fwd kernel ms + effective TFLOP/s (% bf16 peak), Wan2.2 shape, "
                  "87.5% sparse",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Wan2.2-A14B-shaped VSA: q,k,v (1, 39936, 40, 128) bf16 BSHD, grid "
                        "21x30x52 -> 624 cubes, topk 78 (87.5% sparse), sm_scale 1/sqrt(128), "
                        "heavy-tailed q/k with one +-2000-logit head, seed 2",
            "global_batch": B, "seq_len": S, "heads": NH, "head_dim": D, "topk": topk,
            "parallelism": "single GPU",
        },
        "fwd_ms": round(fwd_ms, 4),
        "fwd_ms_per_call": {"p10": round(float(np.percentile(per_call, 10)), 4),
                            "median": round(float(np.median(per_call)), 4),
                            "p90": round(float(np.percentile(per_call, 90)), 4),
                            "calls": int(per_call.size)},
        "fwd_tflop": round(flops / 1e12, 4),
        "fwd_pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "peak_bf16_tflops": PEAK_BF16_TFLOPS,
        "fwd_tflop_real_q": round(flops_real_q / 1e12, 4),
        "fwd_pct_peak_real_q": round(100 * flops_real_q / (fwd_ms * 1e-3) / 1e12
                                     / PEAK_BF16_TFLOPS, 2),
        "clock_during_fwd": clock_fwd,
        "bf16_ceilings": dict(ceilings, fwd_pct_of_mfma_loop=round(
            100 * tflops / ceilings["mfma_loop_tflops"], 1), fwd_pct_of_mfma_vector_loop=round(
            100 * tflops / ceilings["mfma_vector_loop_tflops"], 1), fwd_pct_of_gemm_bf16=round(
            100 * tflops / ceilings["gemm_bf16_16384_tflops"], 1)),
        "fwd_finite": finite,
        "dense": {"topk": Nc, "ms": round(dense_ms, 4), "tflop": round(dense_flops / 1e12, 3),
                  "tflops": round(dense_flops / dense_ms / 1e9, 1),
                  "speedup_sparse_vs_dense": round(dense_ms / fwd_ms, 3)},
        "step_breakdown_ms": {"tile_qkv": round(parts[0], 4), "select": round(parts[1], 4),
                              "fwd": round(parts[2], 4), "untile": round(parts[3], 4)},
        "tile_qkv_gbs": round(tile_bytes / (parts[0] * 1e-3) / 1e9, 1),
        "wall_ms_per_step": round(wall, 3),
        "step_back_to_back_ms": {"eager": round(eager_ms, 4), "hip_graph": round(graph_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic()},
        "cpu_baseline": cpu,
    }
    line["lut"] = lut
    line["two_stage"] = two_stage
    line["order_mask"] = order_mask
    if sweep is not None:
        line["sweep"] = sweep
    if not args.no_hy720:
        del qt, kt, vt, out, out_nat, wsf, ws, idx
        torch.cuda.empty_cache()
        print("[bench] 720p workload", file=sys.stderr, flush=True)
        line["hy720"] = time_pipeline(synth.hy720(), vsa, torch, reps=5)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
