#!/usr/bin/env python3
"""Throughput of the fused attention forward (fa_fwd) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3] [--path fused|naive]
    python bench.py --pass bwd [--workload c3]     the backward pass (fa_bwd) instead

One step is one fa_fwd call over the whole workload (all B*H heads, all N query
rows).  Inputs are seeded synthetic tensors already resident in device memory when
the timed region starts.  Prints ONE JSON line with:
  value      TFLOP/s, counting 4*B*H*N^2*d flops per step
  roofline   the fused kernel against the dense bf16/fp16 matrix-core peak, timed with
             HIP events around every launch on the launch stream; `traffic` comes from
             the committed rocprofv3 counter summary when it was taken on this exact
             kernel source, else null
  cpu_baseline  the CPU fp64 oracle timed on this host on a bounded sample of the same
             workload's query rows (a reported baseline, not the target)
"""
from __future__ import annotations

import argparse
import hashlib
import statistics
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synth.configs import HEADDIM_WORKLOADS, WORKLOADS  # noqa: E402

ALL_WORKLOADS = {**WORKLOADS, **HEADDIM_WORKLOADS}

METRIC = "fwd attention TFLOP/s & % of bf16 MFMA peak, B8 H32 N4096 d128"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # MI355X dense matrix-core peaks
KERNEL_SOURCES = ("exact_attention_90_amd/csrc/fa_fused.hip",
                  "exact_attention_90_amd/csrc/fa_fwd16.hpp",
                  "exact_attention_90_amd/csrc/fa_fwd16.hip",
                  "exact_attention_90_amd/csrc/fa_fwd16_d128.hip",
                  "exact_attention_90_amd/csrc/fa_softmax.hpp",
                  "exact_attention_90_amd/csrc/fa_device.hpp")
# the backward kernels have their own hash (bench --pass bwd), so that a change to them
# does not invalidate the forward pass's committed counters
BWD_KERNEL_SOURCES = ("exact_attention_90_amd/csrc/fa_bwd.hip",
                      "exact_attention_90_amd/csrc/fa_bwd.hpp",
                      "exact_attention_90_amd/csrc/fa_bwd_d128.hip",
                      "exact_attention_90_amd/csrc/fa_bwd_d256.hip",
                      "exact_attention_90_amd/csrc/fa_softmax.hpp",
                      "exact_attention_90_amd/csrc/fa_device.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_traffic.md")
# Frozen forward throughput (TFLOP/s) of each named workload, the reference a later change
# is compared with: the line reports value / frozen as `vs_frozen` and warns below 0.95.
# c3: the driver's own bench run of the eight-wave kernel (2.290 ms per call, 38.4 % of
# peak); the others: this bench on the same kernel (the low end of the measured ranges).
FROZEN_TFLOPS = {"c3": 960.4, "c2": 809.0, "c4": 840.0, "c5": 1043.0, "d256": 812.0}


def host_cpu():
    """The host CPU's model name (lscpu's 'Model name', else /proc/cpuinfo's) and the
    number of processors this process may run on."""
    import subprocess

    model = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model == "unknown":
        try:
            for line in open("/proc/cpuinfo"):
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 0
    return model, nproc


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the kernels' code: the sources with line comments, indentation and blank
    lines removed, so that a comment edit keeps the committed counter records valid."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*$", "", line).strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def kernel_form(w, args) -> str:
    """Which form of the fused 16-bit kernel the library picks for this launch: the
    persistent one (d = 128 or 256, one key range, at least two key tiles, more query
    tiles than the device's compute units hold workgroups) or one tile per workgroup."""
    import torch

    if args.path != "fused" or w.dtype == "f32" or (args.split or 1) != 1:
        return "one tile per workgroup" if args.path == "fused" else args.path
    bm = 256 if w.d in (64, 128) else 128
    tiles = w.B * w.H * -(-w.N // bm)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if w.d in (128, 256) and w.N > 64 and tiles > cus:
        return f"persistent: {cus // 8 * 8} workgroups, {tiles} query tiles of {bm} rows"
    return "one tile per workgroup"


def committed_traffic(workload: str, path: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src = kernel_source_hash(BWD_KERNEL_SOURCES if path == "bwd" else KERNEL_SOURCES)
    for line in open(TRAFFIC_FILE):
        m = re.match(r"\s*traffic-json:\s*(\{.*\})\s*$", line)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("workload") == workload and rec.get("path") == path and rec.get("kernel_src") == src:
            return rec
    return None


def cpu_baseline(x, w, o_gpu, lse_gpu, target_s: float):
    """Time the oracle on evenly spaced query rows (about target_s seconds) and check
    those rows of the GPU output against it."""
    import numpy as np

    import oracle

    total = w.rows
    flops_row = 4.0 * w.N * w.d
    scale32 = float(np.float32(w.scale))
    # calibrate on a strided sample of the same shape as the timed one (the oracle
    # widens each head's K and V once, so scattered rows cost more per row)
    cstride = max(1, total // 2048)
    calib = np.arange(0, total, cstride, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attention(x["q"], x["k"], x["v"], w.dtype, scale32, rows=calib)
    per_row = (time.perf_counter() - t0) / len(calib)
    n = int(min(total, max(64, target_s / max(per_row, 1e-9))))
    for _ in range(3):  # a denser sample costs less per row: grow it toward target_s
        stride = max(1, total // n)
        rows = np.arange(0, total, stride, dtype=np.int64)[:n]
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], w.dtype, scale32, rows=rows)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= total:
            break
        n = int(min(total, n * target_s / max(dt, 1e-3)))
    import torch

    idx = torch.from_numpy(rows).to(o_gpu.device)
    og = o_gpu.reshape(-1, w.d).index_select(0, idx).cpu().numpy().astype(np.float64)
    lg = lse_gpu.reshape(-1).index_select(0, idx).cpu().numpy().astype(np.float64)
    parity = {
        "rows": int(len(rows)),
        "max_abs": float(np.abs(og - o_ref).max()),
        "cosine": float((og.ravel() @ o_ref.ravel()) /
                        (np.linalg.norm(og) * np.linalg.norm(o_ref))),
        "lse_rel": float((np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max()),
    }
    model, nproc = host_cpu()
    base = {
        "value": flops_row * len(rows) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(oracle.num_threads()),
        "cpu_model": model,
        "nproc": nproc,
        "kind": "oracle",
        "sample": (f"{len(rows)} of {total} query rows of {w.name} ({w.short()}): rows "
                   f"0, {stride}, 2*{stride}, ... each against all N={w.N} keys; fp64 C "
                   f"oracle, {dt:.1f} s"),
    }
    return base, parity


def copy_calibration(mib: int, steps: int) -> int:
    """Copy `mib` MiB device-to-device `steps` times: each launch reads and writes
    exactly mib * 2^20 bytes, which calibrates the memory-traffic counters."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": steps}), flush=True)
    return 0


def short_sequence_study(reps: int) -> int:
    """Where the fused kernel stops beating the three-kernel naive path: time per call
    of both paths over a grid of short sequence lengths and head counts (inputs resident
    on the device; events around `reps` back-to-back calls, so launch overhead counts as
    it would for a caller).  One JSON line per point."""
    import numpy as np
    import torch

    import exact_attention_90_amd as fa
    from synth.inputs import make_qkv, to_torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for dtype, d in (("bf16", 128), ("f16", 64)):
        for B, H in ((1, 1), (1, 16), (8, 32)):
            for N in (16, 32, 64, 128, 256, 512, 1024, 2048):
                x = make_qkv(B, H, N, d, dtype, seed=7000 + N)
                q, k, v = (to_torch(x[n], dtype).to(dev) for n in ("q", "k", "v"))
                o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
                lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
                nb = fa.naive_workspace_bytes(B, H, N, q.dtype)
                ws = (torch.empty(nb, dtype=torch.uint8, device=dev),
                      torch.empty(nb, dtype=torch.uint8, device=dev))
                scale32 = float(np.float32(1.0 / math.sqrt(d)))
                calls = {
                    "fused": lambda: fa.fwd(q, k, v, scale32, out=o, lse=lse),
                    "naive": lambda: fa.naive_fwd(q, k, v, scale32, out=o, lse=lse, workspace=ws),
                }
                us = {}
                for name, call in calls.items():
                    for _ in range(10):
                        call()
                    torch.cuda.synchronize(dev)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(reps):
                        call()
                    e1.record(stream)
                    torch.cuda.synchronize(dev)
                    us[name] = e0.elapsed_time(e1) * 1e3 / reps
                flops = 4.0 * B * H * N * N * d
                print(json.dumps({
                    "study": "short_sequence", "dtype": dtype, "B": B, "H": H, "N": N, "d": d,
                    "fused_us": round(us["fused"], 2), "naive_us": round(us["naive"], 2),
                    "naive_over_fused": round(us["naive"] / us["fused"], 2),
                    "fused_tflops": round(flops / (us["fused"] * 1e-6) / 1e12, 3),
                    "naive_tflops": round(flops / (us["naive"] * 1e-6) / 1e12, 3),
                }), flush=True)
                del ws, q, k, v, o, lse
                torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=sorted(ALL_WORKLOADS))
    ap.add_argument("--shape", default=None, metavar="B,H,N,d,dtype",
                    help="measure an ad-hoc shape instead of a named workload (N(0,1) inputs)")
    ap.add_argument("--path", default="fused", choices=["fused", "naive"])
    ap.add_argument("--split", type=int, default=0, metavar="S",
                    help="fa_fwd_split (or, with --pass bwd, fa_bwd_split) with S ranges per head "
                         "(for few heads and long sequences); 0 = fa_fwd")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="fwd: the forward pass (the headline); bwd: the backward pass "
                         "(fa_bwd), counted as five N x N x d products (10 B H N^2 d flops)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--zero-inputs", action="store_true",
                    help="diagnostic: all-zero Q, K, V of the workload's shape instead of the "
                         "seeded N(0,1) draw (same instructions and memory traffic, no data "
                         "toggling; contrasts the power-limited clock with the unlimited one)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run device-to-device copies of MIB MiB (a "
                         "plain copy of known size that scales the FETCH/WRITE counters)")
    ap.add_argument("--short-seq-study", action="store_true",
                    help="instead of one workload, time the fused and naive paths over short "
                         "sequence lengths and head counts (one JSON line per point)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, max(1, args.steps))
    if args.short_seq_study:
        return short_sequence_study(reps=100)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); sharding across GPUs is described, not run.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import exact_attention_90_amd as fa
    from synth.inputs import make_qkv, to_torch

    w = ALL_WORKLOADS[args.workload]
    if args.shape:
        from synth.configs import Workload

        B, H, N, d, dt = args.shape.split(",")
        w = Workload(f"B{B}H{H}N{N}d{d}{dt}", int(B), int(H), int(N), int(d), dt, 1.0, 99,
                     "ad-hoc shape")
    scale32 = float(np.float32(w.scale))
    print(f"[bench] generating {w.name}: {w.short()}", file=sys.stderr, flush=True)
    x = make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult)
    if args.zero_inputs:
        x = {n: np.zeros_like(a) for n, a in x.items()}
    dev = torch.device("cuda:0")
    q, k, v = (to_torch(x[n], w.dtype).to(dev) for n in ("q", "k", "v"))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    if args.which == "bwd":
        return bench_bwd(args, w, x, q, k, v, o, lse, scale32, dev)
    ws = None
    if args.split:
        if args.path != "fused":
            print("bench.py: --split runs the fused path", file=sys.stderr)
            return 2
        ws = torch.empty(fa.split_workspace_bytes(w.B, w.H, w.N, w.d, args.split),
                         dtype=torch.uint8, device=dev)
    if args.path == "naive":
        nb = fa.naive_workspace_bytes(w.B, w.H, w.N, q.dtype)
        ws = (torch.empty(nb, dtype=torch.uint8, device=dev),
              torch.empty(nb, dtype=torch.uint8, device=dev))

    def step():
        if args.split:
            fa.fwd_split(q, k, v, args.split, scale32, out=o, lse=lse, workspace=ws)
        elif args.path == "fused":
            fa.fwd(q, k, v, scale32, out=o, lse=lse)
        else:
            fa.naive_fwd(q, k, v, scale32, out=o, lse=lse, workspace=ws)

    stream = torch.cuda.current_stream(dev)  # the stream every launch goes to
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # timed region: events around every launch, on the launch stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize(dev)
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_step = ms_total / args.steps
    flops = float(w.flops)
    value = flops / (ms_step * 1e-3) / 1e12
    avg_launch_ms = sum(per) / len(per)
    peak = PEAK_TFLOPS[w.dtype]
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12

    traffic = None
    rec = committed_traffic(w.name, args.path)
    if rec is not None:
        traffic = rec.get("bytes_per_launch")

    line = {
        "metric": (METRIC if w.name == "c3" and args.path == "fused" and not args.split else
                   f"fwd attention TFLOP/s ({args.path}"
                   + (f", {args.split} key ranges merged" if args.split else "") + f"), {w.short()}")
        + (" [all-zero inputs: power diagnostic]" if args.zero_inputs else ""),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic, all zeros" if args.zero_inputs else "synthetic",
        "config": {
            "workload": f"{w.name}: non-causal attention forward, {w.short()}, "
                        f"scale 1/sqrt({w.d}), O fp32 + LSE",
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "path": args.path, "key_ranges": args.split or 1,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": "fa_fwd16_kernel" if w.dtype != "f32" else "fa_fwd32_kernel",
            "form": kernel_form(w, args),
            "avg_launch_ms": round(avg_launch_ms, 5),
            "median_launch_ms": round(statistics.median(per), 5),
            "min_launch_ms": round(min(per), 5),
            "tflops_at_median": round(flops / (statistics.median(per) * 1e-3) / 1e12, 3),
            "kernel_src": kernel_source_hash(),
        },
        "cpu_baseline": None,
    }
    frozen = FROZEN_TFLOPS.get(w.name)
    if frozen and args.path == "fused" and not args.split and not args.zero_inputs and not args.shape:
        line["vs_frozen"] = round(value / frozen, 4)
        if value < 0.95 * frozen:
            print(f"[bench] WARNING: {w.name} at {value:.1f} TFLOP/s is more than 5% below its "
                  f"frozen {frozen} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a row sample)", file=sys.stderr, flush=True)
        base, parity = cpu_baseline(x, w, o, lse, args.cpu_seconds)
        line["cpu_baseline"] = base
        line["parity_sample"] = parity
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_bwd(x, dout, w, grads_gpu, target_heads: int):
    """The backward oracle, unchanged, on whole heads (the gradients of a key depend on
    every query): the first `target_heads` heads, one per OpenMP thread.  Returns the
    baseline record and the parity of the GPU's gradients on those heads."""
    import numpy as np

    import oracle

    threads = oracle.num_threads()
    nh = max(1, min(w.B * w.H, target_heads))
    heads = list(range(nh))
    t0 = time.perf_counter()
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], dout, w.dtype,
                               float(np.float32(w.scale)), heads=heads)
    dt = time.perf_counter() - t0
    flops = 10.0 * nh * w.N * w.N * w.d
    parity = {}
    for name, g, r in zip(("dq", "dk", "dv"), grads_gpu, ref):
        a = g.reshape(w.B * w.H, w.N, w.d)[:nh].cpu().numpy().astype(np.float64)
        e = a - r
        parity[name] = {"rms_rel": float(np.linalg.norm(e) / np.linalg.norm(r)),
                        "max_rel": float(np.abs(e).max() / np.abs(r).max())}
    model, nproc = host_cpu()
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "cpu_model": model, "nproc": nproc, "kind": "oracle",
            "sample": f"{nh} of {w.B * w.H} heads of {w.short()}, every query and key of "
                      f"each (10 N^2 d flops per head); fp64 C oracle, {dt:.1f} s"}
    return base, parity


def bench_bwd(args, w, x, q, k, v, o, lse, scale32, dev):
    """Time fa_bwd (prep + dK/dV + dQ kernels) on the workload; one JSON line."""
    import torch

    import exact_attention_90_amd as fa
    from synth.inputs import make_dout

    if args.path != "fused" or (w.dtype == "f32" and w.d > 128):
        print("bench.py: the backward pass runs on the fused path (fp32 inputs: d 64, 128)",
              file=sys.stderr)
        return 2
    g_np = make_dout(w.B, w.H, w.N, w.d, w.seed + 5000)
    if args.zero_inputs:
        g_np = g_np * 0
    g = torch.from_numpy(g_np).to(dev)
    fa.fwd(q, k, v, scale32, out=o, lse=lse)
    nbytes = (fa.bwd_split_workspace_bytes(w.B, w.H, w.N, w.d, q.dtype, args.split) if args.split
              else fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d, q.dtype))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))

    def step():
        if args.split:
            fa.bwd_split(q, k, v, o, lse, g, args.split, scale32, workspace=ws, grads=grads)
        else:
            fa.bwd(q, k, v, o, lse, g, scale32, workspace=ws, grads=grads)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    flops = 10.0 * w.B * w.H * w.N * w.N * w.d
    value = flops / (ms_step * 1e-3) / 1e12
    avg = sum(per) / len(per)
    peak = PEAK_TFLOPS[w.dtype]
    rec = committed_traffic(w.name, "bwd")
    line = {
        "metric": f"bwd attention TFLOP/s (5 products, 10 B H N^2 d"
        + (f", {args.split} ranges summed" if args.split else "") + f"), {w.short()}"
        + (" [all-zero inputs: power diagnostic]" if args.zero_inputs else ""),
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic, all zeros" if args.zero_inputs else "synthetic",
        "config": {"workload": f"{w.name}: attention backward (dQ, dK, dV from O, LSE, dO), "
                               f"{w.short()}, scale 1/sqrt({w.d})",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "path": "fused",
                   "ranges": args.split or 1, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(flops / (avg * 1e-3) / 1e12, 3),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / (avg * 1e-3) / 1e12 / peak, 4),
                     "traffic": rec.get("bytes_per_launch") if rec else None,
                     "kernel": "fa_bwd (prep + dkdv + dq kernels)",
                     "avg_launch_ms": round(avg, 5),
                     "median_launch_ms": round(statistics.median(per), 5),
                     "min_launch_ms": round(min(per), 5),
                     "tflops_at_median": round(flops / (statistics.median(per) * 1e-3) / 1e12, 3),
                     "kernel_src": kernel_source_hash(BWD_KERNEL_SOURCES)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline_bwd(x, g_np, w, grads, target_heads=16)
        line["cpu_baseline"] = base
        line["parity_sample"] = parity
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
