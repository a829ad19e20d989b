#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X; prints ONE JSON line.

A timed step is one training step of causal attention -- fa_fwd followed by
fa_bwd (Delta, dK/dV, dQ) -- on the causal training-step workload
(B=4, H=16, N=4096, d=128, bf16), inputs resident in HBM.  `value` is the
credited attention TFLOP/s of that step: forward 4*B*H*N^2*d and backward
10*B*H*N^2*d (five contractions), both halved for causal.

The same run also times, as separate legs reported under "legs": the causal
prefill forward (B2 H32 N8192 d128 bf16), the long causal forward and the
naive three-kernel baseline (B1 H16 N16384 d64 bf16), the non-causal bf16
d128 forwards (B2 H32 N8192 and B1 H32 N16384), the FP8, grouped-query,
chunked-prefill and decode workloads, the FA1 loop order, the non-causal
fp16 sweep N=512..4096 (fused vs naive, with the byte models), and the
fp32 single-head forward.  The sweep and the single-head legs are short calls:
their times come from back-to-back calls replayed from a HIP graph (host
launch cost excluded), with the single eager call's time beside them.
`cpu_baseline` times the fp64 oracle on a sample of the step's heads on the
host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

Traffic counters (`roofline.traffic`): run the step under two rocprofv3
counter passes (FETCH_SIZE, then WRITE_SIZE) with `--calib-copy-mib M`, which
also runs an elementwise copy of M MiB of known traffic, then
`python bench.py --traffic FETCH.csv WRITE.csv --calib-copy-mib M` writes
profiles/traffic_<kernel>_<workload>.txt: each kernel's per-dispatch bytes
past L2, scaled by what the same counter reads for the copy.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16/fp16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 MFMA (twice the 16-bit rate)
METRIC = "attention TFLOP/s (bf16 fwd/bwd) at N=4k-16k; % of MFMA peak; HBM bytes"
CSRC = os.path.join(ROOT, "io_aware_exact_03_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources the training step's four kernels are compiled from; the
# recorded HBM traffic is valid while they are unchanged.
STEP_SOURCES = ("fa_bwd.hip", "fa_device.hpp", "fa_fwd.hip", "fa_plan.hpp")


def _code_only(text: str) -> str:
    """The source with comments and whitespace removed: what the traffic
    depends on (a comment edit leaves the kernels, and their traffic, as
    they were)."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':  # string literal, kept whole
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def digest_of(sources) -> str:
    h = hashlib.sha256()
    for f in sources:
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(CSRC, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def source_digest() -> str:
    return digest_of(STEP_SOURCES)


# The sources of the fused and naive forwards the traffic legs run.
TRAFFIC_LEG_SOURCES = ("fa_device.hpp", "fa_fwd.hip", "fa_naive.hip", "fa_plan.hpp")


# ---------------------------------------------------------------------------
# Cost model.  Flops: forward 4 N^2 d per head (two contractions), backward
# 10 N^2 d (five distinct contractions), halved for causal.  Bytes: what each
# path must move through HBM at least -- the fused path reads Q, K, V once
# and writes O (plus the fp32 LSE); the naive path also writes S, reads S,
# writes P and reads P ("Flash Attention -- five lessons converging into 80
# lines", Lesson 1: 4 N^2 + 4 N d elements against 4 N d).
# ---------------------------------------------------------------------------
def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def bwd_flops(B, H, N, d, causal):
    f = 10.0 * B * H * N * N * d
    return f / 2 if causal else f


def fused_fwd_bytes(B, H, N, d, e_in, lse=True):
    """Q, K, V read + O written (e_in bytes each) [+ fp32 LSE written]."""
    return B * H * (4 * N * d * e_in + (4 * N if lse else 0))


def naive_fwd_bytes(B, H, N, d, e_in, e_ws, lse=True):
    """The fused bytes plus S and P each written once and read once
    (4 N^2 elements of the workspace type)."""
    return B * H * 4 * N * N * e_ws + fused_fwd_bytes(B, H, N, d, e_in, lse)


def sp_roundtrip_bytes(N, e_ws):
    """The S + P round trips alone, per head: 4 N^2 elements."""
    return 4 * N * N * e_ws


def fused_bwd_bytes(B, H, N, d, e_in):
    """The backward's compulsory traffic: Q, K, V, O, dO read once; LSE read
    once; Delta written once and read once; dQ, dK, dV written in fp32."""
    return B * H * (5 * N * d * e_in + 4 * N + 2 * 4 * N + 3 * 4 * N * d)


def delta_bytes(w):
    """The Delta preprocess reads O and dO and writes one fp32 per row."""
    return w.B * w.H * w.N * (2 * w.d * 2 + 4)


# Flops each kernel of the step executes as contractions (per launch):
# forward S, PV; dK/dV pass S, dP, dV, dK; dQ pass S, dP, dQ.
KERNEL_CONTRACTIONS = {"fa_fwd": 2, "bwd_delta": 0, "bwd_dkdv": 4, "bwd_dq": 3}


def read_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_digest") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_reps(fn, reps: int, torch):
    """Median and min milliseconds of fn() over reps, HIP events on the
    current stream."""
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def time_back_to_back(fn, torch, calls: int = 5, reps: int = 8):
    """Median per-call milliseconds of `calls` back-to-back calls of fn()
    between two HIP events (reps times): the host work of one call overlaps
    the GPU work of the one before, as in a loop of calls, so a call of a
    millisecond or so is not charged the binding's host time."""
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / calls)
    ts.sort()
    return ts[len(ts) // 2]


def time_graph(fn, torch, eager_ms: float, reps: int = 10, target_ms: float = 1.0):
    """Per-call milliseconds of fn() with the host launch cost taken out:
    `calls` back-to-back calls (enough for about target_ms of GPU work) are
    captured into one HIP graph, which is replayed reps times between HIP
    events; returns (median per-call ms, calls)."""
    calls = max(1, min(50, int(math.ceil(target_ms / max(eager_ms, 1e-3)))))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ms, _ = time_reps(g.replay, reps, torch)
    del g
    return ms / calls, calls


def cpu_baseline(w, q, k, v, do, target_s: float):
    """The fp64 oracle (forward + backward) on a sample of the workload's
    heads, one head per worker thread with single-threaded BLAS."""
    import concurrent.futures as cf

    import numpy as np
    from threadpoolctl import threadpool_limits

    import fa_synth
    import oracle

    cores = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        qq, kk, vv, gg = (fa_synth.to_f64(t[sl]) for t in (q, k, v, do))
        oracle.attn_fwd(qq, kk, vv, w.scale, w.causal)
        oracle.attn_bwd(qq, kk, vv, gg, w.scale, w.causal)

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        one(heads[0])
        per_head = time.perf_counter() - t0
        n = max(cores, min(len(heads), int(target_s * cores / max(per_head, 1e-3))))
        n = min(len(heads), (n // cores) * cores or cores)
        sample = heads[:n]
        with cf.ThreadPoolExecutor(cores) as ex:
            t0 = time.perf_counter()
            list(ex.map(one, sample))
            wall = time.perf_counter() - t0
    flops = (fwd_flops(1, 1, w.N, w.d, w.causal) + bwd_flops(1, 1, w.N, w.d, w.causal)) * len(sample)
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{len(sample)} of {len(heads)} heads of {w.name}, forward + backward, fp64 NumPy, one head "
                   f"per thread with single-threaded BLAS; {wall:.1f} s wall; credited flops as on the GPU (the "
                   f"oracle computes the full N x N before masking, twice the credited causal work)"),
        "seconds": wall,
        "heads": len(sample),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", type=int, default=1, help="also time the other workloads (1) or not (0)")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run an elementwise copy of this many MiB (counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_*.txt from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--traffic-legs", action="store_true",
                    help="run only the fused and naive forwards of the non-causal sweep and the long causal "
                         "workload (twice each, after the calibration copy), for counter passes")
    ap.add_argument("--traffic-legs-write", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_naive_vs_fused.md from the counter passes of --traffic-legs")
    ap.add_argument("--decode-traffic", action="store_true",
                    help="run only the two decode workloads (twice each, after the calibration copy), for "
                         "counter passes")
    ap.add_argument("--decode-traffic-write", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_decode.md from the counter passes of --decode-traffic")
    ap.add_argument("--stats", metavar="KERNEL_TRACE_CSV",
                    help="write profiles/kernel_stats_<workload>.md from a rocprofv3 kernel trace of the "
                         "default training-step run (--legs 0 --cpu-baseline 0) and exit")
    ap.add_argument("--ceilings", type=int, default=1, help="also measure the chip's ceilings (1) or not (0)")
    ap.add_argument("--lib", metavar="PATH",
                    help="load this build of libfa.so (a tile variant from io_aware_exact_03_amd.build --variant)")
    ap.add_argument("--tile-probe", action="store_true",
                    help="run only the kernels the tile sweep profiles: the training step and the d = 64 "
                         "forwards (non-causal fp16 B4 H8 N4096, causal bf16 B1 H16 N16384), --steps times each")
    ap.add_argument("--sq-write", nargs=2, metavar=("PASS1_DIR", "PASS2_DIR"),
                    help="write profiles/sq_counters_<step>.md from the two SQ counter passes over the step")
    ap.add_argument("--legs-stats", metavar="KERNEL_TRACE_CSV",
                    help="write profiles/kernel_stats_bench_legs.md from a kernel trace of a full bench run")
    ap.add_argument("--tile-sweep-write", metavar="DIR",
                    help="write profiles/tile_sweep_*.md from DIR/<variant>/{sq,kt} rocprofv3 runs of --tile-probe")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.calib_copy_mib)
        return
    if args.decode_traffic_write:
        write_decode_traffic(args.decode_traffic_write[0], args.decode_traffic_write[1], args.calib_copy_mib)
        return
    if args.traffic_legs_write:
        write_traffic_legs(args.traffic_legs_write[0], args.traffic_legs_write[1], args.calib_copy_mib)
        return
    if args.stats:
        write_stats(args.stats, args.steps, args.warmup)
        return
    if args.tile_sweep_write:
        write_tile_sweep(args.tile_sweep_write)
        return
    if args.sq_write:
        write_sq(args.sq_write[0], args.sq_write[1])
        return
    if args.legs_stats:
        write_legs_stats(args.legs_stats)
        return
    if args.lib:
        os.environ["IO_AWARE_FA_LIB"] = os.path.abspath(args.lib)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: --gpus {args.gpus} requested; this build measures one GPU only (the attention kernels "
              f"run per (batch, head) on a single MI355X; no multi-GPU path exists)", file=sys.stderr)
        sys.exit(2)

    import torch

    import fa_synth
    import io_aware_exact_03_amd as fa

    fa._lib.load()
    dev = torch.device("cuda:0")
    digest = source_digest()
    if args.decode_traffic:
        run_decode_traffic(torch, fa, fa_synth, dev, args.calib_copy_mib)
        return
    if args.traffic_legs:
        run_traffic_legs(torch, fa, fa_synth, dev, args.calib_copy_mib)
        return
    if args.tile_probe:
        run_tile_probe(torch, fa, fa_synth, dev, args.steps, args.warmup)
        return

    # ---------------- the timed step: causal training step ----------------
    w = fa_synth.TRAIN_STEP
    log(f"[bench] inputs {w.describe()}")
    q, k, v, do = fa_synth.workload_inputs(w)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o = torch.empty_like(qd)
    f32 = dict(dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), **f32)
    delta = torch.empty((w.B, w.H, w.N), **f32)
    dq = torch.empty((w.B, w.H, w.N, w.d), **f32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fwd(qd, kd, vd, w.scale, w.causal, out=o, lse=lse)
        for s in (1, 2, 3):
            if ev is not None:
                ev[s].record()
            fa.bwd_stage(s, qd, kd, vd, o, dod, lse, w.scale, w.causal, delta, dq, dk, dv)
        if ev is not None:
            ev[4].record()

    if args.calib_copy_mib:
        # Counter calibration: reads and writes exactly M MiB each.
        src = torch.ones(args.calib_copy_mib * (1 << 18), **f32)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    names = ["fa_fwd", "bwd_delta", "bwd_dkdv", "bwd_dq"]
    kern_ms = {n: sum(e[i].elapsed_time(e[i + 1]) for e in events) / args.steps for i, n in enumerate(names)}
    step_flops = fwd_flops(w.B, w.H, w.N, w.d, w.causal) + bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    value = step_flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.3f} ms, {value:.1f} TFLOP/s; kernels {kern_ms}")

    # roofline of the dominant kernel of the step
    dom = max(kern_ms, key=kern_ms.get)
    unit_flops = 2.0 * w.B * w.H * w.N * w.N * w.d / (2 if w.causal else 1)  # one contraction
    if KERNEL_CONTRACTIONS[dom] > 0:
        achieved = KERNEL_CONTRACTIONS[dom] * unit_flops / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        byts = delta_bytes(w)
        achieved = byts / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    roof["kernel"] = dom
    roof["kernel_ms"] = kern_ms[dom]
    roof["traffic"] = read_traffic(dom, w.name, digest)
    roof["timing"] = "HIP events on the launch stream around each launch of the timed steps"
    prof = read_stats(w.name, digest)
    if prof and dom in prof["kernel_us"]:
        # the same kernel's average over the same steps, from the committed
        # rocprofv3 kernel trace of this code
        p_ms = prof["kernel_us"][dom] / 1e3
        p_ach = roof["achieved"] * kern_ms[dom] / p_ms
        roof["profile"] = {"kernel_ms": p_ms, "achieved": p_ach, "frac": p_ach / roof["peak"],
                           "source": prof["path"]}

    kernels = {}
    for n_ in names:
        c = KERNEL_CONTRACTIONS[n_]
        entry = {"ms": kern_ms[n_]}
        if c:
            tf = c * unit_flops / (kern_ms[n_] * 1e-3) / 1e12
            entry.update({"tflops": tf, "frac_mfma_peak": tf / PEAK_BF16_TFLOPS})
        else:
            entry.update({"gbs": delta_bytes(w) / (kern_ms[n_] * 1e-3) / 1e9})
        kernels[n_] = entry
    fwd_tf = fwd_flops(w.B, w.H, w.N, w.d, w.causal) / (kern_ms["fa_fwd"] * 1e-3) / 1e12
    bwd_ms = kern_ms["bwd_delta"] + kern_ms["bwd_dkdv"] + kern_ms["bwd_dq"]
    bwd_tf = bwd_flops(w.B, w.H, w.N, w.d, w.causal) / (bwd_ms * 1e-3) / 1e12
    del o, lse, delta, dq, dk, dv
    torch.cuda.empty_cache()

    legs = {}
    if args.legs:
        legs = run_legs(torch, fa, fa_synth, dev)
        tl = read_traffic_legs(digest_of(TRAFFIC_LEG_SOURCES))
        for name, entry in (tl or {}).items():
            if name in legs:
                legs[name].update(entry)

    # the ceilings last: their long matrix-core and copy loops heat the chip,
    # which the workloads above should not inherit
    ceil = None
    if args.ceilings:
        ceil = measure_ceilings(torch, fa, dev)
        log(f"[bench] ceilings {ceil}")
        if roof["unit"] == "TFLOP/s":
            roof["measured_peak"] = ceil["mfma_bf16_tflops"]
            roof["frac_of_measured_peak"] = roof["achieved"] / ceil["mfma_bf16_tflops"]

    cpu = None
    if args.cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle) ...")
        cpu = cpu_baseline(w, q, k, v, do, args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "seed": w.seed, "step": "fa_fwd + fa_bwd",
                   "flops_per_step": step_flops},
        "frac_mfma_peak": value / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_tf,
        "bwd_tflops": bwd_tf,
        "kernels": kernels,
        "roofline": roof,
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "legs": legs,
        "source_digest": digest,
    }
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# Tile sweep: the same kernels built with other tile constants (the FA_*
# defines of csrc/fa_plan.hpp), each profiled with one SQ-counter pass and a
# kernel trace of --tile-probe.
# ---------------------------------------------------------------------------
TILE_VARIANTS = [
    # name, defines, forward (waves, BN at d = 64), dQ waves
    ("shipped", (), (8, 128), 8),
    ("fwd_w4", ("FA_FWD16_WAVES=4",), (4, 128), 8),
    ("fwd_bn64", ("FA_FWD16_BN_D64=64",), (8, 64), 8),
    ("fwd_w4_bn64", ("FA_FWD16_WAVES=4", "FA_FWD16_BN_D64=64"), (4, 64), 8),
    ("dq_w4", ("FA_DQ_WAVES=4",), (8, 128), 4),
]
TILE_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT "
                 "SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE")


def run_tile_probe(torch, fa, fa_synth, dev, reps: int, warmup: int):
    """The kernels the tile sweep compares, reps times each after warmup:
    the causal training step (fwd16 and dQ at d = 128, dK/dV) and the d = 64
    forwards of the non-causal sweep (N = 4096) and the long causal
    workload.  Prints one JSON line of mean event milliseconds."""
    res = {"lib": os.environ.get("IO_AWARE_FA_LIB", "shipped")}
    w = fa_synth.TRAIN_STEP
    q, k, v, do = (t.to(dev) for t in fa_synth.workload_inputs(w))
    f32 = dict(dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), **f32)
    bufs = dict(delta=torch.empty((w.B, w.H, w.N), **f32), dq=torch.empty((w.B, w.H, w.N, w.d), **f32),
                dk=torch.empty((w.B, w.H, w.N, w.d), **f32), dv=torch.empty((w.B, w.H, w.N, w.d), **f32))
    def step():
        fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        fa.bwd(q, k, v, o, do, lse, w.scale, w.causal, **bufs)
    for _ in range(warmup):
        step()
    ms, _ = time_reps(step, reps, torch)
    res[w.name] = ms
    del q, k, v, do, o, lse, bufs
    for w in (fa_synth.NONCAUSAL_SWEEP[-1], fa_synth.LONG_CAUSAL):
        q, k, v = (t.to(dev) for t in fa_synth.workload_inputs(w, with_dout=False))
        o, lse = fa.fwd(q, k, v, w.scale, w.causal)
        fn = lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        for _ in range(warmup):
            fn()
        res[w.name], _ = time_reps(fn, reps, torch)
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


def _tile_rows(sq_csv: str, kt_csv: str):
    """Per kernel name: mean duration (us) and the summed counters, averaged
    over its dispatches (counters summed over the counter instances first)."""
    import collections
    import csv

    dur = collections.defaultdict(list)
    with open(kt_csv) as f:
        for r in csv.DictReader(f):
            dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    with open(sq_csv) as f:
        for r in csv.DictReader(f):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
    by_name = collections.defaultdict(list)
    for did, c in per.items():
        by_name[names[did]].append(c)
    out = {}
    for name, lst in by_name.items():
        keys = set().union(*lst)
        ds = sorted(dur.get(name, []))
        out[name] = {"n": len(lst), "dur_us": ds[len(ds) // 2] if ds else float("nan"), "n_trace": len(ds),
                     **{k2: sum(c.get(k2, 0.0) for c in lst) / len(lst) for k2 in keys}}
    return out


def _kernel_label(name: str) -> str:
    """fwd16<BF16, d128, BN64, causal> style label from a kernel's
    demangled name (its template arguments)."""
    import re

    m = re.search(r"(fwd16_kernel|bwd_dq_kernel|bwd_dkdv_kernel)<fa::(\w+), (\d+), (\w+)(?:, (\w+))?(?:, (\w+))?>", name)
    if not m:
        return name.split("(")[0]
    kind, dt, d = m.group(1), m.group(2), m.group(3)
    if kind == "fwd16_kernel":  # <T, D, BN, CAUSAL>
        return f"fwd16<{dt}, d{d}, BN{m.group(4)}, {'causal' if m.group(5) == 'true' else 'non-causal'}>"
    return f"{kind[:-7]}<{dt}, d{d}, {'causal' if m.group(4) == 'true' else 'non-causal'}>"


def write_tile_sweep(root: str):
    """profiles/tile_sweep_{fwd16,dq,dkdv}.md from the --tile-probe runs under
    root/<variant>/sq (counter pass) and root/<variant>/kt (kernel trace)."""
    rows = {}
    for name, _, _, _ in TILE_VARIANTS:
        d = os.path.join(root, name)
        rows[name] = _tile_rows(os.path.join(d, "sq", "run_counter_collection.csv"),
                                os.path.join(d, "kt", "run_kernel_trace.csv"))

    def line(variant, shape, kname, c):
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / 8  # summed over the 8 XCDs
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * gui) if gui else float("nan")
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        lds_act = c.get("SQ_LDS_IDX_ACTIVE", 0.0)
        conflicts = 100 * c.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds_act if lds_act else 0.0
        lds_wait = 100 * c.get("SQ_WAIT_INST_LDS", 0.0) / wc if wc else 0.0
        return (f"| {variant} | `{_kernel_label(kname)}` | {shape} | {c['dur_us']:.1f} | {mf / 1e6:.2f} | "
                f"{c.get('SQ_INSTS_VALU', 0.0) / mf:.2f} | {c.get('SQ_INSTS_LDS', 0.0) / mf:.2f} | "
                f"{conflicts:.2f}% | {lds_wait:.1f}% | {100 * busy:.1f}% |")

    head = ("| variant | kernel | tile (BM x BN, waves) | median time (us) | MFMA (M) | VALU / MFMA | LDS / MFMA | "
            "LDS bank conflicts / LDS active | LDS wait / wave cycles | MFMA busy |\n"
            "|---|---|---|---|---|---|---|---|---|---|\n")
    cmd = ("For each variant V (defines in the table below), on the MI355X box with TMPDIR=/tmp:\n\n```\n"
           "python3 -m io_aware_exact_03_amd.build --variant V -D MACRO=VALUE ...   # not for 'shipped'\n"
           f"rocprofv3 --pmc {TILE_COUNTERS} --output-format csv \\\n"
           "    -d gpurun_out/tile/V/sq -o run -- python3 bench.py --tile-probe --steps 3 --warmup 1 --lib LIB\n"
           "rocprofv3 --kernel-trace --output-format csv -d gpurun_out/tile/V/kt -o run -- \\\n"
           "    python3 bench.py --tile-probe --steps 15 --warmup 2 --lib LIB\n"
           "python3 bench.py --tile-sweep-write gpurun_out/tile\n```\n\n"
           "LIB is io_aware_exact_03_amd/_build/variants/V/libfa.so (for 'shipped', io_aware_exact_03_amd/libfa.so).  "
           "Each variant passed the forward and chunked-prefill parity tests (forward variants) or the backward "
           "parity tests (dQ variant) against the oracle before it was profiled.  Per kernel: the median duration "
           "over the kernel-trace run's dispatches, and the counters averaged over the counter run's.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8), "
           "the fraction of SIMD cycles the matrix cores were busy at the clock the chip held.  Counts are wave "
           "instructions; one MFMA is one 32x32x16 product.\n\n"
           "| variant | defines |\n|---|---|\n"
           + "".join(f"| {n} | {' '.join(dd) or '(none)'} |\n" for n, dd, _, _ in TILE_VARIANTS) + "\n")

    def table(match, shape_of):
        out = head
        for name, _, fw, qw in TILE_VARIANTS:
            for kname, c in sorted(rows[name].items()):
                if match(kname):
                    out += line(name, shape_of(kname, fw, qw), kname, c) + "\n"
        return out

    def fwd_shape(kname, fw, qw):
        import re

        m = re.search(r"fwd16_kernel<fa::\w+, \d+, (\d+),", kname)
        return f"{32 * fw[0]} x {m.group(1) if m else '?'}, {fw[0]}"

    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "tile_sweep_fwd16.md"), "w") as f:
        f.write("# Tile sweep: 16-bit forward (fwd16_kernel)\n\n"
                "Workloads: the causal train step B4 H16 N4096 d128 bf16 (its forward), the non-causal "
                "B4 H8 N4096 d64 fp16 forward and the long causal B1 H16 N16384 d64 bf16 forward.  At d = 128 "
                "the K/V tile stays at 64 keys: five ring buffers of 16 KB each for K and for V fill the 160 KB "
                "LDS, so BN = 128 would need a shallower ring.\n\n"
                + cmd + table(lambda k: "fwd16_kernel" in k, fwd_shape))
    with open(os.path.join(PROFILES, "tile_sweep_dq.md"), "w") as f:
        f.write("# Tile sweep: dQ kernel (bwd_dq_kernel)\n\n"
                "Workload: the causal train step B4 H16 N4096 d128 bf16.  The K/V tile is 64 keys at d = 128 "
                "(four ring buffers fill the LDS).\n\n"
                + cmd + table(lambda k: "bwd_dq_kernel" in k, lambda kname, fw, qw: f"{32 * qw} x 64, {qw}"))
    with open(os.path.join(PROFILES, "tile_sweep_dkdv.md"), "w") as f:
        f.write("# Tile sweep: dK/dV kernel (bwd_dkdv_kernel)\n\n"
                "Workload: the causal train step B4 H16 N4096 d128 bf16.  The dK/dV kernel has one shape: 128 "
                "keys per workgroup as four pairs of waves (32 keys each), 64-query blocks taken as two 32-query "
                "halves in alternating phases.  Its causal plan relies on that shape (the masked query blocks of "
                "a 128-key block are its first two), so every variant builds it unchanged and its rows show the "
                "run-to-run spread of one kernel.\n\n"
                + cmd + table(lambda k: "bwd_dkdv_kernel" in k, lambda kname, fw, qw: "64 x 128, 8"))
    print("wrote profiles/tile_sweep_fwd16.md, tile_sweep_dq.md, tile_sweep_dkdv.md")


TRAFFIC_KERNELS = {"fwd16_kernel": "fa_fwd", "bwd_delta_kernel": "bwd_delta", "bwd_dkdv_kernel": "bwd_dkdv",
                   "bwd_dq_kernel": "bwd_dq"}


def write_traffic(fetch_csv: str, write_csv: str, calib_mib: int):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each step kernel, scaled
    by the copy's reading of the same counter, to profiles/traffic_*.txt."""
    import csv

    import fa_synth

    if calib_mib <= 0:
        sys.exit("--traffic needs the --calib-copy-mib the counter runs used")

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = next((v for k_, v in TRAFFIC_KERNELS.items() if k_ in name), None)
            if key is None and "add" in name and "elementwise" in name:
                key = "calib_copy"
            if key is None:
                continue
            acc.setdefault(key, {}).setdefault(r.get("Dispatch_Id", len(acc)), 0.0)
            acc[key][r.get("Dispatch_Id", len(acc))] += float(r["Counter_Value"])
        return {k_: sum(v.values()) / len(v) for k_, v in acc.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    expect_kib = calib_mib * 1024.0
    if "calib_copy" not in fetch or "calib_copy" not in write:
        sys.exit("no calibration copy found in the counter files")
    f_scale = expect_kib / fetch["calib_copy"]
    w_scale = expect_kib / write["calib_copy"]
    w = fa_synth.TRAIN_STEP
    digest = source_digest()
    for key in TRAFFIC_KERNELS.values():
        if key not in fetch or key not in write:
            continue
        byts = (fetch[key] * f_scale + write[key] * w_scale) * 1024.0
        path = os.path.join(PROFILES, f"traffic_{key}_{w.name}.txt")
        with open(path, "w") as f:
            f.write(f"# HBM-side traffic of {key} per launch on {w.name} (bytes past L2: HBM or the\n"
                    f"# memory-side cache), from rocprofv3 counter passes over bench.py; the calibration\n"
                    f"# copy (torch elementwise add, {calib_mib} MiB in + {calib_mib} MiB out) fixes the scale.\n"
                    f"# Passes (repo root, TMPDIR=/tmp):\n"
                    f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/traffic_fetch -o run -- "
                    f"python3 bench.py --steps 2 --warmup 1 --legs 0 --cpu-baseline 0 --calib-copy-mib {calib_mib}\n"
                    f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/traffic_write -o run -- "
                    f"python3 bench.py --steps 2 --warmup 1 --legs 0 --cpu-baseline 0 --calib-copy-mib {calib_mib}\n"
                    f"#   python3 bench.py --traffic gpurun_out/traffic_fetch/run_counter_collection.csv "
                    f"gpurun_out/traffic_write/run_counter_collection.csv --calib-copy-mib {calib_mib}\n")
            f.write(f"fetch_kib_per_dispatch = {fetch[key]:.1f}\n")
            f.write(f"write_kib_per_dispatch = {write[key]:.1f}\n")
            f.write(f"calib_fetch_kib = {fetch['calib_copy']:.1f}\n")
            f.write(f"calib_write_kib = {write['calib_copy']:.1f}\n")
            f.write(f"fetch_scale = {f_scale:.4f}\n")
            f.write(f"write_scale = {w_scale:.4f}\n")
            f.write(f"hbm_bytes_per_launch = {byts:.0f}\n")
            f.write(f"source_digest = {digest}\n")
        print(f"wrote {path}: {byts / 1e6:.1f} MB per launch")


def _clock_ghz(clk) -> float:
    """Median over workgroups of shader-clock ticks / constant-clock (100 MHz)
    ticks, in GHz."""
    c = clk.view(-1, 2).cpu().double()
    return float((c[:, 0] / c[:, 1] * 0.1).median())


def measure_ceilings(torch, fa, dev):
    """What the chip sustains, measured with the library's own ceiling
    kernels: matrix cores alone (8 independent v_mfma_f32_32x32x16_bf16
    accumulators per wave, two waves per SIMD, one workgroup per CU), a
    streaming copy and a streaming read of 2 GiB."""
    out = {}
    wgs, waves, iters = 256, 8, 4000
    fa.ceiling_mfma(wgs, waves, iters)
    ms, _ = time_reps(lambda: fa.ceiling_mfma(wgs, waves, iters), 5, torch)
    out["mfma_bf16_tflops"] = fa.ceiling_mfma_flops(wgs, waves, iters) / (ms * 1e-3) / 1e12
    _, clk = fa.ceiling_mfma(wgs, waves, iters, clocks=True)
    out["mfma_clock_ghz"] = _clock_ghz(clk)
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    fa.ceiling_copy(src, dst)
    ms, _ = time_reps(lambda: fa.ceiling_copy(src, dst), 10, torch)
    out["copy_gbs"] = 2 * nbytes / (ms * 1e-3) / 1e9  # read + write
    sink = fa.ceiling_read(src)
    ms, _ = time_reps(lambda: fa.ceiling_read(src, sink), 10, torch)
    out["read_gbs"] = nbytes / (ms * 1e-3) / 1e9
    # the same read over 128 MiB, about a decode step's cache (one launch
    # then carries its ramp and tail, as the decode kernels do)
    small = src[: (128 << 20) // 4]
    fa.ceiling_read(small, sink)
    ms, _ = time_reps(lambda: fa.ceiling_read(small, sink), 20, torch)
    out["read_gbs_128mib"] = (128 << 20) / (ms * 1e-3) / 1e9
    del src, dst, sink
    torch.cuda.empty_cache()
    # vector issue cost of the softmax's instructions, one wave (shader-clock
    # cycles per wave instruction; loop overhead included)
    c = {m: min(fa.ceiling_valu(m, 20000) for _ in range(2)) for m in (0, 1, 2)}
    fma = c[1] / 96
    out["valu_issue_cycles"] = {"fma": fma, "exp": (c[0] - 32 * fma) / 32,
                                "exp_fma_mix_per_iter": c[2], "serial_per_iter": c[0] + c[1],
                                "full_overlap_per_iter": 128 * fma}
    # the 16-bit forward's step mix without HBM traffic: operands in
    # registers, read from LDS, and LDS plus the per-tile barrier
    mix = {}
    for mode, name in ((0, "registers"), (1, "lds_operands"), (2, "lds_operands_barrier")):
        fa.ceiling_mix(mode, wgs, 1000)
        ms, _ = time_reps(lambda: fa.ceiling_mix(mode, wgs, 1000), 5, torch)
        tf = fa.ceiling_mix_flops(wgs, 1000) / (ms * 1e-3) / 1e12
        _, clk = fa.ceiling_mix(mode, wgs, 1000, clocks=True)
        mix[name] = {"tflops": tf, "frac_of_mfma_ceiling": tf / out["mfma_bf16_tflops"],
                     "frac_of_spec": tf / PEAK_BF16_TFLOPS, "clock_ghz": _clock_ghz(clk)}
    out["fwd_step_mix"] = mix
    out["spec"] = {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    out["how"] = ("fa_ceiling_mfma: 256 workgroups x 8 waves x 4000 x 8 products; fa_ceiling_copy / "
                  "fa_ceiling_read over 2 GiB (and 128 MiB); medians of HIP-event timings; fa_ceiling_valu: one wave, "
                  "20000 iterations of 32 exp + 32 mul / 96 fma / both; fa_ceiling_mix: 256 workgroups x 8 "
                  "waves x 2000 forward steps of 16 products and 16 weights")
    return out


STEP_KERNELS = {"fwd16_kernel": "fa_fwd", "bwd_delta_kernel": "bwd_delta", "bwd_dkdv_kernel": "bwd_dkdv",
                "bwd_dq_kernel": "bwd_dq"}


def write_stats(trace_csv: str, steps: int, warmup: int):
    """profiles/kernel_stats_<training step>.md from a rocprofv3 kernel trace
    of `bench.py --legs 0 --cpu-baseline 0 --ceilings 0` with the same
    --steps / --warmup: per kernel, the average over the timed steps (the
    last `steps` dispatches), the dispatches the bench's events time."""
    import csv

    import fa_synth
    w = fa_synth.TRAIN_STEP
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        key = next((v for k_, v in STEP_KERNELS.items() if k_ in r["Kernel_Name"]), None)
        if key is None:
            continue
        per.setdefault(key, []).append((int(r["Dispatch_Id"]),
                                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    digest = source_digest()
    path = os.path.join(PROFILES, f"kernel_stats_{w.name}.md")
    total = {}
    lines = []
    for key in ("fa_fwd", "bwd_delta", "bwd_dkdv", "bwd_dq"):
        d = [t for _, t in sorted(per.get(key, []))]
        if len(d) < steps + warmup:
            sys.exit(f"{key}: {len(d)} dispatches in the trace, expected {steps + warmup}")
        timed = d[-steps:]
        total[key] = sum(timed) / len(timed)
        lines.append(f"| `{key}` | {len(d)} | {total[key]:.1f} | {min(timed):.1f} | {max(timed):.1f} |")
    step_us = sum(total.values())
    with open(path, "w") as f:
        f.write(f"# Kernel times: causal training step ({w.describe()})\n\n")
        f.write("Command (repo root on the MI355X box, `TMPDIR=/tmp`):\n\n```\n")
        f.write(f"rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/kstats -o run -- \\\n"
                f"    python3 bench.py --steps {steps} --warmup {warmup} --legs 0 --cpu-baseline 0 --ceilings 0\n"
                f"python3 bench.py --stats gpurun_out/kstats/run_kernel_trace.csv --steps {steps} --warmup {warmup}\n"
                "```\n\n")
        f.write(f"Averages over the {steps} timed steps (the last {steps} dispatches of each kernel; the "
                f"{warmup} warm-up steps before them are left out), the dispatches whose HIP-event times the "
                "bench line's `roofline` uses; the bench reads the lines below back as `roofline.profile`.\n\n")
        f.write("| kernel | dispatches | avg over timed steps (us) | min (us) | max (us) |\n|---|---|---|---|---|\n")
        f.write("\n".join(lines) + "\n\n")
        f.write(f"Sum of the four kernels: {step_us:.1f} us per step.\n\n")
        f.write("```\n")
        for key, v in total.items():
            f.write(f"kernel_avg_us.{key} = {v:.2f}\n")
        f.write(f"steps = {steps}\nsource_digest = {digest}\n```\n")
    print(f"wrote {path}")


def read_stats(workload: str, digest: str):
    path = os.path.join(PROFILES, f"kernel_stats_{workload}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if " = " in line:
            a, b = line.split(" = ", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_digest") != digest:
        return None
    us = {k_.split(".", 1)[1]: float(v) for k_, v in kv.items() if k_.startswith("kernel_avg_us.")}
    return {"kernel_us": us, "path": os.path.relpath(path, ROOT)}


SQ_PASS1 = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
            "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE")
SQ_PASS2 = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
            "SQ_ACTIVE_INST_ANY SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE")


def _counters_by_kernel(counter_csv: str, skip_first: int = 1):
    """{step kernel: {counter: mean per dispatch}} from a counter pass over
    the training step (counters summed over their instances per dispatch;
    the first `skip_first` dispatches of each kernel, the warm-up, left out)."""
    import collections
    import csv

    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(counter_csv)):
        per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for did in sorted(per):
        key = next((v for k_, v in STEP_KERNELS.items() if k_ in names[did]), None)
        if key is not None:
            out[key].append(per[did])
    res = {}
    for key, lst in out.items():
        lst = lst[skip_first:] or lst
        res[key] = {c: sum(d.get(c, 0.0) for d in lst) / len(lst) for c in set().union(*lst)}
    return res


def write_sq(dir1: str, dir2: str):
    """profiles/sq_counters_<training step>.md from the two SQ counter passes
    (dir1 also holds a kernel trace of its run, for the clock)."""
    import csv
    import collections

    import fa_synth
    w = fa_synth.TRAIN_STEP
    p1 = _counters_by_kernel(os.path.join(dir1, "run_counter_collection.csv"))
    p2 = _counters_by_kernel(os.path.join(dir2, "run_counter_collection.csv"))
    dur = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(dir1, "run_kernel_trace.csv"))):
        key = next((v for k_, v in STEP_KERNELS.items() if k_ in r["Kernel_Name"]), None)
        if key is not None:
            dur[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    rows = []
    for key in ("fa_fwd", "bwd_dkdv", "bwd_dq", "bwd_delta"):
        a, b = p1.get(key), p2.get(key)
        if not a or not b:
            continue
        ds = dur[key][1:] or dur[key]
        t = sum(ds) / len(ds)
        gui = a["GRBM_GUI_ACTIVE"] / 8  # summed over the 8 XCDs
        clock = gui / t / 1e9
        mf = b.get("SQ_INSTS_MFMA", 0.0)
        wc = a["SQ_WAVE_CYCLES"]
        per_mf = (lambda x: f"{x / mf:.2f}") if mf else (lambda x: "-")
        busy = f"{100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * gui):.1f}%" if mf else "-"
        conf = 100 * a["SQ_LDS_BANK_CONFLICT"] / a["SQ_LDS_IDX_ACTIVE"] if a["SQ_LDS_IDX_ACTIVE"] else 0.0
        rows.append(f"| `{key}` | {t * 1e6:.1f} | {clock:.2f} | {mf / 1e6:.2f} | {per_mf(b['SQ_INSTS_VALU'])} | "
                    f"{per_mf(b['SQ_INSTS_LDS'])} | {per_mf(b['SQ_INSTS_SALU'])} | {per_mf(b['SQ_INSTS_VMEM_RD'])} | "
                    f"{100 * a['SQ_WAIT_ANY'] / wc:.1f}% | {100 * a['SQ_WAIT_INST_LDS'] / wc:.1f}% | {conf:.2f}% | "
                    f"{busy} |")
    path = os.path.join(PROFILES, f"sq_counters_{w.name}.md")
    with open(path, "w") as f:
        f.write(f"# SQ counters and shader clock of the training-step kernels ({w.describe()})\n\n")
        f.write("Commands (repo root on the MI355X box, `TMPDIR=/tmp`), two passes of their own:\n\n```\n"
                f"rocprofv3 --pmc {SQ_PASS1} --kernel-trace --output-format csv -d gpurun_out/sq1 -o run -- \\\n"
                "    python3 bench.py --steps 2 --warmup 1 --legs 0 --cpu-baseline 0 --ceilings 0\n"
                f"rocprofv3 --pmc {SQ_PASS2} --output-format csv -d gpurun_out/sq2 -o run -- \\\n"
                "    python3 bench.py --steps 2 --warmup 1 --legs 0 --cpu-baseline 0 --ceilings 0\n"
                "python3 bench.py --sq-write gpurun_out/sq1 gpurun_out/sq2\n```\n\n")
        f.write("Per dispatch, averaged over each kernel's dispatches after its first (the warm-up).  Time: the "
                "kernel trace of the first pass (counters slow it little).  Clock: GRBM_GUI_ACTIVE (GPU-busy "
                "cycles, summed over the 8 XCDs) / 8 / time -- the shader clock the chip held under the kernel "
                "(for a kernel of a few tens of microseconds, such as bwd_delta, the counter window runs past "
                "the traced duration and the figure reads high).  "
                "Instruction counts are wave instructions (one MFMA is one 32x32x16 product, 32768 flops); the "
                "'per MFMA' columns divide by the MFMA count.  Waits are fractions of SQ_WAVE_CYCLES.  MFMA busy "
                "= SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8): the fraction of SIMD cycles "
                "the matrix cores were busy, at the clock held.\n\n")
        f.write("| kernel | time (us) | clock (GHz) | MFMA (M) | VALU / MFMA | LDS / MFMA | SALU / MFMA | "
                "VMEM rd / MFMA | wait, any | wait, LDS | LDS bank conflicts / LDS active | MFMA busy |\n"
                "|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        f.write("\n".join(rows) + "\n\n")
        f.write(f"```\nsource_digest = {source_digest()}\n```\n")
    print(f"wrote {path}")


def write_legs_stats(trace_csv: str):
    """profiles/kernel_stats_bench_legs.md: every kernel of a full bench run
    (step and legs), grouped by kernel and launch shape."""
    import collections
    import csv
    import re

    grp = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        if "fa::" not in name:
            continue
        # the anonymous namespace goes before the argument list is cut at its "("
        short = name.replace("(anonymous namespace)::", "")
        short = re.sub(r"\(.*$", "", short).replace("void ", "").replace("fa::", "")
        key = (short, int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])), int(r["Workgroup_Size_X"]))
        grp[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    path = os.path.join(PROFILES, "kernel_stats_bench_legs.md")
    with open(path, "w") as f:
        f.write("# Kernel times of every bench leg (one MI355X)\n\nCommand (repo root on the MI355X box, "
                "`TMPDIR=/tmp`):\n\n```\nrocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/klegs "
                "-o run -- \\\n    python3 bench.py --steps 5 --warmup 2 --cpu-baseline 0\n"
                "python3 bench.py --legs-stats gpurun_out/klegs/run_kernel_trace.csv\n```\n\n"
                "Durations from the kernel trace (end - start per dispatch), grouped by kernel and launch shape "
                "(workgroups x threads); warm-up calls included, so the median is the figure to read.  The "
                "workloads behind each launch shape are the bench legs'.\n\n"
                "| kernel | workgroups x threads | dispatches | median (us) | min (us) |\n|---|---|---|---|---|\n")
        for (short, wgs, nt), d in sorted(grp.items()):
            d.sort()
            f.write(f"| `{short}` | {wgs} x {nt} | {len(d)} | {d[len(d) // 2]:.1f} | {d[0]:.1f} |\n")
        f.write(f"\n```\nsource_digest = {source_digest()}\n```\n")
    print(f"wrote {path}")


# ---------------------------------------------------------------------------
# HBM traffic of the fused forward against the naive three-kernel path, from
# counters ("Flash Attention -- five lessons converging into 80 lines",
# Lessons 1-2: the naive path's N^2 round trips against the fused path's
# N d; "Flash Attention: IO-awareness principle", the S+P traffic table).
# ---------------------------------------------------------------------------
def traffic_leg_workloads():
    import fa_synth
    return tuple(fa_synth.NONCAUSAL_SWEEP) + (fa_synth.LONG_CAUSAL,)


def run_traffic_legs(torch, fa, fa_synth, dev, calib_mib: int):
    """Calibration copy, then per workload: the fused forward twice, the
    naive forward twice (three kernels each), in this fixed order."""
    if calib_mib <= 0:
        sys.exit("--traffic-legs needs --calib-copy-mib")
    src = torch.ones(calib_mib * (1 << 18), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    for w in traffic_leg_workloads():
        q, k, v = (t.to(dev) for t in fa_synth.workload_inputs(w, with_dout=False))
        o, lse = fa.fwd(q, k, v, w.scale, w.causal)
        fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        s_ws = torch.empty((w.B, w.H, w.N, w.N), dtype=torch.float16, device=dev)
        p_ws = torch.empty_like(s_ws)
        for _ in range(2):
            fa.naive_fwd(q, k, v, w.scale, w.causal, out=o, lse=lse, s_ws=s_ws, p_ws=p_ws)
        torch.cuda.synchronize()
        log(f"[bench] traffic legs: {w.name} done")
        del q, k, v, o, lse, s_ws, p_ws
        torch.cuda.empty_cache()


def _counter_dispatches(path: str, counter: str):
    """[(dispatch id, kernel name, summed value)] of one counter, in order."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        name, val = acc.get(did, (r["Kernel_Name"], 0.0))
        acc[did] = (name, val + float(r["Counter_Value"]))
    return [(did, n, v) for did, (n, v) in sorted(acc.items())]


def write_traffic_legs(fetch_csv: str, write_csv: str, calib_mib: int):
    if calib_mib <= 0:
        sys.exit("--traffic-legs-write needs the --calib-copy-mib the counter runs used")
    rows = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        ds = _counter_dispatches(path, counter)
        calib = [v for _, n, v in ds if "elementwise" in n and "add" in n]
        if not calib:
            sys.exit(f"{path}: no calibration copy")
        scale = calib_mib * 1024.0 / (sum(calib) / len(calib))
        fused_k = ("fwd16_kernel", "fwd16_split_kernel")  # the persistent or the key-split forward
        seq = [(n, v * scale * 1024.0) for _, n, v in ds if any(x in n for x in fused_k) or "naive_" in n]
        per_leg = 2 + 2 * 3
        legs = traffic_leg_workloads()
        if len(seq) != per_leg * len(legs):
            sys.exit(f"{path}: {len(seq)} attention dispatches, expected {per_leg * len(legs)}")
        for li, w in enumerate(legs):
            part = seq[li * per_leg:(li + 1) * per_leg]
            fused = [b for n, b in part[:2]]
            assert all(any(x in n for x in fused_k) for n, _ in part[:2]), part[:2]
            naive = part[2:]
            kinds = ("qk", "softmax", "pv")
            for j, (n, _) in enumerate(naive):
                assert f"naive_{kinds[j % 3]}" in n, (n, kinds[j % 3])
            nb = {kd: sum(b for (n, b) in naive[j::3]) / 2 for j, kd in enumerate(kinds)}
            r = rows.setdefault(w.name, {"w": w, "scale": {}})
            r["kernel"] = "key-split" if "fwd16_split_kernel" in part[0][0] else "persistent"
            r[counter] = {"fused": sum(fused) / 2, **nb}
            r["scale"][counter] = scale
    digest = digest_of(TRAFFIC_LEG_SOURCES)
    path = os.path.join(PROFILES, "traffic_naive_vs_fused.md")
    with open(path, "w") as f:
        f.write("# HBM-side bytes: fused forward against the naive three-kernel path\n\n")
        f.write("Command (repo root on the MI355X box, `TMPDIR=/tmp`), two counter passes of their own:\n\n```\n")
        for c, d in (("FETCH_SIZE", "tl_fetch"), ("WRITE_SIZE", "tl_write")):
            f.write(f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/{d} -o run -- \\\n"
                    f"    python3 bench.py --traffic-legs --calib-copy-mib {calib_mib}\n")
        f.write(f"python3 bench.py --traffic-legs-write gpurun_out/tl_fetch/run_counter_collection.csv "
                f"gpurun_out/tl_write/run_counter_collection.csv --calib-copy-mib {calib_mib}\n```\n\n")
        f.write("Bytes past L2 (HBM or the memory-side cache) per call: FETCH_SIZE and WRITE_SIZE (KiB per "
                "dispatch) scaled by what the same counters read for an elementwise copy of "
                f"{calib_mib} MiB in and {calib_mib} MiB out (read scale "
                f"{rows[traffic_leg_workloads()[0].name]['scale']['FETCH_SIZE']:.3f}, write scale "
                f"{rows[traffic_leg_workloads()[0].name]['scale']['WRITE_SIZE']:.3f}), averaged over two calls. "
                "Model bytes: fused = Q, K, V read and O written once (+ fp32 LSE); naive = that plus S and P "
                "each written once and read once, 4 N^2 float16 elements per head.\n\n")
        f.write("| workload | N | fused kernel | fused, counters (MB) | fused, model (MB) | naive QK^T (MB) | "
                "naive softmax (MB) | naive PV (MB) | naive, counters (MB) | naive, model (MB) | ratio, counters | "
                "ratio, model |\n")
        f.write("|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        machine = []
        for name, r in rows.items():
            w = r["w"]
            fu = r["FETCH_SIZE"]["fused"] + r["WRITE_SIZE"]["fused"]
            nk = {kd: r["FETCH_SIZE"][kd] + r["WRITE_SIZE"][kd] for kd in ("qk", "softmax", "pv")}
            nt = sum(nk.values())
            fm = fused_fwd_bytes(w.B, w.H, w.N, w.d, 2)
            nm = naive_fwd_bytes(w.B, w.H, w.N, w.d, 2, 2)
            f.write(f"| `{name}` | {w.N} | {r['kernel']} | {fu / 1e6:.2f} | {fm / 1e6:.2f} | {nk['qk'] / 1e6:.1f} | "
                    f"{nk['softmax'] / 1e6:.1f} | {nk['pv'] / 1e6:.1f} | {nt / 1e6:.1f} | {nm / 1e6:.1f} | "
                    f"{nt / fu:.1f} | {nm / fm:.1f} |\n")
            machine.append(f"{name}.fused_counter_bytes = {fu:.0f}")
            machine.append(f"{name}.naive_counter_bytes = {nt:.0f}")
        f.write("\n```\n" + "\n".join(machine) + f"\nsource_digest = {digest}\n```\n")
    print(f"wrote {path}")


def decode_traffic_workloads():
    import fa_synth
    return (fa_synth.GQA_DECODE, fa_synth.GQA_DECODE_RAGGED)


def decode_inputs(torch, fa, fa_synth, w, dev):
    q, k, v, lens = (t.to(dev) for t in fa_synth.make_decode_inputs(
        w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, w.seed, ragged="ragged" in w.name))
    parts = fa.decode_plan(w.B, w.H, w.kv_heads, w.N, w.d)
    ws = torch.empty(max(1, fa.decode_workspace_bytes(w.B, w.H, w.kv_heads, w.d, parts)), dtype=torch.uint8,
                     device=dev)
    return q, k, v, lens, parts, ws


def decode_alg_bytes(w, lens_sum: float) -> float:
    """K and V read once over the valid lengths, q read, O (16-bit) and the
    fp32 LSE written."""
    return lens_sum * w.kv_heads * w.d * 2 * 2 + 2 * w.B * w.H * w.d * 2 + 4 * w.B * w.H


def run_decode_traffic(torch, fa, fa_synth, dev, calib_mib: int):
    """Calibration copy, then each decode workload twice (split and merge
    kernels), in this fixed order."""
    if calib_mib <= 0:
        sys.exit("--decode-traffic needs --calib-copy-mib")
    src = torch.ones(calib_mib * (1 << 18), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    for w in decode_traffic_workloads():
        q, k, v, lens, parts, ws = decode_inputs(torch, fa, fa_synth, w, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        for _ in range(2):
            fa.decode(q, k, v, w.scale, kv_lens=lens, n_parts=parts, out=o, lse=lse, ws=ws)
        torch.cuda.synchronize()
        log(f"[bench] decode traffic: {w.name} done")
        del q, k, v, lens, ws, o, lse
        torch.cuda.empty_cache()


def write_decode_traffic(fetch_csv: str, write_csv: str, calib_mib: int):
    import fa_synth
    import torch
    if calib_mib <= 0:
        sys.exit("--decode-traffic-write needs the --calib-copy-mib the counter runs used")
    ws = decode_traffic_workloads()
    rows = {w.name: {"w": w} for w in ws}
    scales = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        ds = _counter_dispatches(path, counter)
        calib = [v for _, n, v in ds if "elementwise" in n and "add" in n]
        if not calib:
            sys.exit(f"{path}: no calibration copy")
        scale = calib_mib * 1024.0 / (sum(calib) / len(calib))
        scales[counter] = scale
        seq = [(n, v * scale * 1024.0) for _, n, v in ds if "decode_" in n]
        per = 4  # two calls of split + merge
        if len(seq) != per * len(ws):
            sys.exit(f"{path}: {len(seq)} decode dispatches, expected {per * len(ws)}")
        for wi, w in enumerate(ws):
            part = seq[wi * per:(wi + 1) * per]
            for j, (n, _) in enumerate(part):
                assert ("decode_split" if j % 2 == 0 else "decode_merge") in n, (n, j)
            rows[w.name][counter] = {"split": (part[0][1] + part[2][1]) / 2, "merge": (part[1][1] + part[3][1]) / 2}
    digest = digest_of(("fa_decode.hip", "fa_device.hpp", "fa_plan.hpp"))
    path = os.path.join(PROFILES, "traffic_decode.md")
    with open(path, "w") as f:
        f.write("# HBM-side bytes of a decode step (split and merge kernels)\n\n")
        f.write("Command (repo root on the MI355X box, `TMPDIR=/tmp`), two counter passes of their own:\n\n```\n")
        for c, d in (("FETCH_SIZE", "dt_fetch"), ("WRITE_SIZE", "dt_write")):
            f.write(f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/{d} -o run -- \\\n"
                    f"    python3 bench.py --decode-traffic --calib-copy-mib {calib_mib}\n")
        f.write(f"python3 bench.py --decode-traffic-write gpurun_out/dt_fetch/run_counter_collection.csv "
                f"gpurun_out/dt_write/run_counter_collection.csv --calib-copy-mib {calib_mib}\n```\n\n")
        f.write("Bytes past L2 (HBM or the memory-side cache) per call: FETCH_SIZE and WRITE_SIZE (KiB per "
                "dispatch) scaled by what the same counters read for an elementwise copy of "
                f"{calib_mib} MiB in and {calib_mib} MiB out (read scale {scales['FETCH_SIZE']:.3f}, write scale "
                f"{scales['WRITE_SIZE']:.3f}), averaged over two calls. Algorithmic bytes: K and V read once over "
                "the valid lengths, q read, O and the LSE written.\n\n")
        f.write("| workload | split read (MB) | split write (MB) | merge read (MB) | merge write (MB) | "
                "total (MB) | algorithmic (MB) | total / algorithmic |\n|---|---|---|---|---|---|---|---|\n")
        machine = []
        for name, r in rows.items():
            w = r["w"]
            lens = fa_synth.make_decode_inputs(w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, w.seed,
                                               ragged="ragged" in w.name)[3]
            alg = decode_alg_bytes(w, float(lens.sum().item()))
            fe, wr = r["FETCH_SIZE"], r["WRITE_SIZE"]
            tot = fe["split"] + wr["split"] + fe["merge"] + wr["merge"]
            f.write(f"| `{name}` | {fe['split'] / 1e6:.1f} | {wr['split'] / 1e6:.2f} | {fe['merge'] / 1e6:.2f} | "
                    f"{wr['merge'] / 1e6:.3f} | {tot / 1e6:.1f} | {alg / 1e6:.1f} | {tot / alg:.3f} |\n")
            machine.append(f"{name}.counter_bytes = {tot:.0f}")
        f.write("\n```\n" + "\n".join(machine) + f"\nsource_digest = {digest}\n```\n")
    print(f"wrote {path}")


def read_traffic_legs(digest: str):
    path = os.path.join(PROFILES, "traffic_naive_vs_fused.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if " = " in line:
            a, b = line.split(" = ", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_digest") != digest:
        return None
    out = {}
    for k_, v in kv.items():
        if "." in k_ and k_.endswith("_counter_bytes"):
            leg, field_ = k_.split(".", 1)
            out.setdefault(leg, {})[field_] = float(v)
    return out


def run_legs(torch, fa, fa_synth, dev):
    legs = {}

    # causal prefill forward and long causal forward (bf16), and the
    # non-causal d = 128 forwards beside them
    for w in (fa_synth.CAUSAL_PREFILL, fa_synth.LONG_CAUSAL, fa_synth.NONCAUSAL_PREFILL, fa_synth.NONCAUSAL_LONG):
        q, k, v = (t.to(dev) for t in fa_synth.workload_inputs(w, with_dout=False))
        o, lse = fa.fwd(q, k, v, w.scale, w.causal)
        fn = lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        ms_single, ms_min = time_reps(fn, 20, torch)
        ms = time_back_to_back(fn, torch)
        tf = fwd_flops(w.B, w.H, w.N, w.d, w.causal) / (ms * 1e-3) / 1e12
        alg_bytes = fused_fwd_bytes(w.B, w.H, w.N, w.d, 2)
        entry = {"fwd_ms": ms, "fwd_ms_single_call": ms_single, "fwd_ms_min_single_call": ms_min,
                 "fwd_tflops": tf, "frac_mfma_peak": tf / PEAK_BF16_TFLOPS, "alg_bytes": alg_bytes}
        if w.naive:
            entry.update(naive_leg(torch, fa, w, q, k, v, dev, ms))
        legs[w.name] = entry
        log(f"[bench] {w.name}: {entry}")
        del q, k, v, o, lse
        torch.cuda.empty_cache()

    # FP8 (E4M3) causal prefill, against the dense fp8 MFMA peak
    w = fa_synth.FP8_PREFILL
    q8, k8, v8, ds = fa_synth.make_fp8_inputs(w.B, w.H, w.H, w.N, w.d, seed=w.seed)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o, lse = fa.fwd_fp8(q8, k8, v8, ds, w.scale, w.causal)
    fn = lambda: fa.fwd_fp8(q8, k8, v8, ds, w.scale, w.causal, out=o, lse=lse)
    ms_single, ms_min = time_reps(fn, 20, torch)
    ms = time_back_to_back(fn, torch)
    tf = fwd_flops(w.B, w.H, w.N, w.d, w.causal) / (ms * 1e-3) / 1e12
    entry = {"fwd_ms": ms, "fwd_ms_single_call": ms_single, "fwd_ms_min_single_call": ms_min, "fwd_tflops": tf,
             "frac_fp8_mfma_peak": tf / PEAK_FP8_TFLOPS,
             "alg_bytes": w.B * w.H * (3 * w.N * w.d + 2 * w.N * w.d + 4 * w.N)}
    legs[w.name] = entry
    log(f"[bench] {w.name}: {entry}")
    del q8, k8, v8, o, lse
    torch.cuda.empty_cache()

    # grouped-query causal prefill: forward and backward through the grouped
    # entry points, next to the per-head path on K/V repeated G times
    w = fa_synth.GQA_PREFILL
    q, k, v, do = (t.to(dev) for t in fa_synth.workload_inputs(w))
    G = w.H // w.kv_heads
    o, lse = fa.fwd_gqa(q, k, v, w.scale, w.causal)
    ms_f = time_back_to_back(lambda: fa.fwd_gqa(q, k, v, w.scale, w.causal, out=o, lse=lse), torch)
    f32 = dict(dtype=torch.float32, device=dev)
    bufs = dict(delta=torch.empty((w.B, w.H, w.N), **f32), dq=torch.empty((w.B, w.H, w.N, w.d), **f32),
                dk=torch.empty((w.B, w.kv_heads, w.N, w.d), **f32), dv=torch.empty((w.B, w.kv_heads, w.N, w.d), **f32))
    ms_b = time_back_to_back(lambda: fa.bwd_gqa(q, k, v, o, do, lse, w.scale, w.causal, **bufs), torch)
    del bufs
    kr, vr = k.repeat_interleave(G, dim=1).contiguous(), v.repeat_interleave(G, dim=1).contiguous()
    ms_rep = time_back_to_back(lambda: fa.fwd(q, kr, vr, w.scale, w.causal, out=o, lse=lse), torch)
    tf_f = fwd_flops(w.B, w.H, w.N, w.d, w.causal) / (ms_f * 1e-3) / 1e12
    tf_b = bwd_flops(w.B, w.H, w.N, w.d, w.causal) / (ms_b * 1e-3) / 1e12
    entry = {"G": G, "fwd_ms": ms_f, "fwd_tflops": tf_f, "fwd_frac_mfma_peak": tf_f / PEAK_BF16_TFLOPS,
             "bwd_ms": ms_b, "bwd_tflops": tf_b, "bwd_frac_mfma_peak": tf_b / PEAK_BF16_TFLOPS,
             "fwd_ms_per_head_path_on_repeated_kv": ms_rep}
    legs[w.name] = entry
    log(f"[bench] {w.name}: {entry}")
    del q, k, v, do, o, lse, kr, vr
    torch.cuda.empty_cache()

    # chunked prefill: 2048 new queries after 14336 cached keys (bottom-right
    # causal mask), grouped K/V heads
    w = fa_synth.CHUNK_PREFILL
    Nk = fa_synth.CHUNK_PREFILL_NK
    q, k, v = (t.to(dev) for t in fa_synth.make_chunk_inputs(w.B, w.H, w.kv_heads, w.N, Nk, w.d, w.dtype, w.seed))
    o, lse = fa.fwd_chunk(q, k, v, w.scale, w.causal)
    fn = lambda: fa.fwd_chunk(q, k, v, w.scale, w.causal, out=o, lse=lse)
    ms_single, ms_min = time_reps(fn, 20, torch)
    ms = time_back_to_back(fn, torch)
    # visible (query, key) pairs: query i sees i + Nk - Nq + 1 keys
    pairs = w.B * w.H * (w.N * (Nk - w.N) + w.N * (w.N + 1) / 2)
    tf = 4.0 * pairs * w.d / (ms * 1e-3) / 1e12
    entry = {"fwd_ms": ms, "fwd_ms_single_call": ms_single, "fwd_ms_min_single_call": ms_min, "Nk": Nk,
             "fwd_tflops": tf, "frac_mfma_peak": tf / PEAK_BF16_TFLOPS}
    legs[w.name] = entry
    log(f"[bench] {w.name}: {entry}")
    del q, k, v, o, lse
    torch.cuda.empty_cache()

    # decode steps (one query per head against a K/V cache): HBM-bound, so
    # reported as K/V bytes read per second against the HBM peak
    for w in decode_traffic_workloads():
        q, k, v, lens, parts, ws = decode_inputs(torch, fa, fa_synth, w, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        fn = lambda: fa.decode(q, k, v, w.scale, kv_lens=lens, n_parts=parts, out=o, lse=lse, ws=ws)
        ms_eager, _ = time_reps(fn, 30, torch)
        ms, calls = time_graph(fn, torch, ms_eager)  # a decode step is short: host launch cost excluded
        alg = decode_alg_bytes(w, float(lens.sum().item()))
        gbs = alg / (ms * 1e-3) / 1e9
        entry = {"decode_us": ms * 1e3, "decode_us_eager_call": ms_eager * 1e3, "graph_calls": calls,
                 "parts": parts, "alg_bytes": alg, "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS}
        legs[w.name] = entry
        log(f"[bench] {w.name}: {entry}")
        del q, k, v, lens, ws, o, lse
        torch.cuda.empty_cache()

    # non-causal fp16 sweep, fused vs naive, with the byte models.  These
    # calls are short (tens of microseconds at N = 512), so one call between
    # two events mostly measures the host launch; fwd_ms is the per-call time
    # of back-to-back calls replayed from a HIP graph, and fwd_ms_eager_call
    # the single-call figure beside it.
    for w in fa_synth.NONCAUSAL_SWEEP:
        q, k, v = (t.to(dev) for t in fa_synth.workload_inputs(w, with_dout=False))
        o, lse = fa.fwd(q, k, v, w.scale, w.causal)
        fn = lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        ms_eager, _ = time_reps(fn, 20, torch)
        ms, calls = time_graph(fn, torch, ms_eager)
        tf = fwd_flops(w.B, w.H, w.N, w.d, False) / (ms * 1e-3) / 1e12
        entry = {"fwd_ms": ms, "fwd_tflops": tf, "fwd_ms_eager_call": ms_eager, "graph_calls": calls,
                 "alg_bytes": fused_fwd_bytes(w.B, w.H, w.N, w.d, 2)}
        entry.update(naive_leg(torch, fa, w, q, k, v, dev, ms))
        legs[w.name] = entry
        log(f"[bench] {w.name}: {entry}")
        del q, k, v, o, lse
        torch.cuda.empty_cache()

    # FA1 loop order (K/V outer, running O/l/m through global memory, one
    # workgroup per head) against the fused FA2-order forward
    for w in (fa_synth.NONCAUSAL_SWEEP[1], fa_synth.NONCAUSAL_SWEEP[3], fa_synth.TRAIN_STEP):
        q, k, v = (t.to(dev) for t in fa_synth.workload_inputs(w, with_dout=False))
        ws = torch.empty(fa.fa1_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        fa.fwd_fa1(q, k, v, w.scale, w.causal, out=o, lse=lse, ws=ws)
        ms1, _ = time_reps(lambda: fa.fwd_fa1(q, k, v, w.scale, w.causal, out=o, lse=lse, ws=ws), 3, torch)
        ms2, _ = time_reps(lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse), 10, torch)
        # FA1's compulsory traffic: K, V once; per (key block, query block)
        # step Q_i read, O_i (fp32) read and written, m_i and l_i read and
        # written; then O and LSE written.
        tc, tr, br, bc = -(-w.N // 64), -(-w.N // 128), 128, 64
        steps = sum(tr - ((j * bc) // br if w.causal else 0) for j in range(tc))
        e = 2
        fa1_bytes = w.B * w.H * (2 * w.N * w.d * e + steps * br * (w.d * e + 2 * w.d * 4 + 4 * 4)
                                 + w.N * w.d * e + 4 * w.N)
        entry = {"fa1_ms": ms1, "fa2_ms": ms2, "fa2_speedup_over_fa1": ms1 / ms2,
                 "fa1_tflops": fwd_flops(w.B, w.H, w.N, w.d, w.causal) / (ms1 * 1e-3) / 1e12,
                 "fa1_model_bytes": fa1_bytes, "fa2_model_bytes": fused_fwd_bytes(w.B, w.H, w.N, w.d, e),
                 "fa1_model_gbs": fa1_bytes / (ms1 * 1e-3) / 1e9}
        legs[f"fa1_ablation_{w.name}"] = entry
        log(f"[bench] fa1_ablation_{w.name}: {entry}")
        del q, k, v, ws, o, lse
        torch.cuda.empty_cache()

    # fp32 single head (graph-replayed like the sweep: one call is short)
    w = fa_synth.SINGLE_HEAD_F32
    q, k, v = (t.to(dev) for t in fa_synth.workload_inputs(w, with_dout=False))
    o, lse = fa.fwd(q, k, v, w.scale, w.causal)
    fn = lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
    ms_eager, _ = time_reps(fn, 50, torch)
    ms, calls = time_graph(fn, torch, ms_eager)
    entry = {"fwd_ms": ms, "fwd_gflops": fwd_flops(1, 1, w.N, w.d, False) / (ms * 1e-3) / 1e9,
             "fwd_ms_eager_call": ms_eager, "graph_calls": calls}
    entry.update(naive_leg(torch, fa, w, q, k, v, dev, ms))
    legs[w.name] = entry
    log(f"[bench] {w.name}: {entry}")
    return legs


def naive_leg(torch, fa, w, q, k, v, dev, fused_ms):
    """Time the three-kernel path and report its byte model next to the
    fused one: S and P each written once and read once (N^2 elements of the
    workspace dtype), plus Q, K, V, O and LSE."""
    ws_dtype = torch.float32 if w.dtype == "f32" else torch.float16
    e_ws = 4 if w.dtype == "f32" else 2
    e_in = 4 if w.dtype == "f32" else 2
    s = torch.empty((w.B, w.H, w.N, w.N), dtype=ws_dtype, device=dev)
    p = torch.empty_like(s)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    fn = lambda: fa.naive_fwd(q, k, v, w.scale, w.causal, out=o, lse=lse, s_ws=s, p_ws=p)
    fn()
    ms_eager, _ = time_reps(fn, 5, torch)
    ms, calls = time_graph(fn, torch, ms_eager, reps=5)
    naive_bytes = naive_fwd_bytes(w.B, w.H, w.N, w.d, e_in, e_ws)
    fused_bytes = fused_fwd_bytes(w.B, w.H, w.N, w.d, e_in)
    del s, p, o, lse
    torch.cuda.empty_cache()
    return {"naive_ms": ms, "naive_ms_eager_call": ms_eager, "naive_graph_calls": calls,
            "speedup_fused_over_naive": ms / fused_ms, "naive_model_bytes": naive_bytes,
            "fused_model_bytes": fused_bytes, "model_byte_ratio": naive_bytes / fused_bytes,
            "naive_model_gbs": naive_bytes / (ms * 1e-3) / 1e9}


if __name__ == "__main__":
    main()
