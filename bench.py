"""Benchmark: GQA decode over a KV cache (HBM-bound) and causal prefill
(MFMA-bound) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one decode call (all query heads of every sequence against its
cached prefix) on the headline workload: B=8, Hq=32, Hkv=8, d=128, 8000
cached cells per sequence, bf16 storage, iid N(0,1) synthetic inputs.  The
inputs are resident in HBM before timing starts.  Four copies of the K/V cache
are rotated so that no step finds its cache in the 256 MB Infinity Cache left
over from the previous step.

Prints ONE JSON line.  `value` is algorithmic HBM GB/s (K/V cells read once
per KV group, plus Q and O) over the timed steps; `roofline` relates the decode
kernel's own per-launch duration (HIP events on its stream) to the 8 TB/s HBM
peak; `prefill` reports the causal prefill (B=1, T=4096, Hq=32, Hkv=8,
d=128) in TFLOP/s against the 2.5 PFLOP/s dense bf16 peak; `cpu_baseline`
times the fp64 oracle on the host cores on the same decode workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def decode_bytes(B, Hq, Hkv, d, cells, elem=2):
    """K and V cells read once per KV group, plus Q read and O written."""
    kv = 2 * B * Hkv * cells * d * elem
    return kv + 2 * B * Hq * d * elem


def prefill_flops(Hq, d, T, B=1):
    """4*d flops (QK^T and PV multiply-adds) per permitted (query, key) pair."""
    return 4 * Hq * d * B * T * (T + 1) // 2


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def bench_decode(torch, gqa, synth, steps, warmup):
    cfg = synth.CONFIGS["decode_b8_hq32_hkv8_d128_n8000"]
    B, C, hq, hkv, d, n = cfg["B"], cfg["C"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["n"]
    dev = torch.device("cuda:0")
    copies = 4
    q, k0, v0 = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
    ks, vs = [k0], [v0]
    for i in range(1, copies):
        _, k, v = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, cfg["seed"] + 100 * i, dev)
        ks.append(k)
        vs.append(v)
    seqlens = torch.full((B,), n, dtype=torch.int32, device=dev)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(1, gqa.decode_workspace_bytes(B, C, hq, hkv, d)), dtype=torch.uint8,
                     device=dev)
    kernel = gqa.decode_kernel(B, C, hq, hkv, d)

    def step(i):
        gqa.decode(q, ks[i % copies], vs[i % copies], seqlens=seqlens, out=out, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch durations, events on the launch stream (torch's current stream)
    ev = _events(torch, 2 * steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_all = torch.cuda.Event(enable_timing=True)
    end_all = torch.cuda.Event(enable_timing=True)
    start_all.record()
    for i in range(steps):
        ev[2 * i].record()
        step(i)
        ev[2 * i + 1].record()
    end_all.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start_all.elapsed_time(end_all)
    per_launch = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    nbytes = decode_bytes(B, hq, hkv, d, n)
    ms = total_ms / steps
    avg_launch_ms = sum(per_launch) / steps
    return dict(cfg=cfg, kernel=kernel, ms=ms, wall_s=wall, avg_launch_ms=avg_launch_ms,
                min_launch_ms=min(per_launch), nbytes=nbytes, q=q, k=k0, v=v0, seqlens=[n] * B)


def bench_prefill(torch, gqa, synth, steps, warmup):
    cfg = synth.CONFIGS["prefill_b1_t4096_hq32_hkv8_d128"]
    B, T, hq, hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    dev = torch.device("cuda:0")
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
    out = torch.empty((B, T, hq, d), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        gqa.prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    ev = _events(torch, 2 * steps)
    for i in range(steps):
        ev[2 * i].record()
        gqa.prefill(q, k, v, out=out)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    ms = sum(per) / steps
    flops = prefill_flops(hq, d, T, B)
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(workload="gqa_prefill_b1_t4096_hq32_hkv8_d128_causal_bf16",
                kernel=gqa.prefill_kernel(B, T, T, hq, hkv, d), ms=round(ms, 5),
                flops=flops, tflops=round(tflops, 2),
                frac_of_bf16_peak=round(tflops / BF16_PEAK_TFLOPS, 4),
                tokens_per_s=round(B * T / (ms * 1e-3), 1))


def cpu_baseline(torch, r, budget_s=12.0):
    """The fp64 oracle as it stands, on the host cores, on the decode workload."""
    import numpy as np

    import oracle

    q = r["q"].float().cpu().numpy().astype(np.float64)
    k = r["k"].float().cpu().numpy().astype(np.float64)
    v = r["v"].float().cpu().numpy().astype(np.float64)
    oracle.lib()
    runs, t_total = 0, 0.0
    while t_total < budget_s and runs < 50:
        t0 = time.perf_counter()
        oracle.decode(q, k, v, seqlens=r["seqlens"])
        t_total += time.perf_counter() - t0
        runs += 1
    per = t_total / runs
    return dict(value=round(r["nbytes"] / per / 1e9, 3), unit="GB/s", cores=oracle.threads(),
                kind="oracle",
                sample=f"full decode workload (B=8, Hq=32, Hkv=8, d=128, 8000 cells) in fp64, "
                       f"{runs} runs, {per:.3f} s each, inputs pre-converted to float64")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode and prefill paths shard over sequences or KV groups with no "
              "exchange, so there is nothing multi-GPU to time here)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gqa_kv_cache_02_amd as gqa
    from gqa_kv_cache_02_amd import synth

    gqa.lib()
    r = bench_decode(torch, gqa, synth, args.steps, args.warmup)
    cfg = r["cfg"]
    gbs = r["nbytes"] / (r["ms"] * 1e-3) / 1e9
    achieved = r["nbytes"] / (r["avg_launch_ms"] * 1e-3) / 1e9
    line = {
        "metric": "GQA decode achieved HBM GB/s & % peak; causal prefill TFLOP/s & % MFMA peak",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gqa_decode_b8_hq32_hkv8_d128_n8000_bf16",
                   "B": cfg["B"], "Hq": cfg["Hq"], "Hkv": cfg["Hkv"], "d": cfg["d"],
                   "cached_cells": cfg["n"], "window": None, "kv_cache_copies_rotated": 4,
                   "kernel": r["kernel"]},
        "tokens_per_s": round(cfg["B"] / (r["ms"] * 1e-3), 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "bytes_per_launch": r["nbytes"],
                     "avg_launch_ms": round(r["avg_launch_ms"], 5),
                     "timing": "HIP events around each decode call on its stream"},
    }
    if not args.no_prefill:
        line["prefill"] = bench_prefill(torch, gqa, synth, max(5, args.steps // 10), 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, r)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
