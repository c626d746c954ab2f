"""Benchmark: GQA decode over a KV cache (HBM-bound) and causal prefill
(MFMA-bound) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-prefill] [--copy-calibration]

A step is one decode call -- every query head of every sequence against its
cached prefix, i.e. the split kernel and the merge kernel -- on the headline
workload: B=8, Hq=32, Hkv=8, d=128, 8000 cached cells per sequence, bf16
storage, iid N(0,1) synthetic inputs resident in HBM before timing starts.
Four copies of the K/V cache are rotated so that no step finds its cache in the
256 MB Infinity Cache left over from the previous step.

Prints ONE JSON line.
  value          algorithmic HBM GB/s (K/V cells read once per KV group, plus
                 Q read and O written) over K back-to-back timed steps.
  roofline       the decode call's own duration (HIP events recorded on the
                 launch stream around each call, second pass; mean, minimum
                 and p10/p50/p90), against the 8 TB/s HBM3E peak.  `traffic`
                 is the HBM bytes per call that rocprofv3 counters measured
                 (profiles/, scaled by a plain copy of known size), reported
                 only while the kernel source still has the hash the counters
                 were taken with.  `hbm_copy_reference_gbs` is a live 1 GiB
                 device copy; frac_of_measured_copy is `value` against it.
  prefill        causal prefill B=1, T=4096, Hq=32, Hkv=8, d=128: TFLOP/s of
                 the permitted pairs (4*d flops each) against 2.5 PFLOP/s
                 dense bf16 MFMA, over back-to-back calls (`per_call`: with
                 events around each call); `mfma_counters` carries the matrix-core busy
                 fraction, clock and executed MFMA work that rocprofv3
                 counters measured (profiles/), while the kernel source still
                 has the hash they were taken with.
  prefix_prefill queries against a cached prefix: the last 512 cells of a
                 4096-cell sequence as new rows (B=1, Hq=32, Hkv=8, d=128):
                 TFLOP/s of the permitted pairs against 2.5 PFLOP/s.
  packed_prefill packed segments: sequences of 64..1024 cells back to back in
                 one 4096-cell causal row (B=1, Hq=32, Hkv=8, d=128), each
                 attending only within itself: TFLOP/s of the permitted pairs
                 against 2.5 PFLOP/s.
  ring_decode    decode over a rolling cache of capacity w = 4096 with the new
                 cell committed in the call (B=32, Hq=8, Hkv=2, d=64, ragged
                 lengths in [1, 32768]): GB/s of the K/V cells in each row's
                 window read once per KV group, against 8 TB/s.
  decode_sweep   the endpoint sweep B=16, Hq=8, d=128, 8000 cells at Hkv = 8,
                 2, 1 (MHA, GQA, MQA): GB/s of K/V read once per KV group.
  ragged_window_decode  B=32, Hq=8, Hkv=2, d=64, lengths in [1, 32768],
                 window 4096, linear cache: GB/s of the cells in the windows.
  small_f32_prefill  the fp32 prefill B=1, T=16, Hq=4, Hkv=2, d=8: us per
                 call (latency only), without a window and with window 2.
  The prefix, packed, rolling-cache, sweep and ragged legs time back-to-back calls
  between two events, like `value`; `per_call_ms` adds events around each
  call, which for calls shorter than the binding's host time per call
  measures the host.
  cpu_baseline   the fp64 oracle (plain C, OpenMP) on the host cores, on the
                 same decode workload; with the CPU model, the process's
                 affinity set and a one-thread figure on one batch row.  Every
                 other leg carries its own `cpu_baseline`: the oracle on that
                 leg's whole workload (same inputs, same unit), with the core
                 count.
  traffic        each leg's HBM bytes per call measured by rocprofv3 counters
                 (profiles/bench_workloads_traffic.txt, one process per leg so
                 that no dispatch is attributed to the wrong leg), while the
                 kernel source still has the hash they were taken with.

    python bench.py --leg NAME [--steps K] [--copy-calibration]
runs one leg only (decode, prefill, prefix, packed, ring, sweep8, sweep2,
sweep1, ragged), for hardware-counter runs; and
    python bench.py --summarize-counters DIR
turns the counter CSVs of those runs (DIR/<leg>/{fetch,write}/...) into the
traffic summary committed under profiles/.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_CAL_BYTES = 1 << 30  # plain copy used to calibrate the traffic counters
DECODE_SRC = os.path.join(ROOT, "gqa_kv_cache_02_amd", "csrc", "gqa_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bench_workloads_traffic.txt")
PREFILL_SRC = os.path.join(ROOT, "gqa_kv_cache_02_amd", "csrc", "gqa_prefill.hip")
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_b1_t4096_hq32_hkv8_d128_mfma_counters.txt")


def decode_bytes(B, Hq, Hkv, d, cells, elem=2):
    """K and V cells read once per KV group, plus Q read and O written."""
    kv = 2 * B * Hkv * cells * d * elem
    return kv + 2 * B * Hq * d * elem


def prefill_flops(Hq, d, T, B=1):
    """4*d flops (QK^T and PV multiply-adds) per permitted (query, key) pair."""
    return 4 * Hq * d * B * T * (T + 1) // 2


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_mfma():
    """Matrix-core counters of the causal prefill from the committed rocprofv3
    summary (busy fraction of cycles at the clock the chip held, that clock,
    executed MFMA work), or None when it is missing or was taken on a
    different kernel source."""
    if not os.path.exists(MFMA_FILE):
        return None
    vals = {}
    for ln in open(MFMA_FILE):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("prefill_source_sha256_16") != source_hash(PREFILL_SRC):
        return None
    try:
        return {"mfma_busy_frac": float(vals["mfma_busy_frac"]),
                "sustained_clock_ghz": float(vals["sustained_clock_ghz"]),
                "mfma_gflop_executed": float(vals["mfma_gflop_executed"]),
                "source": "profiles/" + os.path.basename(MFMA_FILE)}
    except (KeyError, ValueError):
        return None


# Legs of the benchmark: the kernel source each one runs, and the library
# kernels of one call (the first is launched once per call).
LEG_SOURCE = {"decode": DECODE_SRC, "ring": DECODE_SRC, "sweep8": DECODE_SRC,
              "sweep2": DECODE_SRC, "sweep1": DECODE_SRC, "ragged": DECODE_SRC,
              "prefill": PREFILL_SRC, "prefix": PREFILL_SRC, "packed": PREFILL_SRC}
LEG_KERNELS = {leg: ("decode_kernel", "decode_merge_kernel") for leg in LEG_SOURCE}
LEG_KERNELS["prefill"] = LEG_KERNELS["prefix"] = LEG_KERNELS["packed"] = \
    ("prefill_mfma_kernel", "prefix_merge_kernel")


def _summary_values(path):
    vals = {}
    for ln in open(path):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def _source_key(src):
    return "prefill_source_sha256_16" if src == PREFILL_SRC else "decode_source_sha256_16"


def measured_traffic(leg="decode"):
    """HBM bytes per call of a leg from the committed counter summary, or None
    when it is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = _summary_values(TRAFFIC_FILE)
    src = LEG_SOURCE[leg]
    if vals.get(_source_key(src)) != source_hash(src):
        return None
    try:
        return int(float(vals[f"{leg}.hbm_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def _counter_rows(dirpath):
    """(dispatch id, kernel name, value in KiB) of every row of the rocprofv3
    counter-collection CSVs under dirpath (one counter per run)."""
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    # a counter read over several instances is one row each: sum per dispatch
    per = {}
    for did, name, val in rows:
        n, v = per.get(did, (name, 0.0))
        per[did] = (n, v + val)
    return [(did, n, v) for did, (n, v) in sorted(per.items())]


def _leg_counter_bytes(rows, leg):
    """Copy-calibration KiB, and (calls, summed KiB over the leg's kernels)."""
    copies = [v for _, n, v in rows if "copy" in n.lower()]
    cal = max(copies) if copies else None
    main, merge = LEG_KERNELS[leg]
    calls = sum(1 for _, n, _ in rows if main in n and "merge" not in n)
    kib = sum(v for _, n, v in rows if (main in n and "merge" not in n) or merge in n)
    return cal, calls, kib


def algorithmic_bytes(leg):
    """The bytes each leg's workload must move, as the bench legs count them
    (None for the causal and prefix prefill legs, whose roofline is
    matrix-core work)."""
    from gqa_kv_cache_02_amd import synth

    if leg == "decode":
        c = synth.CONFIGS["decode_b8_hq32_hkv8_d128_n8000"]
        return decode_bytes(c["B"], c["Hq"], c["Hkv"], c["d"], c["n"])
    if leg.startswith("sweep"):
        c = synth.CONFIGS["decode_sweep_b16_hq8_d128_n8000"]
        return decode_bytes(c["B"], c["Hq"], int(leg[5:]), c["d"], c["n"])
    if leg in ("ragged", "ring"):
        name = "decode_ragged_b32_hq8_hkv2_d64_w4096" if leg == "ragged" \
            else "ring_b32_hq8_hkv2_d64_w4096"
        c = synth.CONFIGS[name]
        lens = synth.ragged_lengths(c["B"], c["n"][0], c["n"][1], c["seed"]).tolist()
        cells = sum(min(int(n), c["window"]) for n in lens)
        nbytes = 2 * c["Hkv"] * cells * c["d"] * 2 + 2 * c["B"] * c["Hq"] * c["d"] * 2
        if leg == "ring":  # the candidate read and committed
            nbytes += 4 * c["B"] * c["Hkv"] * c["d"] * 2
        return nbytes
    if leg == "packed":  # Q and K/V read once, O written once (its roofline is HBM)
        c = synth.CONFIGS["packed_b1_t4096_hq32_hkv8_d128"]
        return 2 * c["B"] * c["T"] * c["d"] * (2 * c["Hq"] + 2 * c["Hkv"])
    return None


def summarize_counters(dirpath):
    """Text of the per-leg traffic summary from counter runs laid out as
    dirpath/<leg>/fetch/... (FETCH_SIZE) and dirpath/<leg>/write/...
    (WRITE_SIZE), each made by `bench.py --leg <leg> --copy-calibration`."""
    cmd_f = ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/<leg>/fetch -o ctr -- "
             "python3 bench.py --leg <leg> --steps 5 --warmup 1 --copy-calibration")
    lines = [
        "# HBM traffic per call of each bench.py leg, from the rocprofv3 counters",
        "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each leg and each counter in a",
        "# process of its own, so that every dispatch of the library's kernels in a run",
        "# belongs to that leg.  Each run also makes a plain 1 GiB device copy; the",
        "# counters are scaled by what they read for it (factor = 1 GiB / counter).",
        "#",
        "# Commands (from the repository root; TMPDIR=/tmp), for every leg in",
        "# decode prefill prefix packed ring sweep8 sweep2 sweep1 ragged:",
        f"#   {cmd_f}",
        "#   (the same with --pmc WRITE_SIZE and -d OUT/<leg>/write)",
        "#   python3 bench.py --summarize-counters OUT",
        "#",
        "# leg       calls  fetch_scale write_scale   read MB  written MB   HBM MB/call  "
        "algorithmic MB  ratio",
    ]
    vals = []
    for leg in LEG_SOURCE:
        fr = _counter_rows(os.path.join(dirpath, leg, "fetch"))
        wr = _counter_rows(os.path.join(dirpath, leg, "write"))
        if not fr or not wr:
            continue
        fcal, fcalls, fkib = _leg_counter_bytes(fr, leg)
        wcal, wcalls, wkib = _leg_counter_bytes(wr, leg)
        if not fcal or not wcal or fcalls == 0 or fcalls != wcalls:
            continue
        fs = COPY_CAL_BYTES / (fcal * 1024.0)
        ws = COPY_CAL_BYTES / (wcal * 1024.0)
        rd = fkib * 1024.0 * fs / fcalls
        wt = wkib * 1024.0 * ws / wcalls
        alg = algorithmic_bytes(leg)
        ratio = f"{(rd + wt) / alg:6.3f}" if alg else "   -  "
        alg_s = f"{alg / 1e6:14.2f}" if alg else "             -"
        lines.append(f"# {leg:8s} {fcalls:6d} {fs:11.4f} {ws:11.4f} {rd / 1e6:9.2f} "
                     f"{wt / 1e6:11.3f} {(rd + wt) / 1e6:13.2f} {alg_s} {ratio}")
        vals.append(f"{leg}.hbm_bytes_per_call = {int(round(rd + wt))}")
    lines.append("#")
    lines.append("# The prefill legs read Q and K/V and write O (and, for the split prefix")
    lines.append("# rows, partials that the merge reads back).  The causal and prefix legs'")
    lines.append("# roofline is matrix-core work; the packed leg's short segments make it HBM.")
    lines += vals
    lines.append(f"decode_source_sha256_16 = {source_hash(DECODE_SRC)}")
    lines.append(f"prefill_source_sha256_16 = {source_hash(PREFILL_SRC)}")
    return "\n".join(lines) + "\n"


def _f64(t):
    """A device tensor's stored values, widened exactly to float64 on the host."""
    import numpy as np

    return t.float().cpu().numpy().astype(np.float64)


def _oracle_baseline(run, work, unit_scale, unit, sample, budget_s=2.0, max_runs=50):
    """The oracle as it stands (`run` calls it on a leg's whole workload, on
    inputs already widened to float64), timed on the host cores: at least one
    run, then more until about budget_s; work / time in the leg's unit."""
    import oracle

    runs, total = 0, 0.0
    while runs == 0 or (total < budget_s and runs < max_runs):
        t0 = time.perf_counter()
        run()
        total += time.perf_counter() - t0
        runs += 1
    per = total / runs
    return dict(value=round(work / per / unit_scale, 5), unit=unit, cores=oracle.threads(),
                kind="oracle", seconds_per_call=round(per, 4),
                sample=f"{sample}; {runs} run(s) of {per:.4f} s; inputs widened to float64 "
                       "before timing")


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
    ws = torch.empty(max(1, gqa.decode_workspace_bytes(B, C, hq, hkv, d)), dtype=torch.uint8,
                     device=dev)
    kernel = gqa.decode_kernel(B, C, hq, hkv, d)

    def step(i):
        gqa.decode(q, ks[i % copies], vs[i % copies], seqlens=seqlens, out=out, workspace=ws)

    for i in range(warmup):
        step(i)
    # timed region: K back-to-back steps, synchronised on both sides
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    # second pass: events on the launch stream around each call
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record()
        step(i)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per_call = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    srt = sorted(per_call)
    pct = lambda f: srt[min(steps - 1, int(f * steps))]
    return dict(cfg=cfg, kernel=kernel, ms=ms, wall_s=wall,
                avg_call_ms=sum(per_call) / steps, min_call_ms=min(per_call),
                p10_call_ms=pct(0.10), p50_call_ms=pct(0.50), p90_call_ms=pct(0.90),
                nbytes=decode_bytes(B, hq, hkv, d, n), q=q, k=k0, v=v0, seqlens=[n] * B)


def bench_prefill(torch, gqa, synth, steps, warmup, cpu=False):
    cfg = synth.CONFIGS["prefill_b1_t4096_hq32_hkv8_d128"]
    B, T, hq, hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    dev = torch.device("cuda:0")
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
    out = torch.empty((B, T, hq, d), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        gqa.prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    # back-to-back calls between two events (as the decode `value`)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        gqa.prefill(q, k, v, out=out)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    # events around each call
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record()
        gqa.prefill(q, k, v, out=out)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    ms_call = sum(per) / steps
    flops = prefill_flops(hq, d, T, B)
    tflops = flops / (ms * 1e-3) / 1e12
    tflops_call = flops / (ms_call * 1e-3) / 1e12
    res = dict(workload="gqa_prefill_b1_t4096_hq32_hkv8_d128_causal_bf16",
               kernel=gqa.prefill_kernel(B, T, T, hq, hkv, d), ms=round(ms, 5),
               flops=flops, tflops=round(tflops, 2),
               frac_of_bf16_peak=round(tflops / BF16_PEAK_TFLOPS, 4),
               tokens_per_s=round(B * T / (ms * 1e-3), 1),
               timing="back-to-back calls between two HIP events on the launch stream",
               per_call={"ms": round(ms_call, 5), "tflops": round(tflops_call, 2),
                         "frac_of_bf16_peak": round(tflops_call / BF16_PEAK_TFLOPS, 4),
                         "timing": "HIP events on the launch stream around each call"},
               mfma_counters=measured_mfma(), traffic=measured_traffic("prefill"))
    if cpu:
        import oracle

        qn, kn, vn = _f64(q), _f64(k), _f64(v)
        res["cpu_baseline"] = _oracle_baseline(
            lambda: oracle.prefill(qn, kn, vn), flops, 1e12, "TFLOP/s",
            "the whole causal prefill workload (B=1, T=4096, Hq=32, Hkv=8, d=128) in fp64",
            budget_s=0.0)
    return res


B2B = "back-to-back calls between two HIP events on the launch stream"
PER_CALL = ("per_call_ms: HIP events on the launch stream around each call; it includes the "
            "binding's host time when a call is shorter than that")


def _time_calls(torch, fn, steps, warmup):
    """(ms per call over `steps` back-to-back calls between two events,
    mean ms with events around each call)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record()
        fn(i)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    return ms, sum(per) / steps


def prefix_flops(Hq, d, C, Tq, B=1):
    """4*d flops per permitted pair; row i of the Tq new ones at cell
    C - Tq + i reads C - Tq + i + 1 keys."""
    pairs = Tq * (C - Tq) + Tq * (Tq + 1) // 2
    return 4 * Hq * d * B * pairs


def bench_prefix(torch, gqa, synth, steps, warmup, cpu=False):
    cfg = synth.CONFIGS["chunk_b1_tq512_c4096_hq32_hkv8_d128"]
    B, Tq, C, hq, hkv, d = cfg["B"], cfg["Tq"], cfg["C"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    dev = torch.device("cuda:0")
    q, k, v = synth.prefill_inputs(B, Tq, hq, hkv, d, torch.bfloat16, cfg["seed"], dev, C=C)
    out = torch.empty((B, Tq, hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, gqa.prefill_prefix_workspace_bytes(B, Tq, C, hq, hkv, d)),
                     dtype=torch.uint8, device=dev)
    ms, ms_call = _time_calls(torch, lambda i: gqa.prefill_prefix(q, k, v, out=out,
                                                                  workspace=ws), steps, warmup)
    flops = prefix_flops(hq, d, C, Tq, B)
    tflops = flops / (ms * 1e-3) / 1e12
    res = dict(workload="gqa_prefill_prefix_b1_tq512_c4096_hq32_hkv8_d128_bf16",
               ms=round(ms, 5), flops=flops, tflops=round(tflops, 2),
               frac_of_bf16_peak=round(tflops / BF16_PEAK_TFLOPS, 4),
               tokens_per_s=round(B * Tq / (ms * 1e-3), 1), per_call_ms=round(ms_call, 5),
               timing=f"{B2B}; {PER_CALL}", traffic=measured_traffic("prefix"))
    if cpu:
        import oracle

        qn, kn, vn = _f64(q), _f64(k), _f64(v)
        res["cpu_baseline"] = _oracle_baseline(
            lambda: oracle.attend_prefix(qn, kn, vn), flops, 1e12, "TFLOP/s",
            "the whole prefix workload (512 new rows against 4096 cells) in fp64")
    return res


def packed_pairs(seg_starts):
    """Permitted pairs of one packed row: a cell at offset i of its segment
    reads the i + 1 cells from the segment start (causal within it)."""
    T = len(seg_starts)
    starts = sorted(set(int(x) for x in seg_starts))
    lens = [b - a for a, b in zip(starts, starts[1:] + [T])]
    return sum(n * (n + 1) // 2 for n in lens), lens


def bench_packed(torch, gqa, synth, steps, warmup, cpu=False):
    cfg = synth.CONFIGS["packed_b1_t4096_hq32_hkv8_d128"]
    B, T, hq, hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    lo, hi = cfg["seg_len"]
    dev = torch.device("cuda:0")
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
    segs_cpu = synth.packed_segment_starts(B, T, lo, hi, cfg["seed"])
    segs = segs_cpu.to(dev)
    out = torch.empty((B, T, hq, d), dtype=torch.bfloat16, device=dev)
    # a full row of new cells (qlens = seqlens = T): the key range is never
    # split, so no workspace
    assert gqa.prefill_prefix_workspace_bytes(B, T, T, hq, hkv, d) == 0
    ms, ms_call = _time_calls(torch, lambda i: gqa.prefill_prefix(q, k, v, seg_starts=segs,
                                                                  out=out), steps, warmup)
    pairs, lens = packed_pairs(segs_cpu[0].tolist())
    flops = 4 * hq * d * B * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    # Q and K/V read once, O written once: with segments this short the
    # workload moves more bytes per flop than the chip's balance point, so
    # its roofline is the larger of the HBM and matrix-core times
    nbytes = algorithmic_bytes("packed")
    t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
    res = dict(workload="gqa_prefill_packed_b1_t4096_hq32_hkv8_d128_bf16",
               segments=lens, ms=round(ms, 5), flops=flops, tflops=round(tflops, 2),
               frac_of_bf16_peak=round(tflops / BF16_PEAK_TFLOPS, 4),
               bytes=nbytes, roofline_bound="hbm" if t_hbm >= t_mfma else "mfma",
               roofline_us=round(max(t_hbm, t_mfma) * 1e6, 2),
               frac_of_roofline=round(max(t_hbm, t_mfma) / (ms * 1e-3), 4),
               tokens_per_s=round(B * T / (ms * 1e-3), 1), per_call_ms=round(ms_call, 5),
               timing=f"{B2B}; {PER_CALL}", traffic=measured_traffic("packed"))
    if cpu:
        import oracle

        qn, kn, vn = _f64(q), _f64(k), _f64(v)
        sn = segs_cpu.numpy()
        res["cpu_baseline"] = _oracle_baseline(
            lambda: oracle.attend_prefix(qn, kn, vn, segs=sn), flops, 1e12, "TFLOP/s",
            f"the whole packed workload ({len(lens)} sequences in one 4096-cell row) in fp64")
    return res


def bench_ring(torch, gqa, synth, steps, warmup, cpu=False):
    cfg = synth.CONFIGS["ring_b32_hq8_hkv2_d64_w4096"]
    B, hq, hkv, d, w = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["window"]
    lo, hi = cfg["n"]
    dev = torch.device("cuda:0")
    lens = synth.ragged_lengths(B, lo, hi, cfg["seed"])
    seqlens = lens.to(dev)
    # 6 rotated copies of the 67 MB rolling cache keep it out of the 256 MB
    # Infinity Cache between steps
    copies = 6
    q, k0, v0 = synth.decode_inputs(B, w, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
    ks, vs = [k0], [v0]
    for i in range(1, copies):
        _, k, v = synth.decode_inputs(B, w, hq, hkv, d, torch.bfloat16, cfg["seed"] + 100 * i, dev)
        ks.append(k)
        vs.append(v)
    kn = synth.randn((B, hkv, d), cfg["seed"] + 50, torch.bfloat16, dev)
    vn = synth.randn((B, hkv, d), cfg["seed"] + 51, torch.bfloat16, dev)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, gqa.decode_workspace_bytes(B, w, hq, hkv, d, w)), dtype=torch.uint8,
                     device=dev)
    # the calls commit their candidate into the cache: keep the cache as it
    # was for the oracle
    k_orig, v_orig = (k0.clone(), v0.clone()) if cpu else (None, None)
    ms, ms_call = _time_calls(torch, lambda i: gqa.decode_cache(q, ks[i % copies], vs[i % copies],
                                                       k_new=kn, v_new=vn, seqlens=seqlens,
                                                       window=w, ring=True, out=out,
                                                       workspace=ws), steps, warmup)
    cells = int(sum(min(int(n), w) for n in lens.tolist()))
    nbytes = 2 * hkv * cells * d * 2 + 2 * B * hq * d * 2 + 4 * B * hkv * d * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = dict(workload="gqa_decode_cache_ring_b32_hq8_hkv2_d64_w4096_bf16",
               ms=round(ms, 5), bytes=nbytes, gbs=round(gbs, 2),
               frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
               tokens_per_s=round(B / (ms * 1e-3), 1), window_cells_read=cells,
               per_call_ms=round(ms_call, 5), timing=f"{B2B}; {PER_CALL}",
               traffic=measured_traffic("ring"))
    if cpu:
        import oracle

        qn, kn0, vn0, knn, vnn = _f64(q), _f64(k_orig), _f64(v_orig), _f64(kn), _f64(vn)
        sl = lens.tolist()
        res["cpu_baseline"] = _oracle_baseline(
            lambda: oracle.decode_cache(qn, kn0, vn0, knn, vnn, seqlens=sl, window=w, ring=True),
            nbytes, 1e9, "GB/s", "the whole rolling-cache workload (B=32, Hq=8, Hkv=2, d=64, "
            "w=C=4096, ragged lengths, committed candidate) in fp64")
    return res


def bench_sweep(torch, gqa, synth, steps, warmup, cpu=False, hkvs=None):
    """Endpoint sweep: B=16, Hq=8, d=128, 8000 cached cells; MHA, GQA group 4
    and MQA.  A K/V copy holds 524, 131 or 66 MB; 4 copies rotate for Hkv >= 2
    and 6 for Hkv = 1, so no step finds its cache in the 256 MB Infinity Cache
    left by the previous ones."""
    cfg = synth.CONFIGS["decode_sweep_b16_hq8_d128_n8000"]
    B, hq, d, n = cfg["B"], cfg["Hq"], cfg["d"], cfg["n"]
    dev = torch.device("cuda:0")
    res = []
    for hkv in (cfg["Hkv"] if hkvs is None else hkvs):
        copies = 4 if hkv >= 2 else 6
        q, k0, v0 = synth.decode_inputs(B, n, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
        ks, vs = [k0], [v0]
        for i in range(1, copies):
            _, k, v = synth.decode_inputs(B, n, hq, hkv, d, torch.bfloat16, cfg["seed"] + 100 * i, dev)
            ks.append(k)
            vs.append(v)
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(1, gqa.decode_workspace_bytes(B, n, hq, hkv, d)), dtype=torch.uint8,
                         device=dev)
        ms, ms_call = _time_calls(torch, lambda i: gqa.decode(q, ks[i % copies], vs[i % copies], out=out,
                                                     workspace=ws), steps, warmup)
        nbytes = decode_bytes(B, hq, hkv, d, n)
        gbs = nbytes / (ms * 1e-3) / 1e9
        leg = dict(Hkv=hkv, ms=round(ms, 5), bytes=nbytes, gbs=round(gbs, 2),
                   frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                   tokens_per_s=round(B / (ms * 1e-3), 1), per_call_ms=round(ms_call, 5),
                   traffic=measured_traffic(f"sweep{hkv}"))
        if cpu:
            import oracle

            qn, kn, vn = _f64(q), _f64(k0), _f64(v0)
            leg["cpu_baseline"] = _oracle_baseline(
                lambda: oracle.decode(qn, kn, vn), nbytes, 1e9, "GB/s",
                f"the whole sweep workload at Hkv={hkv} (B=16, Hq=8, d=128, 8000 cells) in fp64",
                budget_s=1.0)
            del qn, kn, vn
        res.append(leg)
        del ks, vs, q, k0, v0
    return dict(workload="gqa_decode_sweep_b16_hq8_d128_n8000_bf16", results=res,
                timing=f"{B2B}; {PER_CALL}")


def bench_ragged_window(torch, gqa, synth, steps, warmup, cpu=False):
    """Ragged sliding-window decode over a linear cache: B=32, Hq=8, Hkv=2,
    d=64, lengths uniform in [1, 32768], window 4096.  GB/s of the K/V cells
    inside each row's window, read once per KV group; 6 rotated copies."""
    cfg = synth.CONFIGS["decode_ragged_b32_hq8_hkv2_d64_w4096"]
    B, hq, hkv, d, C, w = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["C"], cfg["window"]
    lo, hi = cfg["n"]
    dev = torch.device("cuda:0")
    lens = synth.ragged_lengths(B, lo, hi, cfg["seed"])
    seqlens = lens.to(dev)
    copies = 6
    q, k0, v0 = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, cfg["seed"], dev)
    ks, vs = [k0], [v0]
    for i in range(1, copies):
        _, k, v = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, cfg["seed"] + 100 * i, dev)
        ks.append(k)
        vs.append(v)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, gqa.decode_workspace_bytes(B, C, hq, hkv, d, w)), dtype=torch.uint8,
                     device=dev)
    ms, ms_call = _time_calls(torch, lambda i: gqa.decode(q, ks[i % copies], vs[i % copies],
                                                 seqlens=seqlens, window=w, out=out,
                                                 workspace=ws), steps, warmup)
    cells = int(sum(min(int(n), w) for n in lens.tolist()))
    nbytes = 2 * hkv * cells * d * 2 + 2 * B * hq * d * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = dict(workload="gqa_decode_ragged_b32_hq8_hkv2_d64_w4096_bf16",
               ms=round(ms, 5), bytes=nbytes, gbs=round(gbs, 2),
               frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
               tokens_per_s=round(B / (ms * 1e-3), 1), window_cells_read=cells,
               per_call_ms=round(ms_call, 5), timing=f"{B2B}; {PER_CALL}",
               traffic=measured_traffic("ragged"))
    if cpu:
        import oracle

        del ks, vs
        qn, kn, vn = _f64(q), _f64(k0), _f64(v0)
        sl = lens.tolist()
        res["cpu_baseline"] = _oracle_baseline(
            lambda: oracle.decode(qn, kn, vn, seqlens=sl, window=w), nbytes, 1e9, "GB/s",
            "the whole ragged sliding-window workload (B=32, Hq=8, Hkv=2, d=64, window 4096, "
            "lengths in [1, 32768]) in fp64", budget_s=1.0)
    return res


def bench_small_f32(torch, gqa, synth, steps, warmup):
    """The small fp32 causal prefill (B=1, T=16, Hq=4, Hkv=2, d=8): latency
    only, with no window and with window 2."""
    cfg = synth.CONFIGS["prefill_f32_small"]
    B, T, hq, hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    dev = torch.device("cuda:0")
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.float32, cfg["seed"], dev)
    out = torch.empty((B, T, hq, d), dtype=torch.float32, device=dev)
    res = {}
    for w in cfg["windows"]:
        _, ms_call = _time_calls(torch, lambda i: gqa.prefill(q, k, v, window=w, out=out), steps,
                                 warmup)
        res["no_window" if w is None else f"window_{w}"] = round(ms_call * 1e3, 2)
    return dict(workload="gqa_prefill_b1_t16_hq4_hkv2_d8_causal_f32",
                kernel=gqa.prefill_kernel(B, T, T, hq, hkv, d, dtype=torch.float32),
                us_per_call=res, timing="HIP events on the launch stream around each call")


def copy_calibration(torch):
    """A plain device copy of COPY_CAL_BYTES, so that rocprofv3's FETCH_SIZE
    and WRITE_SIZE counters can be scaled against a known transfer."""
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def hbm_copy_reference(torch, nbytes=1 << 30, reps=10):
    """Read+write GB/s of a plain 1 GiB device copy (torch copy_) on this
    GPU: a measured practical ceiling to read the roofline fraction against."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(3)
    dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(r, budget_s=12.0):
    """The fp64 oracle as it stands, on the host cores, on the decode workload;
    plus one thread on batch row 0 (1/8 of the bytes), scaled to the whole."""
    import ctypes

    import numpy as np

    import oracle

    q = r["q"].float().cpu().numpy().astype(np.float64)
    k = r["k"].float().cpu().numpy().astype(np.float64)
    v = r["v"].float().cpu().numpy().astype(np.float64)
    L = oracle.lib()
    runs, t_total = 0, 0.0
    while t_total < budget_s and runs < 1000:
        t0 = time.perf_counter()
        oracle.decode(q, k, v, seqlens=r["seqlens"])
        t_total += time.perf_counter() - t0
        runs += 1
    per = t_total / runs
    cores = oracle.threads()
    # one thread, one batch row
    set_threads = L.omp_set_num_threads
    set_threads.argtypes = [ctypes.c_int]
    set_threads(1)
    try:
        q1, k1, v1 = q[:1].copy(), k[:1].copy(), v[:1].copy()
        runs1, t1 = 0, 0.0
        while t1 < 1.5 and runs1 < 100:
            t0 = time.perf_counter()
            oracle.decode(q1, k1, v1, seqlens=r["seqlens"][:1])
            t1 += time.perf_counter() - t0
            runs1 += 1
    finally:
        set_threads(cores)
    per1 = t1 / runs1
    B = q.shape[0]
    return dict(value=round(r["nbytes"] / per / 1e9, 3), unit="GB/s", cores=cores,
                kind="oracle",
                sample=f"the whole decode workload (B=8, Hq=32, Hkv=8, d=128, 8000 cells) in "
                       f"fp64, {runs} runs of {per:.4f} s; inputs converted to float64 "
                       "before timing",
                affinity_cores=len(os.sched_getaffinity(0)), cpu_model=_cpu_model(),
                single_thread={"value": round(r["nbytes"] / B / per1 / 1e9, 4), "unit": "GB/s",
                               "sample": f"batch row 0 of {B} (1/{B} of the bytes), one thread, "
                                         f"{runs1} runs of {per1:.4f} s; the rate holds for the "
                                         "whole workload, whose rows are independent"})


def run_leg(torch, gqa, synth, leg, steps, warmup):
    """One leg alone, for counter runs (every library dispatch is this leg's)."""
    if leg == "decode":
        r = bench_decode(torch, gqa, synth, steps, warmup)
        res = {"ms": round(r["ms"], 5)}
    elif leg == "prefill":
        res = bench_prefill(torch, gqa, synth, steps, warmup)
    elif leg == "prefix":
        res = bench_prefix(torch, gqa, synth, steps, warmup)
    elif leg == "packed":
        res = bench_packed(torch, gqa, synth, steps, warmup)
    elif leg == "ring":
        res = bench_ring(torch, gqa, synth, steps, warmup)
    elif leg.startswith("sweep"):
        res = bench_sweep(torch, gqa, synth, steps, warmup, hkvs=[int(leg[5:])])
    else:
        res = bench_ragged_window(torch, gqa, synth, steps, warmup)
    print(json.dumps({"leg": leg, "result": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--leg", choices=sorted(LEG_SOURCE), default=None,
                    help="run one leg only (for hardware-counter runs)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="print the per-leg traffic summary of counter runs under DIR")
    args = ap.parse_args()
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(args.summarize_counters))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode and prefill shard over sequences or KV groups with no exchange, so "
              "there is no multi-GPU step to time)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gqa_kv_cache_02_amd as gqa
    from gqa_kv_cache_02_amd import synth

    gqa.lib()
    if args.leg is not None:
        run_leg(torch, gqa, synth, args.leg, args.steps, args.warmup)
        if args.copy_calibration:
            copy_calibration(torch)
        return
    r = bench_decode(torch, gqa, synth, args.steps, args.warmup)
    cfg = r["cfg"]
    gbs = r["nbytes"] / (r["ms"] * 1e-3) / 1e9
    achieved = r["nbytes"] / (r["avg_call_ms"] * 1e-3) / 1e9
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
                     "traffic": measured_traffic("decode"),
                     "bytes_per_launch": r["nbytes"],
                     "avg_launch_ms": round(r["avg_call_ms"], 5),
                     "min_launch_ms": round(r["min_call_ms"], 5),
                     "p10_p50_p90_launch_ms": [round(r["p10_call_ms"], 5), round(r["p50_call_ms"], 5),
                                               round(r["p90_call_ms"], 5)],
                     "kernel": "decode call = decode_kernel (split) + decode_merge_kernel",
                     "timing": "HIP events on the launch stream around each decode call"},
    }
    copy_gbs = hbm_copy_reference(torch)
    line["roofline"]["hbm_copy_reference_gbs"] = copy_gbs
    line["frac_of_measured_copy"] = round(gbs / copy_gbs, 4)
    cpu = not args.no_cpu_baseline
    if not args.no_prefill:
        line["prefill"] = bench_prefill(torch, gqa, synth, max(10, args.steps // 10), 3, cpu)
        line["prefix_prefill"] = bench_prefix(torch, gqa, synth, max(10, args.steps // 10), 3,
                                              cpu)
        line["packed_prefill"] = bench_packed(torch, gqa, synth, max(10, args.steps // 10), 3,
                                              cpu)
    line["ring_decode"] = bench_ring(torch, gqa, synth, max(20, args.steps // 2), 10, cpu)
    line["decode_sweep"] = bench_sweep(torch, gqa, synth, max(20, args.steps // 2), 10, cpu)
    line["ragged_window_decode"] = bench_ragged_window(torch, gqa, synth,
                                                       max(20, args.steps // 2), 10, cpu)
    line["small_f32_prefill"] = bench_small_f32(torch, gqa, synth, max(20, args.steps // 2), 10)
    if args.copy_calibration:
        copy_calibration(torch)
        line["copy_calibration_bytes"] = COPY_CAL_BYTES
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(r)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
