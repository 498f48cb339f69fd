#!/usr/bin/env python3
"""Benchmark of the HiSparse hot path on one MI355X.

Default workload (the largest single-GPU one): 128 requests, 8 layers sharing one selection per
step, context 65536, fp8 656-byte entries, top_k 2048, device buffer 4096 slots, host capacity
65536 tokens; the selection trace is the seeded recency-window (128) + Zipf(1.05) history with
10 % churn per step.  A step is a whole decode step: every layer resolves the shared selection
(hit detection, LRU replacement, table update, host-to-device fetch of the missing rows) and
runs sparse MLA attention (16 heads) over its resolved slots, with layer-wise prefetch (layer
l + 1's tables and row copies on other streams beside layer l's attention).  The steps are
captured in one hipGraph; the first --warmup steps run untimed from an empty buffer, then
exactly --steps steps are timed.

Metric: resolved top-k selections/s (whole job: requests x layers x steps over the timed
region), with the miss-fetch rate against the host-link peak.  The JSON line also carries:
  roofline       the dominant kernel (the row copies over the host link, fetch_kernel), its
                 average launch time from HIP events on its stream;
  other_workloads the 64-request resolve-only and 256-request resolve + attention rates;
  cpu_baseline   the CPU oracle on a bounded sample of the same trace, on this host's cores.

--workload batch64 times resolve-only steps of 64 requests (bf16 1152-byte rows).
--workload fp8_256 measures resolve + sparse MLA attention (256 requests, fp8 656-byte
entries) and reports attention throughput against the HBM roofline.
--workload topk runs the on-GPU top-k from synthetic indexer scores into the resolver, one
selection per layer (128 requests, 8 layers, 65536 tokens).
--workload pages runs page-granular selections (pages of 16 tokens, 128 pages selected, 256
page slots, 256 requests, fp8): whole steps of write-through append of the newest token, resolve,
and attention cut at the context length.
--workload attend_cost splits an attention launch's time into a per-tile and a fixed part: k = 64
.. 2048 rows per request (256 requests, fp8), read from HBM cold and read from the caches.
--workload sweep is the miss-count study: misses per selection for device buffers of 2048,
4096 and 6144 slots under LRU, FIFO and RANDOM eviction (32 requests, 131072 tokens).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PCIE_GEN5_X16_GBPS = 64.0      # published host link peak per direction (MI355X, PCIe 5.0 x16)
HBM_PEAK_GBPS = 8000.0         # published MI355X HBM3E peak


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


KERNEL_SRC = os.path.join(ROOT, "hierarchical_kv_cache_hs_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _sha256(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def recorded_traffic(key, source):
    """HBM bytes per launch from the committed counter runs, or None if the kernel changed since."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != _sha256(os.path.join(KERNEL_SRC, source)):
        return None
    return rec.get("bytes_per_launch")


def summarize_profile(args):
    """Markdown summary of rocprofv3 output for one kernel (stats, timed dispatches, counters)."""
    import csv
    kern = args.kernel

    def rows(path):
        return list(csv.DictReader(open(path)))

    lines = []
    st = [r for r in rows(os.path.join(args.trace_dir, "run_kernel_stats.csv")) if kern in r["Name"]]
    for r in st:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    tr = sorted((r for r in rows(os.path.join(args.trace_dir, "run_kernel_trace.csv")) if kern in r["Kernel_Name"]),
                key=lambda r: int(r["Dispatch_Id"]))
    if args.skip:
        tr = tr[args.skip:args.skip + args.last] if args.last else tr[args.skip:]
    last = tr[-args.last:] if args.last else tr
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in last]
    print("| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|")
    print("\n".join(lines))
    what = f"dispatches {args.skip}..{args.skip + len(last) - 1}" if args.skip else f"last {len(last)} dispatches"
    print(f"\nTimed steps ({what} of the kernel): average {np.mean(dur):.2f} us, "
          f"median {np.median(dur):.2f} us.")
    out = {"avg_us_timed": float(np.mean(dur))}
    if args.pmc_dir and args.copy_dir:
        scale = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            cr = sorted(rows(os.path.join(f"{args.copy_dir}_{c}", "run_counter_collection.csv")),
                        key=lambda r: int(r["Dispatch_Id"]))[-5:]
            kib = np.median([float(r["Counter_Value"]) for r in cr])
            scale[c] = (256 * 1024) / kib
            kr = sorted((r for r in rows(os.path.join(f"{args.pmc_dir}_{c}", "run_counter_collection.csv"))
                         if kern in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))
            if args.pmc_skip:
                kr = kr[args.pmc_skip:args.pmc_skip + args.pmc_last] if args.pmc_last else kr[args.pmc_skip:]
            kr = kr[-args.pmc_last:] if args.pmc_last else kr
            v = float(np.mean([float(r["Counter_Value"]) for r in kr]))
            out[c] = v
            print(f"\n{c}: {v:.1f} KiB per dispatch over {len(kr)} timed dispatches; a plain copy of 256 MiB "
                  f"reads as {kib:.1f} KiB, so scale x{scale[c]:.3f} -> {v * scale[c] * 1024 / 1e6:.2f} MB per launch")
        out["bytes_per_launch"] = (out["FETCH_SIZE"] * scale["FETCH_SIZE"] + out["WRITE_SIZE"] * scale["WRITE_SIZE"]) * 1024
        out["fetch_scale"], out["write_scale"] = scale["FETCH_SIZE"], scale["WRITE_SIZE"]
        print(f"\nHBM + host-link traffic per launch (scaled FETCH + WRITE): {out['bytes_per_launch'] / 1e6:.2f} MB")
    if args.record:
        try:
            rec = json.load(open(TRAFFIC_FILE))
        except (OSError, ValueError):
            rec = {}
        out["kernel"] = kern
        out["source_sha256"] = _sha256(os.path.join(KERNEL_SRC, args.source))
        rec[args.record] = out
        json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)


def measure_h2d_peak(torch, nbytes=1 << 30, reps=5):
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return nbytes / ms / 1e6


def measure_hbm_peak(torch, hsa, nbytes=1 << 32, reps=5):
    """Measured HBM rates on this GPU: the library's dense streaming read (16-byte loads over
    4 GiB, far beyond the caches) and a device-to-device copy (bytes read + written over the
    time).  The larger one is the measured peak the resolve + attention fraction is also
    given against."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    hsa.stream_read(src, sink, stream)
    half = src[: nbytes // 8]
    dst = torch.empty_like(half)
    dst.copy_(half)
    torch.cuda.synchronize()
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    a.record(stream)
    for _ in range(reps):
        hsa.stream_read(src, sink, stream)
    b.record(stream)
    for _ in range(reps):
        dst.copy_(half)
    c.record(stream)
    torch.cuda.synchronize()
    read = nbytes / (a.elapsed_time(b) / reps) / 1e6
    copy = nbytes / (b.elapsed_time(c) / reps) / 1e6
    del src, dst, half, sink
    return {"read_GBps": read, "copy_GBps": copy, "peak_GBps": max(copy, read)}


def cpu_baseline_resolve(w, trace, warm, budget_s=15.0):
    """The oracle, as it stands, on the timed steps of the same trace.

    The trace is replayed from an empty cache as many times as fit in about budget_s
    seconds; only steps warm.. of each pass are timed, as on the GPU."""
    import oracle
    from synth import kv as skv
    n, E = w.n, w.entry_bytes
    host = np.empty((n, 1, w.cap, E), dtype=np.uint8)
    for r in range(n):
        skv.fill_rows(w.seed, r, 0, 0, w.cap, w.layout, host[r, 0].ctypes.data, E)
    threads = oracle.default_threads()
    done, el, passes = 0, 0.0, 0
    while passes == 0 or el < budget_s:
        oc = oracle.OracleCache(n, 1, w.B, w.cap, layout=w.layout, host=host, threads=threads)
        for t in range(warm):
            oc.resolve(0, trace[t])
        t0 = time.perf_counter()
        for t in range(warm, trace.shape[0]):
            oc.resolve(0, trace[t])
        el += time.perf_counter() - t0
        done += trace.shape[0] - warm
        passes += 1
    # the same on one thread, a shorter sample (one pass over the timed steps at most)
    oc1 = oracle.OracleCache(n, 1, w.B, w.cap, layout=w.layout, host=host, threads=1)
    for t in range(warm):
        oc1.resolve(0, trace[t])
    done1, el1 = 0, 0.0
    for t in range(warm, trace.shape[0]):
        t0 = time.perf_counter()
        oc1.resolve(0, trace[t])
        el1 += time.perf_counter() - t0
        done1 += 1
        if el1 > budget_s / 3:
            break
    return {"value": n * done / el, "unit": "selections/s", "cores": threads, "kind": "oracle",
            "value_1_thread": n * done1 / el1,
            "sample": f"oracle resolve (LRU tables + row copies) of all {n} requests on steps {warm}.."
                      f"{trace.shape[0] - 1} of the same trace, {passes} passes from an empty cache "
                      f"({done} steps timed, {el:.1f} s); on one thread, steps {warm}..{warm + done1 - 1} "
                      f"({el1:.1f} s)"}


def cpu_baseline_attend(w, step, budget_s=15.0):
    """The oracle's fp64 attention, as it stands, over the selection of one timed step.

    Requests are attended in batches of 16 until about budget_s seconds of oracle time
    have passed; the rows are generated outside the timed calls."""
    import oracle
    from synth import kv as skv
    from synth import trace as tr
    trace = tr.generate(w.trace_spec(), steps=step + 1)
    threads = oracle.default_threads()
    q = skv.queries(w.seed, step, w.n, 0, 16)
    done, el, r0 = 0, 0.0, 0
    while done == 0 or el < budget_s:
        rs = [(r0 + i) % w.n for i in range(16)]
        r0 += 16
        sel = trace[step, rs]
        rows = np.stack([skv.rows_at(w.seed, r, 0, sel[i], w.layout) for i, r in enumerate(rs)])
        idx = np.tile(np.arange(w.k, dtype=np.int32), (len(rs), 1))
        t0 = time.perf_counter()
        oracle.attend_rows(q[rs], idx, rows, w.layout, 1.0 / math.sqrt(576), threads=threads)
        el += time.perf_counter() - t0
        done += len(rs)
    return {"value": done * w.k / el, "unit": "attended tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle fp64 attention of {done} request selections (k {w.k}, 16 heads) of step {step}, "
                      f"in batches of 16 ({el:.1f} s)"}


def bench_resolve(args, torch, hsa, w):
    from synth import kv as skv
    from synth import trace as tr

    T = args.warmup + args.steps
    spec = w.trace_spec()
    if T > spec.steps:
        spec = w.with_(steps=T).trace_spec()
    t0 = time.perf_counter()
    trace = tr.generate(spec, steps=T)
    log(f"trace {trace.shape} in {time.perf_counter() - t0:.1f}s")
    d_trace = torch.from_numpy(trace).cuda()

    handles = {}
    for name, flags in (("io", 0), ("noio", hsa.FLAG_NO_IO), ("split", 0)):
        hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 0, flags)
        if not flags & hsa.FLAG_NO_IO:
            t0 = time.perf_counter()
            for r in range(w.n):
                ptr, cap, stride = hs.host_kv_ptr(0, r)
                skv.fill_rows(w.seed, r, 0, 0, cap, w.layout, ptr, stride)
            log(f"host pool {hsa.host_bytes(hs.cfg) / 2**30:.2f} GiB filled in {time.perf_counter() - t0:.1f}s")
        handles[name] = hs

    slots = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
    miss = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    results = {}
    for name, hs in handles.items():
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            w0.record(stream)
            for t in range(args.warmup):
                hs.resolve(0, d_trace[t], slots, miss[t], stream=stream)
            w1.record(stream)
        stream.synchronize()
        warm_ms = w0.elapsed_time(w1) if args.warmup else 0.0
        # capture the timed steps; the graph holds only resolver launches, so the region
        # time over the launch count is the kernel's average launch duration
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(args.steps):
                    t = args.warmup + i
                    hs.resolve(0, d_trace[t], slots, miss[t], stream=stream, split=(name == "split"))
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):      # replay() launches on the current stream
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        region_ms = a.elapsed_time(b)
        m = miss[args.warmup:].cpu().numpy().astype(np.int64)
        results[name] = {"region_ms": region_ms, "kernel_ms": region_ms / args.steps, "miss": m, "warm_ms": warm_ms,
                         "warm_miss": miss[:args.warmup].cpu().numpy().astype(np.int64)}
        log(f"{name}: {region_ms:.3f} ms for {args.steps} steps; {region_ms / args.steps * 1e3:.1f} us per launch")
        del g

    io, noio, split = results["io"], results["noio"], results["split"]
    assert (io["miss"] == noio["miss"]).all() and (io["miss"] == split["miss"]).all()
    K = args.steps
    total_miss = int(io["miss"].sum())
    fetch_bytes = total_miss * w.entry_bytes
    sel_per_s = w.n * K / (io["region_ms"] / 1e3)
    avg_kernel_s = io["kernel_ms"] / 1e3
    avg_kernel_noio_s = noio["kernel_ms"] / 1e3
    bytes_per_launch = fetch_bytes / K
    achieved = bytes_per_launch / avg_kernel_s / 1e9
    fetch_only_s = max(avg_kernel_s - avg_kernel_noio_s, 1e-12)
    h2d = measure_h2d_peak(torch)
    log(f"H2D memcpy peak {h2d:.1f} GB/s")
    traffic = recorded_traffic("resolve_batch64", "resolve.hip")
    out = {
        "metric": "resolved top-k selections/s + miss-fetch GB/s vs host-link peak, 1 MI355X",
        "value": sel_per_s,
        "unit": "selections/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": io["region_ms"] / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32",
        "data": "synthetic",
        "config": {"workload": w.description, "global_batch": w.n, "seq_len": w.ctx, "top_k": w.k,
                   "device_buffer_size": w.B, "host_to_device_ratio": w.ratio, "entry_bytes": w.entry_bytes,
                   "steps_timed": f"{args.warmup}..{args.warmup + K - 1}", "graph": True},
        "selected_tokens_per_s": sel_per_s * w.k,
        "misses_per_selection": total_miss / (w.n * K),
        "miss_fetch_GBps": fetch_bytes / (io["region_ms"] / 1e3) / 1e9,
        "miss_fetch_GBps_fetch_only": bytes_per_launch / fetch_only_s / 1e9,
        "h2d_peak_GBps_measured": h2d,
        "miss_fetch_frac_of_measured_peak": (fetch_bytes / (io["region_ms"] / 1e3) / 1e9) / h2d,
        "split_tables_and_fetch_us_per_step": split["kernel_ms"] * 1e3,
        # the untimed warmup steps from an empty buffer (step 0 misses every token), launched
        # one by one, and the mean over every step of the trace
        "cold_start": {"steps": args.warmup, "ms": io["warm_ms"],
                       "misses_per_selection": float(io["warm_miss"].mean()) if args.warmup else None,
                       "step0_misses_per_selection": float(io["warm_miss"][0].mean()) if args.warmup else None,
                       "miss_fetch_GBps": (float(io["warm_miss"].sum()) * w.entry_bytes / (io["warm_ms"] / 1e3) / 1e9
                                           if args.warmup and io["warm_ms"] > 0 else None),
                       "all_steps_misses_per_selection": float(np.concatenate([io["warm_miss"], io["miss"]]).mean()),
                       "all_steps_selections_per_s": w.n * (args.warmup + K) / ((io["warm_ms"] + io["region_ms"]) / 1e3)},
        "resolve_only": {"us_per_step": avg_kernel_noio_s * 1e6,
                         "selections_per_s": w.n / avg_kernel_noio_s,
                         "share_of_io_step": avg_kernel_noio_s / avg_kernel_s},
        "roofline": {"bound": "host_link", "achieved": achieved, "peak": PCIE_GEN5_X16_GBPS, "unit": "GB/s",
                     "frac": achieved / PCIE_GEN5_X16_GBPS, "traffic": traffic,
                     "kernel": "resolve_kernel", "avg_kernel_us": avg_kernel_s * 1e6,
                     "algorithmic_bytes_per_launch": bytes_per_launch,
                     "frac_of_measured_peak": achieved / h2d},
    }
    for hs in handles.values():
        hs.close()
    return out, trace


def bench_attend(args, torch, hsa, w, legs=True):
    """Resolve + attention on the fp8 256-request workload (attention against HBM).  With
    legs=False the overlapped-step and append legs are skipped."""
    from synth import kv as skv
    from synth import trace as tr

    T = args.warmup + args.steps
    spec = w.with_(steps=max(T, w.steps)).trace_spec()
    trace = tr.generate(spec, steps=T)
    d_trace = torch.from_numpy(trace).cuda()
    hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 16, 0)
    for r in range(w.n):
        ptr, cap, stride = hs.host_kv_ptr(0, r)
        skv.fill_rows(w.seed, r, 0, 0, cap, w.layout, ptr, stride)
    qs = torch.from_numpy(np.stack([skv.queries(w.seed, t % 8, w.n, 0, 16) for t in range(8)]).view(np.int16)) \
        .cuda().view(torch.bfloat16)
    slots = torch.empty(T, w.n, w.k, dtype=torch.int32, device="cuda")
    miss = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    out = torch.empty(w.n, 16, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.n, 16, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(576)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            hs.resolve(0, d_trace[t], slots[t], miss[t], stream=stream)
            hs.attend(0, qs[t % 8], slots[t], scale, out, lse, stream=stream)
    stream.synchronize()

    def timed(g):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):      # replay() launches on the current stream
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                t = args.warmup + i
                hs.resolve(0, d_trace[t], slots[t], miss[t], stream=stream)
                hs.attend(0, qs[t % 8], slots[t], scale, out, lse, stream=stream)
    region_ms = timed(g)
    # attention alone, cold: before every launch a 1 GiB read evicts the rows from the L2 and
    # the 256 MB last-level cache (a read leaves clean lines, so the timed launch pays no
    # write-back), as in a real step where other layers' rows intervene; HIP events on the
    # launch stream bracket each attention launch
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    att_ms = []
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            t = args.warmup + i
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hs.attend(0, qs[t % 8], slots[t], scale, out, lse, stream=stream)
            b.record(stream)
            b.synchronize()
            att_ms.append(a.elapsed_time(b))
    # the fp32-output mode on the same rows and slots (a no-IO handle given a copy of the buffer)
    hs_f32 = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 16, hsa.FLAG_NO_IO | hsa.FLAG_ATTN_OUT_F32)
    hs_f32.state(0)["kv_buffer"].copy_(hs.state(0)["kv_buffer"])
    out32 = torch.empty(w.n, 16, 512, dtype=torch.float32, device="cuda")
    f32_ms = []
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            t = args.warmup + i
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hs_f32.attend(0, qs[t % 8], slots[t], scale, out32, lse, stream=stream)
            b.record(stream)
            b.synchronize()
            f32_ms.append(a.elapsed_time(b))
    hs_f32.close()
    del flush, out32

    # Attention alone, cold and back to back: four layers of a no-IO handle hold copies of the
    # rows, and one graph of K launches cycles over them, so that every launch reads rows the
    # three launches before it (1 GB) have evicted from the L2 and the 256 MB last-level cache,
    # and no launch gap is counted: graph region time / K is the kernel's average duration.
    # (The per-launch HIP events above add each launch's gap.)  The same for the fp32 mode.
    def cold_graph_us(flags, out_t):
        NL = 4
        h = hsa.HiSparse(w.k, w.B, w.ratio, w.n, NL, w.layout, 16, hsa.FLAG_NO_IO | flags)
        for l in range(NL):
            h.state(l)["kv_buffer"].copy_(hs.state(0)["kv_buffer"])
        gc = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gc, stream=stream):
                for i in range(args.steps):
                    t = args.warmup + i
                    h.attend(i % NL, qs[t % 8], slots[t], scale, out_t, lse, stream=stream)
        timed(gc)
        us = timed(gc) / args.steps * 1e3
        del gc
        h.close()
        return us

    att_graph_us = cold_graph_us(0, out)
    out32 = torch.empty(w.n, 16, 512, dtype=torch.float32, device="cuda")
    f32_graph_us = cold_graph_us(hsa.FLAG_ATTN_OUT_F32, out32)
    del out32
    # resolution alone: a handle that moves no rows, the same selections, one graph of K launches
    hs_noio = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 0, hsa.FLAG_NO_IO)
    slots_n = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
    miss_n = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            hs_noio.resolve(0, d_trace[t], slots_n, miss_n[t], stream=stream)
    stream.synchronize()
    gn = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gn, stream=stream):
            for i in range(args.steps):
                hs_noio.resolve(0, d_trace[args.warmup + i], slots_n, miss_n[args.warmup + i], stream=stream)
    noio_us = timed(gn) / args.steps * 1e3
    assert torch.equal(miss_n[args.warmup:], miss[args.warmup:])
    del gn
    # the same resolves cold, as inside a real step where the attention's rows have evicted the
    # tables from the caches: replay from an empty state, a 1 GiB read before each launch
    hs_noio.reset_requests(0, w.n, stream=stream)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    cold_ms = []
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            hs_noio.resolve(0, d_trace[t], slots_n, miss_n[t], stream=stream)
        for i in range(args.steps):
            t = args.warmup + i
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hs_noio.resolve(0, d_trace[t], slots_n, miss_n[t], stream=stream)
            b.record(stream)
            b.synchronize()
            cold_ms.append(a.elapsed_time(b))
    noio_cold_us = float(np.mean(cold_ms)) * 1e3
    del flush
    hs_noio.close()
    res_ms = [region_ms / args.steps - att_graph_us / 1e3]
    tail = bench_resident_tail_leg(args, torch, hsa, w, hs, d_trace, stream, timed)
    overlap = bench_overlap_leg(args, torch, hsa, w, hs, d_trace, qs, miss, stream, timed, scale, region_ms) \
        if legs else None
    append = bench_append_leg(args, torch, hsa, w, d_trace, miss, stream, timed) if legs else None
    K = args.steps
    att_s = att_graph_us / 1e6
    valid = (slots[args.warmup:] >= 0).sum().item() / K
    att_bytes = w.n * (4 * w.k) + valid * w.entry_bytes + w.n * 16 * (576 * 2 + 512 * 2 + 4)
    achieved = att_bytes / att_s / 1e9
    m = miss[args.warmup:].cpu().numpy().astype(np.int64)
    traffic = recorded_traffic("attend_fp8_256", "attend.hip")
    ra_bytes = w.n * (16 * w.k + 4 * w.B + 16 * float(m.mean())) + att_bytes
    hbm = measure_hbm_peak(torch, hsa)
    log(f"HBM measured: copy {hbm['copy_GBps']:.0f} GB/s, read {hbm['read_GBps']:.0f} GB/s")
    out_line = {
        "metric": "attention tokens/s over resolved slots, 1 MI355X",
        "value": w.n * w.k / att_s,
        "unit": "attended tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": region_ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.description + f" (churn {w.churn})", "global_batch": w.n, "seq_len": w.ctx,
                   "top_k": w.k, "heads": 16, "graph": True},
        "resolve_us_per_step": float(np.mean(res_ms)) * 1e3,
        "resolve_noio_us_per_step": noio_us,
        "resolve_noio_cold_us_per_step": noio_cold_us,
        "attention_f32_output_us": f32_graph_us,
        # the same launches timed one by one after a 1 GiB read (HIP events; each adds its gap)
        "attention_cold_event_us": float(np.mean(att_ms)) * 1e3,
        "attention_f32_output_cold_event_us": float(np.mean(f32_ms)) * 1e3,
        "misses_per_selection": float(m.mean()),
        "append": append,
        "attend_while_fetching": overlap,
        "resident_tail": tail,
        # resolution (table work, no row copies) + attention against HBM, over the sum of their
        # times: per selection 16k + 4B + 16m bytes of tables plus the attention bytes
        "hbm_resolve_plus_attend": {
            "bytes": ra_bytes,
            "us": noio_us + att_s * 1e6,
            "frac": ra_bytes / ((noio_us * 1e-6 + att_s) * HBM_PEAK_GBPS * 1e9),
            "hbm_measured": hbm,
            "frac_of_measured_peak": ra_bytes / ((noio_us * 1e-6 + att_s) * hbm["peak_GBps"] * 1e9),
            # the resolve timed cold, one by one with HIP events (which add its launch gap)
            "cold_us": noio_cold_us + att_s * 1e6,
            "cold_frac": ra_bytes / ((noio_cold_us * 1e-6 + att_s) * HBM_PEAK_GBPS * 1e9),
            "cold_frac_of_measured_peak": ra_bytes / ((noio_cold_us * 1e-6 + att_s) * hbm["peak_GBps"] * 1e9)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "kernel": "attend_kernel",
                     "avg_kernel_us": att_s * 1e6, "algorithmic_bytes_per_launch": att_bytes,
                     "frac_of_measured_peak": achieved / hbm["peak_GBps"]},
    }
    hs.close()
    return out_line


def measure_d2h_peak(torch, nbytes=1 << 30, reps=5):
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return nbytes / ms / 1e6


def bench_resident_tail_leg(args, torch, hsa, w, hs, d_trace, stream, timed):
    """The fused resolve (tables and row copies in one kernel per request) alone, K steps in one
    graph, on the packed handle and on a handle with the resident-tail layout (each row's first
    640 bytes in the host pool, five 128-byte lines over the link instead of six; the last 16
    bytes in device memory), back to back on the same GPU.  Both start from an empty buffer and
    replay the same trace; misses, slots and the final slot bytes must be identical."""
    K, W = args.steps, args.warmup
    T = W + K

    def resolve_only(h):
        slots = torch.empty(T, w.n, w.k, dtype=torch.int32, device="cuda")
        miss = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
        h.reset_requests(0, w.n, stream=stream)
        with torch.cuda.stream(stream):
            for t in range(W):
                h.resolve(0, d_trace[t], slots[t], miss[t], stream=stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for t in range(W, T):
                    h.resolve(0, d_trace[t], slots[t], miss[t], stream=stream)
        us = timed(g) / K * 1e3
        del g
        return us, slots, miss

    packed_us, p_slots, p_miss = resolve_only(hs)
    ht = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 16, hsa.FLAG_RESIDENT_TAIL)
    fill_history(torch, ht, w)
    tail_us, t_slots, t_miss = resolve_only(ht)
    occ = hs.state(0)["slot_owner"] >= 0       # slots filled since the reset (others keep old bytes)
    same = torch.equal(p_slots, t_slots) and torch.equal(p_miss, t_miss) and \
        torch.equal(hs.state(0)["slot_owner"], ht.state(0)["slot_owner"]) and \
        torch.equal(hs.state(0)["kv_buffer"][occ], ht.state(0)["kv_buffer"][occ])
    ht.close()
    misses = float(p_miss[W:].double().sum()) / K
    log(f"fused resolve alone: packed rows {packed_us:.1f} us, resident tail {tail_us:.1f} us per step "
        f"(identical results: {same})")
    return {"packed_resolve_us_per_step": packed_us, "resolve_us_per_step": tail_us,
            "speedup": packed_us / tail_us, "identical_to_packed": bool(same),
            "packed_link_GBps": misses * w.entry_bytes / (packed_us * 1e-6) / 1e9,
            "link_GBps": misses * (w.entry_bytes - 16) / (tail_us * 1e-6) / 1e9,
            "link_bytes_per_miss": w.entry_bytes - 16, "tail_bytes_per_token_on_device": 16}


def bench_overlap_leg(args, torch, hsa, w, hs, d_trace, qs, miss_serial, stream, timed, scale, serial_ms):
    """The same steps with the attention of the resident tokens overlapping the miss copy:
    list-only resolve, then the copy on a second stream beside the resident part of the
    attention, then the fetched part and the merge; captured in one graph with the fork and
    join of the two streams.  The handle is reset to the empty state and replays the trace."""
    from hierarchical_kv_cache_hs_amd.decode_step import attend_while_fetching
    T = args.warmup + args.steps
    side = torch.cuda.Stream()
    slots = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
    miss = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    out = torch.empty(w.n, 16, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.n, 16, dtype=torch.float32, device="cuda")
    hs.reset_requests(0, w.n, stream=stream)
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            attend_while_fetching(hs, 0, d_trace[t], qs[t % 8], scale, slots, miss[t], out, lse, stream, side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                t = args.warmup + i
                attend_while_fetching(hs, 0, d_trace[t], qs[t % 8], scale, slots, miss[t], out, lse, stream, side)
    ms = timed(g)
    assert torch.equal(miss[args.warmup:], miss_serial[args.warmup:])
    # the fused resolve (tables and copy in one kernel) then the attention, as timed above
    step_us = ms / args.steps * 1e3
    log(f"attend while fetching: {step_us:.1f} us per step against {serial_ms / args.steps * 1e3:.1f} serial")
    del g
    return {"us_per_step": step_us, "serial_us_per_step": serial_ms / args.steps * 1e3,
            "saved_frac": 1.0 - ms / serial_ms,
            "attended_tokens_per_s_whole_step": w.n * w.k / (step_us * 1e-6),
            "selections_per_s_whole_step": w.n / (step_us * 1e-6)}


def bench_append_leg(args, torch, hsa, w, d_trace, miss_plain, stream, timed):
    """Write-through append of each step's newest token before its resolve (the growing
    context's guaranteed miss), and bulk prefill offload into the pinned history."""
    from synth import kv as skv
    T = args.warmup + args.steps
    hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 0, 0)
    for r in range(w.n):
        ptr, cap, stride = hs.host_kv_ptr(0, r)
        skv.fill_rows(w.seed, r, 0, 0, cap, w.layout, ptr, stride)
    # the newest position of step t is ctx + t - 1; its row is the synthetic row of that position
    pos = torch.from_numpy(np.stack([np.full(w.n, w.ctx + t - 1, dtype=np.int32) for t in range(T)])).cuda()
    rows = torch.from_numpy(np.stack([np.stack([skv.rows_at(w.seed, r, 0, np.array([w.ctx + t - 1]), w.layout)[0]
                                                for r in range(w.n)]) for t in range(T)])).cuda()
    slots = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
    miss = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            hs.append(0, pos[t], rows[t], stream=stream)
            hs.resolve(0, d_trace[t], slots, miss[t], stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                t = args.warmup + i
                hs.append(0, pos[t], rows[t], stream=stream)
                hs.resolve(0, d_trace[t], slots, miss[t], stream=stream)
    step_ms = timed(g) / args.steps
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(ga, stream=stream):
            for i in range(args.steps):
                hs.append(0, pos[args.warmup + i], rows[args.warmup + i], stream=stream)
    append_ms = timed(ga) / args.steps
    m_app = miss[args.warmup:].double().mean().item()
    m_plain = miss_plain[args.warmup:].double().mean().item()
    assert hs.device_error() == 0
    # prefill offload: 8 requests' 32768-token prompts, device rows -> pinned history
    nreq, count = 8, min(32768, w.cap)
    src = torch.randint(0, 256, (count, w.entry_bytes), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record(stream)
        for r in range(nreq):
            hs.offload(0, r, 0, src, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    off_ms = a.elapsed_time(b)
    ok = bool((hs.host_kv(0, nreq - 1)[:count] == src.cpu().numpy()).all())
    padded = torch.randint(0, 256, (count, w.entry_bytes + 112), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        a.record(stream)
        for r in range(nreq):
            hs.offload(0, r, 0, padded, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    off_pad_ms = a.elapsed_time(b)
    ok = ok and bool((hs.host_kv(0, 0)[:count] == padded[:, :w.entry_bytes].cpu().numpy()).all())
    d2h = measure_d2h_peak(torch)
    hs.close()
    return {"misses_per_selection": m_app, "misses_per_selection_without_append": m_plain,
            "append_plus_resolve_us_per_step": step_ms * 1e3, "append_us_per_step": append_ms * 1e3,
            "offload_GBps": nreq * count * w.entry_bytes / (off_ms / 1e3) / 1e9,
            "offload_padded_rows_GBps": nreq * count * w.entry_bytes / (off_pad_ms / 1e3) / 1e9,
            "d2h_peak_GBps_measured": d2h, "offload_rows_verified": ok,
            "offload_sample": f"{nreq} requests x {count} rows of {w.entry_bytes} B"}


def bench_sweep(args, torch, hsa):
    """Misses per selection against device buffer size and eviction policy on the 32-request,
    131072-token workload (the note's miss-count experiment, section 3 and Fig. 3), plus the
    fetching LRU resolver's rate per buffer size."""
    from synth import configs as C
    from synth import kv as skv
    from synth import trace as tr

    w0 = C.SWEEP
    steps = w0.steps
    trace = tr.generate(w0.trace_spec(), steps=steps)      # one trace for every buffer size
    d_trace = torch.from_numpy(trace).cuda()
    warm = min(10, steps - 1)
    stream = torch.cuda.Stream()
    policies = (("lru", hsa.EVICT_LRU), ("fifo", hsa.EVICT_FIFO), ("random", hsa.EVICT_RANDOM))
    study, fetch = {}, {}
    for B in C.SWEEP_BUFFERS:
        w = C.sweep_point(B)
        study[B] = {}
        for name, pol in policies:
            hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 0, hsa.FLAG_NO_IO, eviction=pol,
                              eviction_seed=12345)
            slots = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
            miss = torch.zeros(steps, w.n, dtype=torch.int32, device="cuda")
            with torch.cuda.stream(stream):
                for t in range(steps):
                    hs.resolve(0, d_trace[t], slots, miss[t], stream=stream)
            stream.synchronize()
            m = miss.double()
            study[B][name] = {"all_steps": m.mean().item(), "steady": m[warm:].mean().item()}
            hs.close()
            log(f"B {B} {name}: {study[B][name]}")
        # the method's fetching resolver on the same trace: graph of the steady steps
        hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 0, 0)
        for r in range(w.n):
            ptr, cap, stride = hs.host_kv_ptr(0, r)
            skv.fill_rows(w.seed, r, 0, 0, cap, w.layout, ptr, stride)
        slots = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
        miss = torch.zeros(steps, w.n, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(stream):
            for t in range(warm):
                hs.resolve(0, d_trace[t], slots, miss[t], stream=stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for t in range(warm, steps):
                    hs.resolve(0, d_trace[t], slots, miss[t], stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / (steps - warm)
        mb = miss[warm:].double().sum().item() * w.entry_bytes / (steps - warm)
        fetch[B] = {"us_per_step": ms * 1e3, "miss_fetch_GBps": mb / (ms / 1e3) / 1e9,
                    "misses_per_selection": miss[warm:].double().mean().item()}
        assert abs(fetch[B]["misses_per_selection"] - study[B]["lru"]["steady"]) < 1e-9
        del g
        hs.close()
    return {
        "metric": "misses per selection vs device buffer size and eviction policy, 1 MI355X",
        "value": study[4096]["lru"]["steady"], "unit": "misses/selection (LRU, B 4096, steps >= 10)",
        "n_gpus": 1, "steps": steps - warm, "warmup": warm, "ms_per_step": fetch[4096]["us_per_step"] / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "i32", "data": "synthetic",
        "config": {"workload": w0.description, "global_batch": w0.n, "seq_len": w0.ctx, "top_k": w0.k,
                   "device_buffer_size": list(C.SWEEP_BUFFERS), "eviction_seed": 12345},
        "study": {str(B): v for B, v in study.items()},
        "lru_fetch": {str(B): v for B, v in fetch.items()},
    }


def bench_topk(args, torch, hsa):
    """On-GPU top-k from synthetic indexer scores feeding the resolver, one selection per layer
    (128 requests, 8 layers, 65536-token contexts, k 2048, B 4096, fp8 entries).  Scores follow
    the recipe of synth/scores.py -- per-(request, layer) importance, per-step noise 0.08,
    +100 on the last 128 positions -- drawn on the device from a seeded generator.  The steps
    run the hinted top-k (hs_topk_hinted, one hint per layer carried from step to step, as in a
    decode loop); the top-k launches are also timed alone, without and with hints."""
    import oracle
    from oracle.topk import topk as topk_oracle
    n, L, ctx, k, B, W = 128, 8, 65536, 2048, 4096, 128
    K, warm = min(args.steps, 10), min(args.warmup, 3)
    T = warm + K
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    imp = torch.randn(L, n, ctx, device="cuda", generator=gen)
    scores = torch.empty(T, L, n, ctx, device="cuda")
    for t in range(T):
        scores[t] = imp + 0.08 * torch.randn(L, n, ctx, device="cuda", generator=gen)
    scores[:, :, :, ctx - W:] += 100.0
    del imp
    lens = torch.full((n,), ctx, dtype=torch.int32, device="cuda")
    hs = hsa.HiSparse(k, B, ctx // B, n, L, hsa.LAYOUT_FP8, 0, hsa.FLAG_NO_IO)
    sel = torch.empty(T, L, n, k, dtype=torch.int32, device="cuda")
    slots = torch.empty(L, n, k, dtype=torch.int32, device="cuda")
    miss = torch.zeros(T, L, n, dtype=torch.int32, device="cuda")
    hints = torch.full((L, n), -1, dtype=torch.int32, device="cuda")   # no guess before the first step
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def step(t):
        for l in range(L):
            hs.topk(scores[t, l], lens, sel[t, l], stream=stream, hint=hints[l])
            hs.resolve(l, sel[t, l], slots[l], miss[t, l], stream=stream)

    def timed(g):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    with torch.cuda.stream(stream):
        for t in range(warm):
            step(t)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for t in range(warm, T):
                step(t)
    step_ms = timed(g) / K
    gt = torch.cuda.CUDAGraph()
    sel_plain = torch.empty_like(sel)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gt, stream=stream):
            for t in range(warm, T):
                for l in range(L):
                    hs.topk(scores[t, l], lens, sel_plain[t, l], stream=stream)
    topk_us = timed(gt) / (K * L) * 1e3
    # the top-k alone with hints (each launch's guess is the previous step's result for that
    # layer; the replay's first step takes the last step's): the same selections
    gh = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gh, stream=stream):
            for t in range(warm, T):
                for l in range(L):
                    hs.topk(scores[t, l], lens, sel[t, l], stream=stream, hint=hints[l])
    topk_hinted_us = timed(gh) / (K * L) * 1e3
    hinted_same = bool(torch.equal(sel[warm:], sel_plain[warm:]))
    del gt, gh, sel_plain
    # a sampled check against the oracle, and the oracle's own rate on the same rows
    rows = scores[T - 1, 3, :8].cpu().numpy()
    t0 = time.perf_counter()
    want = topk_oracle(rows, np.full(8, ctx), k)
    cpu_s = time.perf_counter() - t0
    ok = bool((sel[T - 1, 3, :8].cpu().numpy() == want).all())
    bytes_launch = n * (ctx * 4 + k * 4 + 4)
    achieved = bytes_launch / (topk_hinted_us * 1e-6) / 1e9
    m = miss[warm:].double()
    s_prev, s_last = sel[T - 2].cpu().numpy(), sel[T - 1].cpu().numpy()
    churn = float(np.mean([k - np.intersect1d(s_prev[l, r], s_last[l, r]).size for l in range(L) for r in range(0, n, 16)]))
    hs.close()
    return {
        "metric": "top-k selections/s from indexer scores (per layer) feeding the resolver, 1 MI355X",
        "value": n * L / (step_ms / 1e3), "unit": "selections/s (top-k + resolve, no IO)",
        "n_gpus": 1, "steps": K, "warmup": warm, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{n} requests, {L} layers with their own selections, ctx {ctx}, k {k}, B {B}, "
                               "fp8 656 B, indexer scores: importance + 0.08 noise + recency 128",
                   "global_batch": n, "layers": L, "seq_len": ctx, "top_k": k},
        "topk_us_per_launch": topk_us,
        "topk_hinted_us_per_launch": topk_hinted_us,
        "topk_hinted_equals_plain": hinted_same,
        "topk_plain_frac_of_hbm": bytes_launch / (topk_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "resolve_noio_plus_topk_us_per_layer": step_ms * 1e3 / L,
        "misses_per_selection": m.mean().item(),
        "history_churn_per_step": churn,
        "topk_verified_rows": ok,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": recorded_traffic("topk_c4", "topk.hip"),
                     "kernel": "topk_kernel (hinted)", "avg_kernel_us": topk_hinted_us,
                     "algorithmic_bytes_per_launch": bytes_launch},
        "cpu_baseline": {"value": 8 * k / cpu_s, "unit": "selected positions/s", "cores": 1, "kind": "oracle",
                         "sample": f"oracle top-k (numpy stable sort) of 8 rows of {ctx} scores"},
    }


def cpu_baseline_pages(w, trace, warm, budget_s=15.0, requests=16):
    """The oracle, as it stands, on whole steps of the page workload for a sample of requests:
    append of the newest token, page resolve (tables + page copies), then fp64 attention cut
    at the context length."""
    import oracle
    from synth import kv as skv
    P = w.page_tokens
    n = min(requests, w.n)
    host = np.empty((n, 1, w.cap * P, w.entry_bytes), dtype=np.uint8)
    for r in range(n):
        skv.fill_rows(w.seed, r, 0, 0, w.cap * P, w.layout, host[r, 0].ctypes.data, w.entry_bytes)
    threads = oracle.default_threads()
    oc = oracle.OracleCache(n, 1, w.B, w.cap, layout=w.layout, host=host, threads=threads, page_tokens=P)
    for t in range(warm):
        oc.resolve(0, trace[t, :n])
    done, el, t = 0, 0.0, warm
    while (done == 0 or el < budget_s) and t < trace.shape[0]:
        q = skv.queries(w.seed, t % 8, n, 0, 16)
        lens = np.full(n, w.len_tokens(t))
        pos = lens - 1
        new = np.stack([skv.rows_at(w.seed, r, 0, pos[r:r + 1], w.layout)[0] for r in range(n)])
        t0 = time.perf_counter()
        oc.append(0, pos, new)
        slots, _ = oc.resolve(0, trace[t, :n])
        oc.attend_pages(0, q, slots, trace[t, :n], lens, 1.0 / math.sqrt(576))
        el += time.perf_counter() - t0
        done += 1
        t += 1
    return {"value": n * done * w.k * P / el, "unit": "attended tokens/s (append + resolve + attention)", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle append + page resolve + fp64 attention of requests 0..{n - 1} on steps {warm}..{t - 1} "
                      f"({done} steps, {el:.1f} s)"}


def cpu_baseline_prefetch(w, trace, warm, budget_s=15.0, requests=4):
    """The oracle, as it stands, on whole 8-layer decode steps for a sample of requests: every
    layer resolves the shared selection (tables + row copies), then fp64 attention per layer.
    After the warm-up steps (untimed, from an empty cache), steps warm.. are timed one by one
    until about budget_s seconds of oracle time have passed (the whole trace, again from an
    empty cache, if it ends first); the rate is selections (request-layer pairs resolved and
    attended) per second."""
    import oracle
    from synth import kv as skv
    n = min(requests, w.n)
    L = w.layers
    host = np.empty((n, L, w.cap, w.entry_bytes), dtype=np.uint8)
    for r in range(n):
        for l in range(L):
            skv.fill_rows(w.seed, r, l, 0, w.cap, w.layout, host[r, l].ctypes.data, w.entry_bytes)
    threads = oracle.default_threads()
    T = trace.shape[0]
    qs = {t: [skv.queries(w.seed, t, n, l, 16) for l in range(L)] for t in range(warm, T)}
    done, el, passes, last = 0, 0.0, 0, warm
    while passes == 0 or el < budget_s:
        oc = oracle.OracleCache(n, L, w.B, w.cap, layout=w.layout, host=host, threads=threads)
        for t in range(warm):
            for l in range(L):
                oc.resolve(l, trace[t, :n])
        for t in range(warm, T):
            t0 = time.perf_counter()
            for l in range(L):
                slots, _ = oc.resolve(l, trace[t, :n])
                oc.attend(l, qs[t][l], slots, 1.0 / math.sqrt(576))
            el += time.perf_counter() - t0
            done += 1
            last = max(last, t)
            if el >= budget_s:
                break
        passes += 1
    return {"value": done * n * L / el, "unit": "selections/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle resolve (tables + row copies) and fp64 attention of {L} layers for requests "
                      f"0..{n - 1} on steps {warm}..{last} of the same trace after {warm} untimed steps from "
                      f"an empty cache, {passes} pass(es) ({done} steps, {done * n * L} selections, {el:.1f} s)"}


def bench_pages(args, torch, hsa, w):
    """Page-granular selections: whole steps of write-through append of the newest token,
    resolve, and attention cut at the context length."""
    from synth import kv as skv
    from synth import trace as tr

    P = w.page_tokens
    K = args.steps
    T = args.warmup + K
    trace = tr.generate(w.with_(steps=max(T, w.steps)).trace_spec(), steps=T)
    d_trace = torch.from_numpy(trace).cuda()
    lens = torch.tensor([[w.len_tokens(t)] * w.n for t in range(T)], dtype=torch.int32, device="cuda")
    hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 16, 0, page_tokens=P)
    t0 = time.perf_counter()
    for r in range(w.n):
        ptr, cap, stride = hs.host_kv_ptr(0, r)
        skv.fill_rows(w.seed, r, 0, 0, cap, w.layout, ptr, stride)
    log(f"host pool {hsa.host_bytes(hs.cfg) / 2**30:.2f} GiB filled in {time.perf_counter() - t0:.1f}s")
    qs = torch.from_numpy(np.stack([skv.queries(w.seed, t % 8, w.n, 0, 16) for t in range(8)]).view(np.int16)) \
        .cuda().view(torch.bfloat16)
    # each step's newest token (position len - 1), appended before the step's resolve; its row
    # is the history's own, so the appends keep history and device pages consistent
    newest = np.array([w.len_tokens(t) - 1 for t in range(T)], dtype=np.int64)
    d_pos = torch.from_numpy(np.repeat(newest[:, None], w.n, axis=1).astype(np.int32)).cuda()
    d_new = torch.from_numpy(np.stack([skv.rows_at(w.seed, r, 0, newest, w.layout) for r in range(w.n)], axis=1)).cuda()
    slot_new = torch.empty(w.n, dtype=torch.int32, device="cuda")
    slots = torch.empty(T, w.n, w.k, dtype=torch.int32, device="cuda")
    miss = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    miss_r = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    out = torch.empty(w.n, 16, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.n, 16, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(576)
    stream = torch.cuda.Stream()

    def timed(g):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def warm(h, m, attend):
        with torch.cuda.stream(stream):
            for t in range(args.warmup):
                if attend:
                    h.append(0, d_pos[t], d_new[t], slot_new, stream=stream)
                h.resolve(0, d_trace[t], slots[t], m[t], stream=stream)
                if attend:
                    h.attend_pages(0, qs[t % 8], slots[t], d_trace[t], lens[t], scale, out, lse, stream=stream)
        stream.synchronize()

    # resolve alone (the fused kernel: tables and page copies), from an empty cache
    warm(hs, miss_r, False)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for t in range(args.warmup, T):
                hs.resolve(0, d_trace[t], slots[t], miss_r[t], stream=stream)
    resolve_us = timed(g) / K * 1e3
    del g
    # whole steps, from an empty cache again
    hs.reset_requests(0, w.n)
    torch.cuda.synchronize()
    warm(hs, miss, True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for t in range(args.warmup, T):
                hs.append(0, d_pos[t], d_new[t], slot_new, stream=stream)
                hs.resolve(0, d_trace[t], slots[t], miss[t], stream=stream)
                hs.attend_pages(0, qs[t % 8], slots[t], d_trace[t], lens[t], scale, out, lse, stream=stream)
    region_ms = timed(g)
    del g
    assert torch.equal(miss, miss_r)      # appends change no table
    out_serial = out.clone()
    # whole steps again with the attention split by residency: the part over resident pages runs
    # beside the copy of the missing pages, the part over the fetched pages after it
    from hierarchical_kv_cache_hs_amd.decode_step import attend_while_fetching
    side = torch.cuda.Stream()
    miss_o = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    hs.reset_requests(0, w.n)
    torch.cuda.synchronize()
    warm(hs, miss_o, True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for t in range(args.warmup, T):
                hs.append(0, d_pos[t], d_new[t], slot_new, stream=stream)
                attend_while_fetching(hs, 0, d_trace[t], qs[t % 8], scale, slots[t], miss_o[t], out, lse, stream, side,
                                      lens=lens[t])
    overlap_ms = timed(g)
    del g
    overlap_ok = torch.equal(miss_o, miss) and (out.float() - out_serial.float()).abs().max().item() <= 2e-2
    log(f"pages: whole step {region_ms / K * 1e3:.1f} us serial, {overlap_ms / K * 1e3:.1f} us with the split attention")
    # the appends alone, on the final state (write-through into resident pages and the history)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for t in range(args.warmup, T):
                hs.append(0, d_pos[t], d_new[t], slot_new, stream=stream)
    append_us = timed(g) / K * 1e3
    del g
    # attention alone, cold (a 1 GiB read before each launch evicts the rows from the caches)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    att_ms = []
    with torch.cuda.stream(stream):
        for t in range(args.warmup, T):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hs.attend_pages(0, qs[t % 8], slots[t], d_trace[t], lens[t], scale, out, lse, stream=stream)
            b.record(stream)
            b.synchronize()
            att_ms.append(a.elapsed_time(b))
    del flush
    # resolution alone: a handle that moves no rows
    hs_noio = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 0, hsa.FLAG_NO_IO, page_tokens=P)
    miss_n = torch.zeros(T, w.n, dtype=torch.int32, device="cuda")
    slots_n = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            hs_noio.resolve(0, d_trace[t], slots_n, miss_n[t], stream=stream)
    stream.synchronize()
    gn = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gn, stream=stream):
            for t in range(args.warmup, T):
                hs_noio.resolve(0, d_trace[t], slots_n, miss_n[t], stream=stream)
    noio_us = timed(gn) / K * 1e3
    del gn
    assert torch.equal(miss_n[args.warmup:], miss[args.warmup:])
    hs_noio.close()

    att_s = float(np.mean(att_ms)) / 1e3
    # attended rows per launch: valid pages' tokens below the context length
    S = d_trace[args.warmup:].long()
    off = torch.arange(P, device="cuda")
    tok = S[..., None] * P + off
    ok = (S[..., None] >= 0) & (tok < lens[args.warmup:, :, None, None])
    rows_per_launch = ok.sum().item() / K
    att_bytes = w.n * (8 * w.k + 4) + rows_per_launch * w.entry_bytes + w.n * 16 * (576 * 2 + 512 * 2 + 4)
    achieved = att_bytes / att_s / 1e9
    m = miss[args.warmup:].double().mean().item()
    page_bytes = P * w.entry_bytes
    fetch_Bps = m * w.n * page_bytes / (resolve_us * 1e-6)
    step_tokens = w.n * w.k * P
    # the line's value: the faster of the two step schedules (the split one only if its attention
    # stayed within the bf16 tier of the serial run)
    split_best = overlap_ok and overlap_ms < region_ms
    best_ms = overlap_ms if split_best else region_ms
    line = {
        "metric": "attended tokens/s through append + resolve + attention over page selections, 1 MI355X",
        "value": step_tokens * K / (best_ms / 1e3),
        "unit": "attended tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": best_ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.description, "global_batch": w.n, "page_tokens": P, "seq_len": w.len_tokens(0),
                   "top_k_pages": w.k, "device_buffer_pages": w.B, "heads": 16, "graph": True,
                   "schedule": "attention split by residency" if split_best else "serial"},
        "page_selections_per_s": w.n * K / (best_ms / 1e3),
        # the same steps with the attention split by residency (resident pages beside the copy)
        "attend_while_fetching": {"us_per_step": overlap_ms / K * 1e3, "serial_us_per_step": region_ms / K * 1e3,
                                  "attended_tokens_per_s": step_tokens * K / (overlap_ms / 1e3),
                                  "within_bf16_tier_of_serial": bool(overlap_ok)},
        "append_us_per_step": append_us,
        "resolve_us_per_step": resolve_us,
        "resolve_noio_us_per_step": noio_us,
        "misses_per_selection_pages": m,
        "miss_fetch_GBps": fetch_Bps / 1e9,
        "miss_fetch_frac_of_link": fetch_Bps / 1e9 / PCIE_GEN5_X16_GBPS,
        "attention_us": att_s * 1e6,
        "attention_tokens_per_s": rows_per_launch / att_s,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": recorded_traffic("attend_pages", "attend.hip"),
                     "kernel": "attend_kernel", "avg_kernel_us": att_s * 1e6, "algorithmic_bytes_per_launch": att_bytes},
    }
    hs.close()
    return line, trace


def fill_history(torch, hs, w):
    """Every history row of a handle from the seeded generator: whole rows into the host pool,
    or with the resident-tail layout the first 640 bytes of each row there and the last 16
    into the device tail plane."""
    from synth import kv as skv
    for l in range(hs.L):
        tails = hs.tail_plane(l) if hs.tail_bytes else None
        for r in range(hs.n):
            ptr, cap, stride = hs.host_kv_ptr(l, r)
            if tails is None:
                skv.fill_rows(w.seed, r, l, 0, cap, w.layout, ptr, stride)
            else:
                stage = np.empty((cap, hs.tail_bytes), dtype=np.uint8)
                skv.fill_rows_split(w.seed, r, l, 0, cap, w.layout, ptr, stride, stride, stage.ctypes.data,
                                    hs.tail_bytes)
                tails[r].copy_(torch.from_numpy(stage))
    torch.cuda.synchronize()


def bench_prefetch(args, torch, hsa, w):
    """Whole decode steps over 8 layers sharing one selection (128 requests, ctx 65536, fp8 rows,
    k 2048, B 4096): every layer resolves the step's selection (hit detection, LRU replacement,
    table update, host-to-device fetch of the misses) and attends over its resolved slots.
    Schedules: serial (resolve and attend layer after layer), layer-wise prefetch (the tables of
    every layer on one side stream, the row copies on another, each attention waiting for its
    layer's copy), prefetch with each attention split by residency, and prefetch with the
    attention of only the last 1 or 3 layers split.  Each is captured as one
    hipGraph of exactly --steps steps, replayed after --warmup untimed steps from an empty
    buffer; the line's value is the fastest schedule whose outputs match the serial run.  The
    host pool keeps whole 656-byte rows."""
    from hierarchical_kv_cache_hs_amd.decode_step import DecodeSteps
    from synth import kv as skv
    from synth import trace as tr

    K, W = args.steps, args.warmup
    T = W + K
    w = w.with_(steps=max(w.steps, T))
    t0 = time.perf_counter()
    trace = tr.generate(w.trace_spec(), steps=T)
    log(f"trace {trace.shape} in {time.perf_counter() - t0:.1f}s")
    d_trace = torch.from_numpy(trace).cuda()
    hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, w.layers, w.layout, 16, 0)
    t0 = time.perf_counter()
    fill_history(torch, hs, w)
    log(f"host pool {hsa.host_bytes(hs.cfg) / 2**30:.1f} GiB filled in {time.perf_counter() - t0:.1f}s")
    # every step and layer has its own queries
    t0 = time.perf_counter()
    qsteps = [torch.from_numpy(np.stack([skv.queries(w.seed, t, w.n, l, 16) for l in range(w.layers)]).view(np.int16))
              .cuda().view(torch.bfloat16) for t in range(T)]
    log(f"queries for {T} steps in {time.perf_counter() - t0:.1f}s")
    scale = 1.0 / math.sqrt(576)
    sels = [d_trace[t] for t in range(T)]

    def warm(attend):
        hs.reset_requests(0, w.n)
        if W:
            DecodeSteps(hs, sels[:W], qsteps[:W], scale, prefetch=False, attend=attend).replay()

    def timed(prefetch, attend, split_attention=False, split_last=0):
        warm(attend)
        steps = DecodeSteps(hs, sels[W:], qsteps[W:], scale, prefetch=prefetch, attend=attend,
                            split_attention=split_attention, split_last=split_last)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(steps.stream):
            a.record(steps.stream)
            steps.graph.replay()
            b.record(steps.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K, steps

    t_ser, s_ser = timed(False, True)
    t_pre, s_pre = timed(True, True)
    same = torch.equal(s_ser.out, s_pre.out) and torch.equal(s_ser.miss, s_pre.miss) and \
        torch.equal(s_ser.lse, s_pre.lse)
    del s_pre

    # an attention merged from two parts equals the single launch up to fp32 summation order
    def close(s_x):
        return torch.equal(s_ser.miss, s_x.miss) and torch.equal(s_ser.slots, s_x.slots) and \
            (s_ser.out.float() - s_x.out.float()).abs().max().item() <= 2e-2

    t_spl, s_x = timed(True, True, split_attention=True)
    spl_close = close(s_x)
    # the attention of the last m layers split by residency: their resident parts run beside the
    # last copies (on the compute units the copy kernel leaves free)
    t_lst, lst_close = {}, {}
    for m in (1, 3):
        t_lst[m], s_x = timed(True, True, split_last=m)
        lst_close[m] = close(s_x)
    del s_x
    t_res, _ = timed(False, False)
    log(f"serial {t_ser:.3f} ms, prefetch {t_pre:.3f} ms, prefetch + split attention {t_spl:.3f} ms, "
        + ", ".join(f"prefetch + last {m} split {t:.3f} ms" for m, t in t_lst.items())
        + f", resolve only {t_res:.3f} ms per step")
    schedules = [(t_pre, "prefetch")]
    if spl_close:
        schedules.append((t_spl, "prefetch, attention split by residency"))
    for m, t in t_lst.items():
        if lst_close[m]:
            schedules.append((t, f"prefetch, attention of the last {m} layer{'s' if m > 1 else ''} split by residency"))
    t_best, best_name = min(schedules)
    misses = s_ser.miss.double()                                  # [K][L][n]
    # bytes each miss moves over the host link: the whole row, or its host part (the rest comes
    # from the device tail plane)
    link_bytes = w.entry_bytes - hs.tail_bytes
    miss_bytes_step = float(misses.sum()) * link_bytes / K

    # The row-copy kernel (fetch_kernel) timed on its own stream: the same steps again, enqueued
    # without a graph in the prefetch schedule (a captured graph exposes no per-kernel time on
    # this platform), with HIP events on the copy stream before each step's first copy launch and
    # after its last; there the copies wait once for the step's tables and then run back to back,
    # beside the attention of earlier layers, so the span over the launch count is the average
    # launch duration (the dispatch gaps between the copies included).
    warm(True)
    # (the prefetch schedule without the split attention: there the copies have a stream of their
    # own, so nothing else runs between the step's first and last copy on it)
    eager = DecodeSteps(hs, sels[W:], qsteps[W:], scale, prefetch=True, attend=True, split_attention=False,
                        capture=False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(eager.stream)
    eager.run_eager(time_fetches=True)
    e1.record(eager.stream)
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) / K
    fetch_ms = np.array([a.elapsed_time(b) for a, b in eager.fetch_events])   # per step, L launches
    assert fetch_ms.size == K and torch.equal(eager.miss, s_ser.miss)
    fetch_bytes_launch = miss_bytes_step / w.layers
    fetch_avg_s = float(fetch_ms.sum()) / (K * w.layers) / 1e3
    fetch_GBps = fetch_bytes_launch / fetch_avg_s / 1e9
    log(f"fetch_kernel: {fetch_avg_s * 1e6:.1f} us per launch ({K * w.layers} launches), {fetch_GBps:.1f} GB/s; "
        f"eager step {t_eager:.3f} ms")

    # attention alone over the 8 layers (each launch reads another layer's rows), K steps
    ga = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(ga, stream=st):
            for i in range(K):
                for l in range(w.layers):
                    hs.attend(l, qsteps[W + i][l], s_ser.slots[l], scale, s_ser.out[l], s_ser.lse[l], stream=st)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        a.record(st)
        ga.replay()
        b.record(st)
    torch.cuda.synchronize()
    t_att_only = a.elapsed_time(b) / K
    del ga
    valid = float((s_ser.slots >= 0).sum().item()) / w.layers
    att_bytes = valid * w.entry_bytes + w.n * (4 * w.k + 16 * (576 * 2 + 512 * 2 + 4))   # per launch
    h2d = measure_h2d_peak(torch)
    log(f"H2D memcpy peak {h2d:.1f} GB/s")
    t_att = t_ser - t_res
    step_GBps = miss_bytes_step / (t_best / 1e3) / 1e9
    traffic = recorded_traffic("fetch_prefetch_c4", "resolve.hip")
    out = {
        "metric": "resolved top-k selections/s + miss-fetch GB/s vs host-link peak, 1 MI355X",
        "value": w.n * w.layers / (t_best / 1e3), "unit": "selections/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": t_best, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # resolution is integer work; the attention computes in bf16 (fp8 rows decoded exactly)
        # with fp32 accumulation
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.description, "global_batch": w.n, "layers": w.layers, "seq_len": w.ctx,
                   "top_k": w.k, "device_buffer_size": w.B, "host_to_device_ratio": w.ratio,
                   "entry_bytes": w.entry_bytes, "kv_rows": "fp8 e4m3 latent + fp32 scales + bf16 rope",
                   "host_rows": "whole 656-B rows in the host pool",
                   "graph": True, "steps_timed": f"{W}..{W + K - 1}", "queries": "distinct per step and layer",
                   "schedule": best_name},
        "selected_tokens_per_s": w.n * w.layers * w.k / (t_best / 1e3),
        "attended_tokens_per_s": w.n * w.layers * w.k / (t_best / 1e3),
        "misses_per_selection": float(misses.mean()),
        "link_bytes_per_miss": link_bytes,
        "miss_GB_per_step": miss_bytes_step / 1e9,
        # whole-step miss rate: the step's miss bytes over its time
        "miss_fetch_GBps": step_GBps,
        "miss_fetch_frac_of_link": step_GBps / PCIE_GEN5_X16_GBPS,
        "miss_fetch_frac_of_measured_peak": step_GBps / h2d,
        "h2d_peak_GBps_measured": h2d,
        "serial_ms_per_step": t_ser, "prefetch_ms_per_step": t_pre, "prefetch_split_attention_ms_per_step": t_spl,
        "resolve_only_ms_per_step": t_res,
        "eager_ms_per_step": t_eager,
        "prefetch_equals_serial": bool(same),
        "prefetch_split_attention_within_bf16_tier_of_serial": bool(spl_close),
        "prefetch_split_last_ms_per_step": {str(m): t for m, t in t_lst.items()},
        "prefetch_split_last_within_bf16_tier_of_serial": {str(m): bool(c) for m, c in lst_close.items()},
        "overlap_saved_ms_per_step": t_ser - t_best,
        "attention_ms_per_step": t_att,
        "attention_hidden_fraction": (t_ser - t_best) / t_att if t_att > 0 else None,
        "attention_alone": {"ms_per_step": t_att_only, "us_per_launch": t_att_only * 1e3 / w.layers,
                            "bytes_per_launch": att_bytes,
                            "GBps": att_bytes * w.layers / (t_att_only / 1e3) / 1e9,
                            "frac_of_hbm": att_bytes * w.layers / (t_att_only / 1e3) / 1e9 / HBM_PEAK_GBPS},
        # the dominant kernel: the row copies over the host link, timed launch by launch
        "roofline": {"bound": "host_link", "achieved": fetch_GBps, "peak": PCIE_GEN5_X16_GBPS, "unit": "GB/s",
                     "frac": fetch_GBps / PCIE_GEN5_X16_GBPS, "traffic": traffic, "kernel": "fetch_kernel",
                     "avg_kernel_us": fetch_avg_s * 1e6, "launches_timed": int(K * w.layers),
                     "algorithmic_bytes_per_launch": fetch_bytes_launch,
                     "frac_of_measured_peak": fetch_GBps / h2d,
                     "timing": "HIP events on the copy stream around each step's 8 back-to-back copy launches, "
                               "the timed steps re-run without a graph in the prefetch schedule"},
    }
    hs.close()
    return out, trace


def bench_extras(args, torch, hsa):
    """The 64-request resolve-only and the 256-request resolve + attention workloads, run beside
    the headline with the same --steps / --warmup: their rates go into the line as extra keys."""
    from synth import configs as C
    res, _ = bench_resolve(args, torch, hsa, C.BATCH64)
    keep = ("value", "ms_per_step", "misses_per_selection", "miss_fetch_GBps", "miss_fetch_frac_of_measured_peak",
            "resolve_only", "roofline", "config")
    c1 = {k: res[k] for k in keep}
    c1["unit"] = res["unit"]
    att = bench_attend(args, torch, hsa, C.FP8_256, legs=False)
    keep = ("value", "unit", "ms_per_step", "resolve_noio_us_per_step", "resolve_noio_cold_us_per_step",
            "attention_f32_output_us", "misses_per_selection", "hbm_resolve_plus_attend", "resident_tail", "roofline",
            "config")
    c2 = {k: att[k] for k in keep}
    return {"resolve_64_requests_bf16": c1, "resolve_attend_256_requests_fp8": c2}


def bench_attend_cost(args, torch, hsa):
    """Where a sparse-attention launch spends its time (fp8 rows, 256 requests, 16 heads, one
    workgroup per request): launches over k = 64 .. 2048 selected rows per request, each timed
    cold (after a 1 GiB read that evicts the caches) with HIP events on the launch stream, and
    the same launches over only 64 distinct rows per request, read over and over (they stay in
    the caches, so the time is the kernel's own tile pipeline).  A least-squares line over k
    gives the time per 64-token tile and the fixed time per launch, for both."""
    n, H, B = 256, 16, 2048
    ks = (64, 256, 512, 1024, 2048)
    reps = max(5, min(args.steps, 40))
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    scale = 1.0 / math.sqrt(576)
    times = {"hbm": {}, "cached": {}}
    for k in ks:
        hs = hsa.HiSparse(k, B, 1, n, 1, hsa.LAYOUT_FP8, H, hsa.FLAG_NO_IO)
        buf = hs.state(0)["kv_buffer"]
        g = torch.Generator(device="cuda")
        g.manual_seed(1000 + k)
        # bytes below 64: finite fp8 codes, bf16 rope values and scales of moderate size
        buf.copy_(torch.randint(0, 64, buf.shape, dtype=torch.uint8, device="cuda", generator=g))
        perm = torch.argsort(torch.rand(n, B, device="cuda", generator=g), dim=1).to(torch.int32)
        q = (torch.randn(n, H, 576, device="cuda", generator=g) * 0.1).to(torch.bfloat16).contiguous()
        out = torch.empty(n, H, 512, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(n, H, dtype=torch.float32, device="cuda")
        for kind, slots in (("hbm", perm[:, :k].contiguous()),
                            ("cached", perm[:, :64].repeat(1, k // 64).contiguous())):
            assert slots.shape == (n, k) and int(slots.min()) >= 0 and int(slots.max()) < B
            us = []
            with torch.cuda.stream(stream):
                for i in range(args.warmup + reps):
                    if kind == "hbm":
                        flush.sum()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    hs.attend(0, q, slots, scale, out, lse, stream=stream)
                    b.record(stream)
                    b.synchronize()
                    if i >= args.warmup:
                        us.append(a.elapsed_time(b) * 1e3)
            assert bool(torch.isfinite(lse).all())
            times[kind][k] = float(np.median(us))
            log(f"attend cost k {k} {kind}: {times[kind][k]:.1f} us")
        hs.close()
        del buf
    fit = {}
    for kind, t in times.items():
        tiles = np.array([k / 64 for k in ks])
        slope, icpt = np.polyfit(tiles, np.array([t[k] for k in ks]), 1)
        fit[kind] = {"us_per_tile": float(slope), "us_fixed": float(icpt)}
    tile_bytes = n * 64 * 656
    t2048 = times["hbm"][2048]
    return {
        "metric": "sparse MLA attention launch time vs selected rows per request, 1 MI355X",
        "value": t2048, "unit": "us per launch (k 2048, cold, HIP events)",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup, "ms_per_step": t2048 / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "256 requests, 16 heads, fp8 656-byte rows, k 64..2048, 2048 slots",
                   "global_batch": n, "top_k": list(ks)},
        "us_per_launch": {kind: {str(k): v for k, v in t.items()} for kind, t in times.items()},
        "fit": fit,
        "tile_bytes": tile_bytes,
        "tile_GBps_hbm": tile_bytes / (fit["hbm"]["us_per_tile"] * 1e-6) / 1e9,
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=190)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefetch",
                    choices=["prefetch", "batch64", "fp8_256", "sweep", "topk", "pages", "attend_cost"])
    ap.add_argument("--no-extras", action="store_true",
                    help="prefetch workload: skip the 64- and 256-request workloads run beside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--summarize-profile", action="store_true",
                    help="print a markdown summary of rocprofv3 csv output (--trace-dir, --kernel, ...)")
    ap.add_argument("--trace-dir")
    ap.add_argument("--kernel")
    ap.add_argument("--last", type=int, default=0)
    ap.add_argument("--pmc-dir", help="prefix of the counter runs' directories (<prefix>_FETCH_SIZE, ...)")
    ap.add_argument("--copy-dir", help="prefix of the copy-calibration counter runs' directories")
    ap.add_argument("--pmc-last", type=int, default=0)
    ap.add_argument("--skip", type=int, default=0, help="with --last: take --last dispatches after the first --skip")
    ap.add_argument("--pmc-skip", type=int, default=0, help="the same for the counter runs")
    ap.add_argument("--record", help="store the traffic under this key in profiles/traffic.json")
    ap.add_argument("--source", default="resolve.hip", help="kernel source file the record is keyed to")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 256 MiB (x5), to scale hardware byte counters")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    import torch
    import hierarchical_kv_cache_hs_amd as hsa
    from synth import configs as C

    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4}))
        return
    if args.workload == "batch64":
        line, trace = bench_resolve(args, torch, hsa, C.BATCH64)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_resolve(C.BATCH64, trace, args.warmup, args.cpu_budget)
            log(f"cpu baseline {line['cpu_baseline']['value']:.1f} selections/s")
        else:
            line["cpu_baseline"] = None
    elif args.workload == "prefetch":
        line, trace = bench_prefetch(args, torch, hsa, C.PREFETCH)
        if not args.no_extras:
            line["other_workloads"] = bench_extras(args, torch, hsa)
        line["cpu_baseline"] = None if args.no_cpu_baseline else \
            cpu_baseline_prefetch(C.PREFETCH.with_(steps=trace.shape[0]), trace, args.warmup, args.cpu_budget)
    elif args.workload == "sweep":
        line = bench_sweep(args, torch, hsa)
    elif args.workload == "topk":
        line = bench_topk(args, torch, hsa)
    elif args.workload == "attend_cost":
        line = bench_attend_cost(args, torch, hsa)
    elif args.workload == "pages":
        line, trace = bench_pages(args, torch, hsa, C.PAGES)
        line["cpu_baseline"] = None if args.no_cpu_baseline else \
            cpu_baseline_pages(C.PAGES, trace, args.warmup, args.cpu_budget)
    else:
        line = bench_attend(args, torch, hsa, C.FP8_256)
        line["cpu_baseline"] = None if args.no_cpu_baseline else \
            cpu_baseline_attend(C.FP8_256, args.warmup, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
