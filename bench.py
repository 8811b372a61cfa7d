#!/usr/bin/env python3
"""Benchmark of sparse paged decode attention on one MI355X.

A step is one ``sda_decode`` call (the split kernel, plus the combine kernel
when splits > 1) over one batch of the workload.  Inputs are resident in HBM
before timing.  The step rotates among ``--sets`` independently drawn
query/selection sets over the same cache, so back-to-back calls do not reuse
the last-level cache.

Prints ONE JSON line.  ``value`` is the effective KV bandwidth in GB/s.  The
algorithmic bytes of a call are the visible selected K|V rows plus Q of the
active rows, plus the output of every row; the K calls' total is divided by
the wall time of the timed region.  Each input set's argument block is
marshalled once before timing; a step is one C call.  ``roofline`` compares
the per-launch algorithmic bytes with the average launch duration (two HIP
events on the launch stream around the timed region) against the 8 TB/s HBM
peak.
``cpu_baseline`` times the fp64 oracle on a bounded sample of rows on the
host cores.

``--swa NAME`` measures the gated sliding-window decode (``sda_swa_decode``)
on one of its workloads instead; its algorithmic bytes are each row's window
of K|V rows, plus Q and the output.  ``--select NAME`` measures region
selection (``sda_select_regions``): its bytes are the candidate scores, the
row metadata and the selected ids.  ``--logits NAME`` measures the decode
indexer logits (``sda_indexer_logits``): its bytes are each request's scored
region summaries and scales (read once per request), the queries and
weights, and the fp32 score matrix written.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "effective KV GB/s (% of HBM peak) and rows/s for sparse decode attention"
KERNEL_SRC = os.path.join(ROOT, "sparse_paged_decode_02_amd", "csrc", "sda_kernels.hip")
SELECT_SRC = os.path.join(ROOT, "sparse_paged_decode_02_amd", "csrc", "sda_select.hip")
LOGITS_SRC = os.path.join(ROOT, "sparse_paged_decode_02_amd", "csrc", "sda_logits.hip")


def kernel_hash() -> str:
    """First 16 hex digits of the kernel source's SHA-256 (ties counters to code)."""
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def select_kernel_hash() -> str:
    with open(SELECT_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def logits_kernel_hash() -> str:
    with open(LOGITS_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(w, positions, regions, active) -> tuple:
    """(bytes, visible tokens) of one call: visible selected K|V token rows
    (384 elements each) and Q (heads x 192 bf16) of active rows, plus the
    output (heads x 192 bf16) of every row."""
    e = 1 if w.kv == "fp8" else 2
    rt = w.rt
    reg = regions.astype(np.int64)
    pos = positions.astype(np.int64)[:, None]
    t0 = reg * rt
    vis = np.where(reg >= 0, np.clip(pos - t0 + 1, 0, rt), 0)
    tokens = int((vis.sum(axis=1) * (active != 0)).sum())
    nact = int((active != 0).sum())
    q = nact * w.heads * 192 * 2
    out = w.rows * w.heads * 192 * 2
    return tokens * 384 * e + q + out, tokens


def workload_desc(w) -> str:
    return ("%s: %d rows = %d req x qlen %d x G %d, %d heads x 192, %s cache, block %d, "
            "R %d, context %d" % (w.name, w.rows, w.requests, w.query_len, w.groups, w.heads,
                                  w.kv, w.block, w.R, w.pages_per_req * w.block))


def swa_algorithmic_bytes(w, seq_lens) -> tuple:
    """(bytes, K|V tokens) of one sliding-window call: for every request and
    KV group, the K|V token rows (384 bf16) of the union of its query tokens'
    windows, each read once; plus Q and output (heads x 192 bf16) of every
    row."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    last = lens - 1
    first = np.maximum(0, lens - w.query_len - w.window + 1)
    ntok = np.clip(last - first + 1, 0, None)
    tokens = int(ntok.sum()) * w.groups
    return tokens * 384 * 2 + 2 * w.rows * w.heads * 192 * 2, tokens


def swa_workload_desc(w) -> str:
    return ("%s: %d rows = %d req x qlen %d x G %d, %d heads x 192, bf16 cache, block %d, "
            "window %d, seq_len U[%d,%d]" % (w.name, w.rows, w.requests, w.query_len, w.groups,
                                            w.heads, w.block, w.window, w.seq_lo, w.seq_hi))


# Untimed calls before the warmup steps, until this much back-to-back work has
# run.  After the GPU has idled (the host draws the next workload's inputs),
# the first ~15 ms of calls run up to 15% slower (large-batch FP8 on MI355X:
# 540 us on average over calls 5..25 after a 3 s idle, 498 us once settled);
# decode steps in serving run back to back.
SETTLE_MS = 50.0


def settle(call, stream, settle_ms: float = SETTLE_MS) -> int:
    """Run calls until settle_ms of wall time has passed; returns the count."""
    import torch
    n = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            call(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_calls(call, steps: int, warmup: int, stream, settle_ms: float = SETTLE_MS):
    """Settle, warm up, then time `steps` back-to-back calls: wall seconds
    (between synchronisations), average launch ms (two HIP events on the
    launch stream around the timed region) and a second pass of per-launch
    durations.  The settle count is kept in time_calls.settled."""
    import torch
    time_calls.settled = settle(call, stream, settle_ms) if settle_ms > 0 else 0
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_avg_ms = ev0.elapsed_time(ev1) / steps
    # Distribution of single-launch durations: a second pass over the same K
    # calls with events around each launch (kept out of the timed region).
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        call(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([starts[i].elapsed_time(ends[i]) for i in range(steps)])
    return wall, launch_avg_ms, launch_ms


def time_flushed(call, steps: int, stream, flush_mib: int) -> dict:
    """Per-call durations with `flush_mib` MiB written between calls (outside
    the events), so that no call finds the previous calls' bytes in the
    last-level cache: a cross-check of the rotating input sets."""
    import torch
    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device=stream.device)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        buf.fill_(i & 0xFF)
        starts[i].record(stream)
        call(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    us = np.array([starts[i].elapsed_time(ends[i]) * 1e3 for i in range(steps)])
    del buf
    return {"flush_mib": flush_mib, "calls": steps, "median_us": round(float(np.median(us)), 2),
            "p10_us": round(float(np.percentile(us, 10)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2)}


def record(args, *, value, wall, launch_avg_ms, launch_ms, bytes_per_launch, rows, dtype,
           config, kernel, traffic, metric=METRIC):
    achieved = bytes_per_launch / (launch_avg_ms * 1e-3) / 1e9
    settled = getattr(time_calls, "settled", 0)
    return {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": config,
        "settle_calls": settled,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "rows_per_s": round(rows * args.steps / wall, 1),
        "us_per_call": {"median": round(float(np.median(launch_ms)) * 1e3, 2),
                        "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                        "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "avg_launch_us": round(launch_avg_ms * 1e3, 3),
        },
    }


def swa_cpu_baseline(inp, gpu_out, rows_sample: int, threads: int, min_seconds: float):
    """Time the fp64 oracle (as it stands) on a sample of sliding-window rows,
    repeated until min_seconds of host time have been spent."""
    from oracle import oracle
    from oracle.hostprep import swa_host_problem

    w = inp.w
    rng = np.random.default_rng(0)
    rows = sorted(rng.choice(w.rows, size=min(rows_sample, w.rows), replace=False).tolist())
    hp = swa_host_problem(inp.query, inp.cache, inp.block_table, inp.seq_lens, scale=inp.scale,
                          window=w.window, query_len=w.query_len, gate=inp.gate, rows=rows)
    passes, dt, out = timed_passes(lambda: oracle.swa_decode(hp, rows=rows, threads=threads),
                                   min_seconds)
    lens = inp.seq_lens.cpu().numpy().astype(np.int64)
    ntok = 0
    for r in rows:
        tok = r // w.groups
        req, j = tok // w.query_len, tok % w.query_len
        ntok += max(0, min(int(lens[req]) - w.query_len + j + 1, w.window))
    nbytes = ntok * 384 * 2 + 2 * len(rows) * w.heads * 192 * 2
    g = gpu_out.float().cpu().numpy().astype(np.float64).reshape(w.rows, w.heads, 192)[rows]
    err = np.abs(g - out[rows])
    return {
        "value": passes * nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d rows of the first input set, %d passes (fp64 C oracle, %d threads), "
                  "%.2f s wall; rows/s %.1f" % (len(rows), passes, threads, dt,
                                               passes * len(rows) / dt),
        "parity_max_abs": float(err.max()),
        "parity_mean_abs": float(err.mean()),
    }


def run_swa(args, dev) -> int:
    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    w = gen.SWA_WORKLOADS[args.swa]
    pack, plan_splits = B.sda_swa_plan(w.tokens, w.groups, w.heads, w.query_len, w.window)
    pack = args.pack or pack
    splits = args.splits or w.splits or plan_splits
    print("[bench] drawing %s" % swa_workload_desc(w), file=sys.stderr, flush=True)
    base = gen.make_swa_inputs(w, device=dev, splits=splits)
    sets = [base] + [gen.make_swa_inputs(w, device=dev, seed=w.seed + 100003 * i,
                                         cache=base.cache, splits=splits)
                     for i in range(1, args.sets)]
    nbytes = [swa_algorithmic_bytes(w, s.seq_lens.cpu().numpy())[0] for s in sets]
    outs = [torch.empty_like(s.query) for s in sets]
    ws_bytes = B.sda_workspace_bytes(w.rows, w.heads, splits)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    prepared = []
    for s, o in zip(sets, outs):
        B.check_swa_tensors(s.query, s.cache, s.block_table, s.seq_lens, o, s.gate)
        prepared.append(B.make_swa_args(
            s.query, s.cache, s.block_table, s.seq_lens, o, scale=s.scale, window=w.window,
            query_len=w.query_len, splits=splits, pack=pack, gate=s.gate,
            workspace=workspace if ws_bytes else None))

    def call(i):
        rc = B.sda_swa_decode_raw(prepared[i % len(prepared)], handle)
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    wall, launch_avg_ms, launch_ms = time_calls(call, args.steps, args.warmup, stream, args.settle_ms)
    total_bytes = sum(nbytes[i % len(sets)] for i in range(args.steps))
    bytes_per_launch = float(np.mean([nbytes[i % len(sets)] for i in range(args.steps)]))
    rec = record(args, value=total_bytes / wall / 1e9, wall=wall, launch_avg_ms=launch_avg_ms,
                 launch_ms=launch_ms, bytes_per_launch=bytes_per_launch, rows=w.rows,
                 dtype="bf16",
                 config={"workload": swa_workload_desc(w), "rows": w.rows, "heads": w.heads,
                         "splits": splits, "pack": pack, "input_sets": len(sets),
                         "seed": w.seed},
                 kernel="sda split kernel, window mode" + (
                     " + combine" if splits > 1 else " (combine fused)"),
                 traffic=load_traffic(w.name, splits) if pack == B.sda_swa_plan(
                     w.tokens, w.groups, w.heads, w.query_len, w.window)[0] else None,
                 metric="effective KV GB/s (% of HBM peak) and rows/s for gated "
                        "sliding-window decode")
    if not args.no_cpu_baseline:
        threads, why = host_threads()
        print("[bench] cpu baseline: oracle on %d rows, %d threads (%s)"
              % (args.cpu_rows, threads, why), file=sys.stderr, flush=True)
        rec["cpu_baseline"] = swa_cpu_baseline(base, outs[0], args.cpu_rows, threads,
                                               args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def select_algorithmic_bytes(w, lengths) -> int:
    """Candidate scores (fp32) + current and length (int32) per row + the
    int32 [rows, topk] output."""
    n = np.clip(np.asarray(lengths, dtype=np.int64), 0, w.num_regions)
    return int(n.sum()) * 4 + w.rows * 8 + w.rows * w.topk * 4


def select_cpu_baseline(inp, gpu_out, min_seconds: float):
    """Time the oracle's selection (as it stands, one host thread) on the
    first input set, repeated until min_seconds have been spent."""
    from oracle import oracle
    s = inp.scores.cpu().numpy()
    cur = inp.current.cpu().numpy()
    lens = inp.topk_lengths.cpu().numpy()
    passes, dt, ref = timed_passes(lambda: oracle.select_regions(s, cur, inp.w.topk, lens),
                                   min_seconds)
    nbytes = select_algorithmic_bytes(inp.w, lens)
    return {
        "value": passes * nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "all %d rows of the first input set, %d passes (C oracle: sort per row, one "
                  "thread), %.2f s wall; rows/s %.1f" % (inp.w.rows, passes, dt,
                                                         passes * inp.w.rows / dt),
        "parity_exact": bool(np.array_equal(gpu_out.cpu().numpy(), ref)),
    }


def logits_algorithmic_bytes(w, positions) -> int:
    pos = np.asarray(positions, dtype=np.int64).reshape(w.requests, w.query_len * w.groups)
    last = np.where(pos < 0, -1, pos // w.region_tokens).max(axis=1)
    nreg = np.clip(last + 1, 0, w.num_regions)
    summaries = int(nreg.sum()) * (256 + 4)
    per_row = w.heads * 256 + w.heads * 4 + 4 + 8
    return summaries + w.rows * per_row + w.rows * w.num_regions * 4


def logits_cpu_baseline(inp, gpu_out, rows_sample: int, threads: int, min_seconds: float):
    from oracle import oracle
    from oracle.hostprep import logits_host_problem
    w = inp.w
    rng = np.random.default_rng(0)
    rows = sorted(rng.choice(w.rows, size=min(rows_sample, w.rows), replace=False).tolist())
    hp = logits_host_problem(inp, rows=rows)
    passes, dt, ref = timed_passes(lambda: oracle.indexer_logits(hp, rows=rows, threads=threads),
                                   min_seconds)
    pos = inp.positions.cpu().numpy().astype(np.int64)[rows]
    nreg = np.clip(np.where(pos < 0, -1, pos // w.region_tokens) + 1, 0, w.num_regions)
    nbytes = int(nreg.sum()) * 260 + len(rows) * (w.heads * 260 + 12 + w.num_regions * 4)
    g = gpu_out.cpu().numpy().astype(np.float64)[rows]
    r = ref[rows]
    m = np.isfinite(r)
    max_abs = float(np.max(np.abs(g[m] - r[m]))) if m.any() else 0.0
    return {
        "value": passes * nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d rows of the first input set, %d passes (fp64 C oracle, %d threads), "
                  "%.2f s wall; rows/s %.1f" % (len(rows), passes, threads, dt,
                                               passes * len(rows) / dt),
        "parity_max_abs": max_abs,
    }


def run_logits(args, dev) -> int:
    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    w = gen.LOGITS_WORKLOADS[args.logits]
    desc = ("%s: %d rows = %d req x qlen %d x G %d, %d e4m3 heads x 256, %d regions of %d "
            "tokens (%d per page), positions U[%d,%d]"
            % (w.name, w.rows, w.requests, w.query_len, w.groups, w.heads, w.num_regions,
               w.region_tokens, w.rpb, w.pos_lo, w.pos_hi))
    print("[bench] drawing %s" % desc, file=sys.stderr, flush=True)
    base = gen.make_logits_inputs(w, device=dev)
    sets = [base] + [gen.make_logits_inputs(w, device=dev, seed=w.seed + 100003 * i,
                                            summaries=base.summaries, scales=base.scales)
                     for i in range(1, args.sets)]
    nbytes = [logits_algorithmic_bytes(w, s.positions.cpu().numpy()) for s in sets]
    outs = [torch.empty((w.rows, w.num_regions), dtype=torch.float32, device=dev) for _ in sets]
    curs = [torch.empty(w.rows, dtype=torch.int32, device=dev) for _ in sets]
    lens = [torch.empty(w.rows, dtype=torch.int32, device=dev) for _ in sets]
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    prepared = [B.make_logits_args(s.query, s.weights, s.summaries, s.scales, s.block_table,
                                   s.positions, o, groups=w.groups, query_len=w.query_len,
                                   region_tokens=w.region_tokens, current=c, topk_lengths=l)
                for s, o, c, l in zip(sets, outs, curs, lens)]

    def call(i):
        rc = B.sda_indexer_logits_raw(prepared[i % len(prepared)], handle)
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    wall, launch_avg_ms, launch_ms = time_calls(call, args.steps, args.warmup, stream, args.settle_ms)
    total_bytes = sum(nbytes[i % len(sets)] for i in range(args.steps))
    bytes_per_launch = float(np.mean([nbytes[i % len(sets)] for i in range(args.steps)]))
    rec = record(args, value=total_bytes / wall / 1e9, wall=wall, launch_avg_ms=launch_avg_ms,
                 launch_ms=launch_ms, bytes_per_launch=bytes_per_launch, rows=w.rows,
                 dtype="e4m3 inputs, bf16 MFMA, fp32 scores",
                 config={"workload": desc, "rows": w.rows, "num_regions": w.num_regions,
                         "input_sets": len(sets), "seed": w.seed},
                 kernel="logits_kernel", traffic=load_traffic(w.name, 1, "logits_kernel"),
                 metric="effective GB/s (% of HBM peak) and rows/s for decode indexer logits")
    if not args.no_cpu_baseline:
        threads, _ = host_threads()
        print("[bench] cpu baseline: oracle logits", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = logits_cpu_baseline(base, outs[0], args.cpu_rows, threads,
                                                  args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def run_select(args, dev) -> int:
    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    w = gen.SELECT_WORKLOADS[args.select]
    desc = ("%s: %d rows, %d score columns (%d-token regions), topk %d, positions U[%d,%d]"
            % (w.name, w.rows, w.num_regions, w.region_tokens, w.topk, w.pos_lo, w.pos_hi))
    print("[bench] drawing %s" % desc, file=sys.stderr, flush=True)
    sets = [gen.make_select_inputs(w, device=dev, seed=w.seed + 100003 * i)
            for i in range(args.sets)]
    nbytes = [select_algorithmic_bytes(w, s.topk_lengths.cpu().numpy()) for s in sets]
    outs = [torch.empty((w.rows, w.topk), dtype=torch.int32, device=dev) for _ in sets]
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    prepared = [B.make_select_args(s.scores, s.current, w.topk, o, s.topk_lengths)
                for s, o in zip(sets, outs)]

    def call(i):
        rc = B.sda_select_regions_raw(prepared[i % len(prepared)], handle)
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    wall, launch_avg_ms, launch_ms = time_calls(call, args.steps, args.warmup, stream, args.settle_ms)
    total_bytes = sum(nbytes[i % len(sets)] for i in range(args.steps))
    bytes_per_launch = float(np.mean([nbytes[i % len(sets)] for i in range(args.steps)]))
    rec = record(args, value=total_bytes / wall / 1e9, wall=wall, launch_avg_ms=launch_avg_ms,
                 launch_ms=launch_ms, bytes_per_launch=bytes_per_launch, rows=w.rows,
                 dtype="fp32 scores, int32 ids",
                 config={"workload": desc, "rows": w.rows, "num_regions": w.num_regions,
                         "topk": w.topk, "input_sets": len(sets), "seed": w.seed},
                 kernel="select_kernel", traffic=load_traffic(w.name, 1, "select_kernel"),
                 metric="effective GB/s (% of HBM peak) and rows/s for region selection")
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: oracle selection", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = select_cpu_baseline(sets[0], outs[0], args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def run_chain(args, dev) -> int:
    """One DSA decode step on the bf16-gated decode batch (64 requests x G 4,
    16 heads, bf16 cache of 64-token pages, positions U[4096, 32767]) at the
    pages' 8-token regions: indexer logits (8 e4m3 heads) over every region of
    each row's request, top-512 selection with the current region forced,
    then the sparse decode over the selected regions (~4K tokens per row).
    Each stage is timed alone on its own inputs, then the three back to back
    (the selection reads the logits' scores, the decode the selection's
    regions), then the three as one replayed HIP graph.  One input set: the
    stages hand their outputs on."""
    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    topk = 512
    w = gen.Workload("dsa-chain", requests=64, query_len=1, groups=4, heads=16, block=64,
                     pages_per_req=512, R=topk, kv="bf16", pos_lo=4096, pos_hi=32767,
                     inactive_frac=0.0, gated=True, splits=1, region_tokens=8,
                     seed=gen.workload_seed(31))
    lw = gen.LogitsWorkload("dsa-chain-logits", requests=w.requests, query_len=w.query_len,
                            groups=w.groups, heads=8, block=w.block,
                            pages_per_req=w.pages_per_req, pos_lo=w.pos_lo, pos_hi=w.pos_hi,
                            region_tokens=8, seed=gen.workload_seed(32))
    desc = ("dsa-chain: %d rows = %d req x G %d; logits %d e4m3 heads x 256 over %d regions "
            "of 8 tokens; top-%d selection; sparse decode %d heads x 192, bf16 cache, block %d, "
            "gated" % (w.rows, w.requests, w.groups, lw.heads, lw.num_regions, topk, w.heads,
                       w.block))
    print("[bench] drawing %s" % desc, file=sys.stderr, flush=True)
    dec = gen.make_inputs(w, device=dev, splits=1)
    li = gen.make_logits_inputs(lw, device=dev)
    S = lw.num_regions
    scores = torch.empty((w.rows, S), dtype=torch.float32, device=dev)
    cur = torch.empty(w.rows, dtype=torch.int32, device=dev)
    lens = torch.empty(w.rows, dtype=torch.int32, device=dev)
    regions = torch.empty((w.rows, topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(dec.query)
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    la = B.make_logits_args(li.query, li.weights, li.summaries, li.scales, dec.block_table,
                            dec.positions, scores, groups=w.groups, query_len=w.query_len,
                            region_tokens=8, current=cur, topk_lengths=lens)
    sa = B.make_select_args(scores, cur, topk, regions, lens)
    da = B.make_args(dec.query, dec.cache, regions, dec.block_table, dec.positions, dec.active,
                     out, scale=dec.scale, query_len=w.query_len, splits=1, gate=dec.gate,
                     region_tokens=8)

    def check(rc):
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    stages = {
        "logits": lambda i: check(B.sda_indexer_logits_raw(la, handle)),
        "selection": lambda i: check(B.sda_select_regions_raw(sa, handle)),
        "decode": lambda i: check(B.sda_decode_raw(da, handle)),
    }

    def chain(i):
        for fn in stages.values():
            fn(i)

    chain(0)  # the selection's regions feed the decode timed alone
    torch.cuda.synchronize()
    res = {}
    for name, fn in list(stages.items()) + [("chain", chain)]:
        wall, avg_ms, launch_ms = time_calls(fn, args.steps, args.warmup, stream,
                                             args.settle_ms)
        res[name] = {"us_per_call": round(wall / args.steps * 1e6, 2),
                     "hip_event_us": round(avg_ms * 1e3, 2),
                     "median_us": round(float(np.median(launch_ms)) * 1e3, 2)}
    # The same step captured once in a HIP graph and replayed (the library
    # calls allocate nothing and record no memset, so they capture as they
    # are); the replays must reproduce the eager outputs bit for bit.
    torch.cuda.synchronize()
    eager_regions, eager_out = regions.clone(), out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        check(B.sda_indexer_logits_raw(la, h))
        check(B.sda_select_regions_raw(sa, h))
        check(B.sda_decode_raw(da, h))
    wall, avg_ms, launch_ms = time_calls(lambda i: graph.replay(), args.steps, args.warmup,
                                         stream, args.settle_ms)
    torch.cuda.synchronize()
    res["chain_graph"] = {"us_per_call": round(wall / args.steps * 1e6, 2),
                          "hip_event_us": round(avg_ms * 1e3, 2),
                          "median_us": round(float(np.median(launch_ms)) * 1e3, 2),
                          "matches_eager": bool(torch.equal(regions, eager_regions) and
                                                torch.equal(out.view(torch.int16),
                                                            eager_out.view(torch.int16)))}
    del graph
    pos = dec.positions.cpu().numpy()
    sel = regions.cpu().numpy()
    dbytes, tokens = algorithmic_bytes(w, pos, sel, dec.active.cpu().numpy())
    res["decode"]["bytes_per_call"] = int(dbytes)
    res["decode"]["GB/s"] = round(dbytes / (res["decode"]["us_per_call"] * 1e-6) / 1e9, 1)
    res["decode"]["visible_tokens_per_row"] = round(tokens / w.rows, 1)
    lbytes = logits_algorithmic_bytes(lw, pos)
    res["logits"]["bytes_per_call"] = int(lbytes)
    res["logits"]["GB/s"] = round(lbytes / (res["logits"]["us_per_call"] * 1e-6) / 1e9, 1)
    chain_us = res["chain"]["us_per_call"]
    rec = {"metric": "DSA decode step (indexer logits -> top-512 selection -> sparse decode)",
           "value": round(w.rows / (chain_us * 1e-6), 1), "unit": "rows/s",
           "higher_is_better": True, "us_per_step": chain_us, "steps": args.steps,
           "warmup": args.warmup, "data": "synthetic", "stages": res,
           "config": {"workload": desc, "rows": w.rows, "seed": w.seed}}
    print(json.dumps(rec), flush=True)
    return 0


def load_traffic(workload_name: str, splits: int, kernel: str = "split_kernel"):
    """Counter-derived HBM bytes per launch from the committed profile summary,
    or None unless it was measured on the current kernel source and split count."""
    path = os.path.join(ROOT, "profiles", "%s_%s.md" % (kernel, workload_name))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        parts = line.strip().split("=")
        if len(parts) == 2:
            fields[parts[0].strip()] = parts[1].strip()
    want_hash = {"select_kernel": select_kernel_hash, "logits_kernel": logits_kernel_hash}.get(
        kernel, kernel_hash)()
    if fields.get("kernel_sha256_16") != want_hash or fields.get("splits") != str(splits):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed_passes(fn, min_seconds: float):
    """Run fn() until at least min_seconds have elapsed (at least once);
    return (passes, seconds, result of the first pass)."""
    t0 = time.perf_counter()
    first = fn()
    n = 1
    while time.perf_counter() - t0 < min_seconds:
        fn()
        n += 1
    return n, time.perf_counter() - t0, first


def cpu_baseline(inp, gpu_out, rows_sample: int, threads: int, min_seconds: float):
    """Time the fp64 oracle (as it stands) on a sample of active rows,
    repeated until min_seconds of host time have been spent."""
    from oracle import oracle
    from oracle.hostprep import host_problem_from_inputs

    act = inp.active.cpu().numpy()
    cand = np.nonzero(act)[0]
    rng = np.random.default_rng(0)
    rows = sorted(rng.choice(cand, size=min(rows_sample, len(cand)), replace=False).tolist())
    hp = host_problem_from_inputs(inp, rows=rows)
    out = np.full((inp.w.rows, inp.w.heads, 192), np.nan)
    passes, dt, _ = timed_passes(lambda: oracle.decode(hp, out=out, rows=rows, threads=threads),
                                 min_seconds)
    sub_act = np.zeros_like(act)
    sub_act[rows] = 1
    nbytes, _ = algorithmic_bytes(inp.w, inp.positions.cpu().numpy()[rows],
                                  inp.regions.cpu().numpy()[rows], sub_act[rows])
    # the output term counts every row of a call; count only the sampled ones here
    g = gpu_out.float().cpu().numpy().astype(np.float64)[rows]
    err = np.abs(g - out[rows])
    return {
        "value": passes * nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d active rows of the first input set, %d passes (fp64 C oracle, %d "
                  "threads), %.2f s wall; rows/s %.1f" % (len(rows), passes, threads, dt,
                                                         passes * len(rows) / dt),
        "parity_max_abs": float(err.max()),
        "parity_mean_abs": float(err.mean()),
    }


def host_threads() -> tuple:
    """(threads for the CPU baseline, how that count was chosen).  Every core
    this process may run on, capped by OMP_NUM_THREADS when it is set: a
    GPU host that shares its cores among GPUs states each GPU's share there."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and 0 < int(cap) < avail:
        return int(cap), "%d usable cores, OMP_NUM_THREADS=%s" % (avail, cap)
    return max(1, avail), "%d usable cores" % avail


def parse_also(args) -> list:
    """Workloads timed after the headline in the same run: by default the
    other decode workloads (2, 3, 4) when the headline is workload 5."""
    if args.also is None:
        return [2, 3, 4] if args.config == 5 else []
    return [int(x) for x in args.also.split(",") if x.strip()]


def summary_of(rec: dict) -> dict:
    """The per-workload fields of a record, for the `other_configs` key."""
    keep = ("value", "unit", "ms_per_step", "settle_calls", "pct_hbm_peak", "rows_per_s",
            "us_per_call", "dtype", "config", "roofline")
    return {k: rec[k] for k in keep if k in rec}


def measure_sparse(args, dev, k: int, with_cpu: bool) -> dict:
    """Time sda_decode on workload k: draw its cache and `args.sets` input
    sets, marshal each set's arguments once, time the calls, and free
    everything before returning the record."""
    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    w = gen.WORKLOADS[k]
    splits = args.splits or w.splits or B.sda_splits(w.rows)

    print("[bench] drawing %s" % workload_desc(w), file=sys.stderr, flush=True)
    base = gen.make_inputs(w, device=dev, splits=splits)
    sets = [base]
    bt = base.block_table.cpu().numpy()
    for i in range(1, args.sets):
        sets.append(gen.make_inputs(w, device=dev, seed=w.seed + 100003 * i, cache=base.cache,
                                    block_table=bt, splits=splits))
    nbytes = []
    for s in sets:
        b, _ = algorithmic_bytes(w, s.positions.cpu().numpy(), s.regions.cpu().numpy(),
                                 s.active.cpu().numpy())
        nbytes.append(b)
    outs = [torch.empty_like(s.query) for s in sets]
    ws_bytes = B.sda_workspace_bytes(w.rows, w.heads, splits)
    if args.no_row_order and splits == 1:
        ws_bytes = 0
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)

    # The argument block of every input set is marshalled once (the tensors
    # stay alive in `sets`/`outs`); each step is then one C call.
    prepared = []
    for s, o in zip(sets, outs):
        B.check_tensors(s.query, s.cache, s.regions, s.block_table, s.positions, s.active, o,
                        s.k_scale, s.v_scale, s.gate)
        prepared.append(B.make_args(
            s.query, s.cache, s.regions, s.block_table, s.positions, s.active, o,
            scale=s.scale, query_len=w.query_len, splits=splits, k_scale=s.k_scale,
            v_scale=s.v_scale, gate=s.gate, region_tokens=w.region_tokens,
            workspace=workspace if ws_bytes else None))

    # The library names the kernels it launches for these arguments on this
    # device (the schedule depends on the compute-unit count).
    rc, kernels = B.sda_decode_kernels_raw(prepared[0], handle)
    if rc != B.SDA_OK:
        raise B.SdaError(rc, B.status_string(rc))
    ordered = bool(kernels & B.SDA_KERNEL_ORDER)
    row_stream = bool(kernels & B.SDA_KERNEL_ROW_STREAM)

    def call(i):
        rc = B.sda_decode_raw(prepared[i % len(prepared)], handle)
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    wall, launch_avg_ms, launch_ms = time_calls(call, args.steps, args.warmup, stream, args.settle_ms)
    total_bytes = sum(nbytes[i % len(sets)] for i in range(args.steps))
    bytes_per_launch = float(np.mean([nbytes[i % len(sets)] for i in range(args.steps)]))
    rec = record(args, value=total_bytes / wall / 1e9, wall=wall, launch_avg_ms=launch_avg_ms,
                 launch_ms=launch_ms, bytes_per_launch=bytes_per_launch, rows=w.rows,
                 dtype="bf16" if w.kv == "bf16" else "fp8-e4m3 cache, bf16 MFMA",
                 config={"workload": workload_desc(w), "rows": w.rows, "heads": w.heads,
                         "splits": splits, "row_order": "heaviest first" if ordered else "index",
                         "input_sets": len(sets), "seed": w.seed},
                 kernel=("sda row-stream kernel (combine fused)" if row_stream else
                         ("sda order kernel + " if ordered else "") + "sda split kernel"
                         + (" + combine" if splits > 1 else " (combine fused)")),
                 traffic=load_traffic(w.name, splits,
                                      "row_stream_kernel" if row_stream else "split_kernel"))
    if args.flush_mib > 0:
        rec["flushed"] = time_flushed(call, args.steps, stream, args.flush_mib)
    if with_cpu:
        threads, why = host_threads()
        print("[bench] cpu baseline: oracle on %d rows, %d threads (%s)"
              % (args.cpu_rows, threads, why), file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(base, outs[0], args.cpu_rows, threads,
                                           args.cpu_seconds)
        rec["cpu_baseline"]["threads_from"] = why
    del prepared, outs, workspace, sets, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


SDA_PROBE_MAX_BLOCKS = 2048  # include/sda_probe.h


class ProbeArgs(ctypes.Structure):
    """Mirror of ``sda_probe_args`` (include/sda_probe.h)."""
    _fields_ = [("base", ctypes.c_void_p), ("kv_dtype", ctypes.c_int32),
                ("token_stride", ctypes.c_int64), ("groups", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("block_offsets", ctypes.c_void_p),
                ("group_start", ctypes.c_void_p), ("sink", ctypes.c_void_p)]


def probe_lib():
    """libsda_probe.so, the gather-ceiling probe built beside libsda.so."""
    from sparse_paged_decode_02_amd import build as sda_build
    if not os.path.exists(sda_build.PROBE_LIB):
        raise RuntimeError("libsda_probe.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(sda_build.PROBE_LIB)
    lib.sda_probe_gather.restype = ctypes.c_int
    lib.sda_probe_gather.argtypes = [ctypes.POINTER(ProbeArgs), ctypes.c_void_p]
    lib.sda_probe_args_size.restype = ctypes.c_size_t
    if lib.sda_probe_args_size() != ctypes.sizeof(ProbeArgs):
        raise RuntimeError("sda_probe_args size mismatch")
    lib.sda_probe_valu.restype = ctypes.c_int
    lib.sda_probe_valu.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    return lib


# include/sda_probe.h: kind -> (name, instructions per wave per round)
VALU_KINDS = {0: ("v_fma_f32", 64), 1: ("v_xor_b32 + v_add_u32", 128),
              2: ("v_lshrrev_b32 + v_lshl_or_b32", 128)}


def run_valu(args, dev) -> int:
    """SIMD cycles per wave64 VALU instruction of each probe kind: 8 workgroups of
    4 waves per CU (8 waves per SIMD), `iters` rounds each, timed with HIP
    events on the launch stream; cycles assume the 2.4 GHz peak clock, and the
    ratio to the FMA figure is clock-free."""
    import torch
    plib = probe_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    groups, iters = 8 * cus, 2000
    sink = torch.empty(groups * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for kind, (name, per_round) in VALU_KINDS.items():
        def call():
            rc = plib.sda_probe_valu(kind, groups, iters, ctypes.c_void_p(sink.data_ptr()), handle)
            if rc != 0:
                raise RuntimeError("sda_probe_valu returned %d" % rc)
        call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = max(1, min(args.steps, 10))
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        instr_per_simd = groups * 4 * iters * per_round / (4 * cus)
        res[name] = {"ms_per_call": round(ms, 4),
                     "simd_cycles_per_instr_at_2p4GHz": round(ms * 1e-3 * 2.4e9 / instr_per_simd, 3)}
    fma = res["v_fma_f32"]["simd_cycles_per_instr_at_2p4GHz"]
    for name in res:
        res[name]["relative_to_fma"] = round(res[name]["simd_cycles_per_instr_at_2p4GHz"] / fma, 3)
    print(json.dumps({"metric": "VALU issue cost per wave64 instruction", "cus": cus,
                      "workgroups": groups, "waves_per_simd": 8, "iters": iters,
                      "kinds": res}), flush=True)
    return 0


def probe_blocks(w, cache_strides, positions, regions, active, block_table) -> tuple:
    """Each active row's visible regions as byte offsets into the cache (the
    blocks its split workgroup reads), in slot order: (offsets, group_start).
    A region is visible iff its id >= 0 and its first token <= the row's
    position; the probe reads all of its rt token rows."""
    e = 1 if w.kv == "fp8" else 2
    cps, cgs, cts = cache_strides
    rt, G = w.rt, w.groups
    reg = regions.astype(np.int64)
    pos = positions.astype(np.int64)[:, None]
    rows = np.arange(w.rows)
    req = rows // (G * w.query_len)
    vis = (reg >= 0) & (reg * rt <= pos) & (active != 0)[:, None]
    t0 = np.where(vis, reg * rt, 0)
    page = block_table.astype(np.int64)[req[:, None], t0 // w.block]
    off = (page * cps + (rows % G)[:, None] * cgs + (t0 % w.block) * cts) * e
    offsets = off[vis]  # row-major: each row's visible slots in slot order
    start = np.zeros(w.rows + 1, dtype=np.int32)
    start[1:] = np.cumsum(vis.sum(axis=1))
    return offsets.astype(np.int64), start


def run_gather(args, dev) -> int:
    """The split kernel against the gather ceiling of its own access pattern:
    the probe reads the same region blocks (every visible region of every
    active row, all rt token rows) through the same chunk loop and launch
    shape, with no attention math.  Both are timed on the same rotating input
    sets in one run; ``kernel_frac_of_ceiling`` is the probe's time over the
    kernel's."""
    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    w = gen.WORKLOADS[args.gather_ceiling]
    splits = w.splits or B.sda_splits(w.rows)
    plib = probe_lib()
    print("[bench] drawing %s" % workload_desc(w), file=sys.stderr, flush=True)
    base = gen.make_inputs(w, device=dev, splits=splits)
    bt = base.block_table.cpu().numpy()
    sets = [base] + [gen.make_inputs(w, device=dev, seed=w.seed + 100003 * i, cache=base.cache,
                                     block_table=bt, splits=splits) for i in range(1, args.sets)]
    e = 1 if w.kv == "fp8" else 2
    row_bytes = 384 * e
    cstr = tuple(int(x) for x in base.cache.stride()[:3])
    stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    keep, probe_args, kernel_args, pbytes, kbytes = [], [], [], [], []
    ws = torch.empty(B.sda_workspace_bytes(w.rows, w.heads, splits), dtype=torch.uint8,
                     device=dev)
    sink = torch.zeros(max(w.rows, args.balanced_groups) * 4, dtype=torch.int32, device=dev)
    block_bytes = w.rt * cstr[2] * e
    for s in sets:
        pos, reg, act = (s.positions.cpu().numpy(), s.regions.cpu().numpy(),
                         s.active.cpu().numpy())
        offs, start = probe_blocks(w, cstr, pos, reg, act, bt)
        groups = w.rows
        if args.balanced_groups:
            # the same blocks dealt in equal contiguous shares to N groups:
            # the balanced decomposition's ceiling (no idle CU, no tail)
            groups = args.balanced_groups
            start = np.round(np.linspace(0, len(offs), groups + 1)).astype(np.int32)
            assert int(np.diff(start).max()) <= SDA_PROBE_MAX_BLOCKS
        if args.sequential:
            offs = np.arange(len(offs), dtype=np.int64) * block_bytes
            assert len(offs) * block_bytes <= base.cache.numel() * e
        t_off = torch.from_numpy(offs).to(dev)
        t_start = torch.from_numpy(start).to(dev)
        a = ProbeArgs()
        a.base = base.cache.data_ptr()
        a.kv_dtype = B.SDA_KV_FP8_E4M3 if w.kv == "fp8" else B.SDA_KV_BF16
        a.token_stride = cstr[2] * e
        a.groups, a.block_tokens = groups, w.rt
        a.block_offsets, a.group_start, a.sink = t_off.data_ptr(), t_start.data_ptr(), \
            sink.data_ptr()
        probe_args.append(a)
        pbytes.append(len(offs) * w.rt * row_bytes)
        o = torch.empty_like(s.query)
        keep += [t_off, t_start, o]
        kernel_args.append(B.make_args(
            s.query, s.cache, s.regions, s.block_table, s.positions, s.active, o,
            scale=s.scale, query_len=w.query_len, splits=splits, k_scale=s.k_scale,
            v_scale=s.v_scale, gate=s.gate, region_tokens=w.region_tokens, workspace=ws))
        kbytes.append(algorithmic_bytes(w, pos, reg, act)[0])

    def probe_call(i):
        rc = plib.sda_probe_gather(ctypes.byref(probe_args[i % len(probe_args)]), handle)
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    def kernel_call(i):
        rc = B.sda_decode_raw(kernel_args[i % len(kernel_args)], handle)
        if rc != B.SDA_OK:
            raise B.SdaError(rc, B.status_string(rc))

    res = {}
    for name, fn, nb in (("probe", probe_call, pbytes), ("kernel", kernel_call, kbytes)):
        _, avg_ms, launch_ms = time_calls(fn, args.steps, args.warmup, stream, args.settle_ms)
        mean_bytes = float(np.mean([nb[i % len(nb)] for i in range(args.steps)]))
        gbs = mean_bytes / (avg_ms * 1e-3) / 1e9
        res[name] = {"avg_launch_us": round(avg_ms * 1e3, 3),
                     "median_us": round(float(np.median(launch_ms)) * 1e3, 2),
                     "bytes_per_call": int(mean_bytes), "GB/s": round(gbs, 1),
                     "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    res["probe"]["bytes"] = ("every visible region's %d token rows of %d bytes%s"
                             % (w.rt, row_bytes, ", consecutive blocks" if args.sequential
                                else ""))
    res["kernel"]["bytes"] = "algorithmic (visible K|V rows, Q of active rows, output)"
    kernel_alg_at_probe_time = np.mean(kbytes) / (res["probe"]["avg_launch_us"] * 1e-6) / 1e9
    rec = {"metric": "gather ceiling of the sparse decode access pattern",
           "workload": workload_desc(w), "splits": splits,
           "pattern": ("sequential blocks" if args.sequential else "the workload's blocks")
           + (", dealt evenly to %d groups" % args.balanced_groups if args.balanced_groups
              else ", one group per row"),
           "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
           "input_sets": len(sets), "seed": w.seed, "probe": res["probe"],
           "kernel": res["kernel"],
           "ceiling_for_kernel_metric_GBps": round(float(kernel_alg_at_probe_time), 1),
           "kernel_frac_of_ceiling": round(res["probe"]["avg_launch_us"]
                                           / res["kernel"]["avg_launch_us"], 4),
           "kernel_sha256_16": kernel_hash()}
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="headline workload: 1..5, or 6 / 7 = the bf16-gated / FP8-cache "
                         "shape at 8-token regions (default 5, the largest)")
    ap.add_argument("--also", default=None, metavar="LIST",
                    help="comma-separated workloads timed after the headline in the same "
                         "run, reported under `other_configs` (default: 2,3,4 when the "
                         "headline is 5; '' for none)")
    ap.add_argument("--swa", default="", metavar="NAME",
                    help="measure the gated sliding-window decode on workload NAME "
                         "(swa-gated, swa-mtp) instead")
    ap.add_argument("--select", default="", metavar="NAME",
                    help="measure region selection on workload NAME (select-decode, "
                         "select-large) instead")
    ap.add_argument("--logits", default="", metavar="NAME",
                    help="measure the decode indexer logits on workload NAME (logits-decode, "
                         "logits-mtp) instead")
    ap.add_argument("--chain", action="store_true",
                    help="time one DSA decode step (indexer logits -> top-512 selection -> "
                         "sparse decode at 8-token regions), each stage alone and the three "
                         "back to back")
    ap.add_argument("--gather-ceiling", type=int, default=0, metavar="K",
                    help="time the gather probe on workload K's region blocks beside the "
                         "split kernel on the same inputs (one JSON line)")
    ap.add_argument("--sequential", action="store_true",
                    help="with --gather-ceiling: consecutive blocks instead of the "
                         "workload's")
    ap.add_argument("--balanced-groups", type=int, default=0, metavar="N",
                    help="--gather-ceiling: deal all blocks evenly to N workgroups instead "
                         "of one per row")
    ap.add_argument("--valu-rate", action="store_true",
                    help="time the VALU issue-rate probe (SIMD cycles per wave64 instruction "
                         "of a few kinds; one JSON line)")
    ap.add_argument("--pack", type=int, default=0,
                    help="with --swa: query tokens per workgroup (0: the library's plan)")
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed back-to-back calls before the warmup steps, until this many "
                         "ms have passed (0: none)")
    ap.add_argument("--splits", type=int, default=0, help="0: the workload's rule")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="sparse decode: also time each call after writing MIB MiB (a "
                         "last-level-cache flush), reported as `flushed`")
    ap.add_argument("--no-row-order", action="store_true",
                    help="sparse decode with splits == 1: pass no workspace, so rows start "
                         "in index order instead of heaviest first")
    ap.add_argument("--cpu-rows", type=int, default=48)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU-baseline sample until this much host time is spent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (rows "
              "are independent and would shard across GPUs with no exchange). Run with "
              "--gpus 1.", file=sys.stderr)
        return 2

    import torch
    from sparse_paged_decode_02_amd import binding as B
    from sparse_paged_decode_02_amd import inputs as gen

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale between counter readings and bytes moved.
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "calls": args.steps}), flush=True)
        return 0
    if args.gather_ceiling:
        return run_gather(args, dev)
    if args.valu_rate:
        return run_valu(args, dev)
    if args.swa:
        return run_swa(args, dev)
    if args.select:
        return run_select(args, dev)
    if args.logits:
        return run_logits(args, dev)
    if args.chain:
        return run_chain(args, dev)
    headline = measure_sparse(args, dev, args.config, with_cpu=not args.no_cpu_baseline)
    others = parse_also(args)
    if others:
        # The other decode workloads of the same run, one after another (each
        # draws its own cache; the previous one is freed first).
        headline["other_configs"] = {}
        for k in others:
            rec = measure_sparse(args, dev, k, with_cpu=False)
            headline["other_configs"][gen.WORKLOADS[k].name] = summary_of(rec)
    print(json.dumps(headline), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
