#!/usr/bin/env python3
"""Benchmark of sparse top-k MLA attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                    [--no-secondary] [--copy-calibration BYTES] [--pack] [--crossover]

A step is one call of the library on one batch of seeded synthetic input that is
already resident in HBM. The default workload is the large compute-bound prefill:
T=8192 tokens, h=128 heads, topk=2048, fp8 KV with per-64 scales, d_qk=576, d_v=512,
context 65536.

The script prints one JSON line with:
  - the whole-job throughput in algorithmic TFLOP/s, 2*h*(d_qk + d_v) per valid
    (token, index);
  - a roofline object for the attention kernel: its average launch duration is the timed
    region's time per step, from HIP events on the launch stream;
  - the CPU oracle timed on a bounded sample of the same workload;
  - a decode object: 32 sequences of one token (h=64, topk=512), time per step over a
    graph of back-to-back steps, cold graph replays, and its HBM roofline on gathered bytes;
  - secondary lines: the tp2-shard prefill and the dual-cache window (warm and cold), the
    large prefill cold, the fp8 compute mode on the tp2 shard, and the packing kernel
    (bf16 rows into the fp8 pool, HBM GB/s).
    Cold: a 1 GiB fill evicts L2 and the MALL before each timed launch (outside the timed
    region).
--pack times only the packing kernel; --crossover measures the decode form against the
prefill form per configuration and token count (cold, graph replay); --trace-set launches one
workload cold for a rocprofv3 kernel trace, and --summarize-trace reads such a trace back.
Only one GPU is supported. With --gpus above 1 it exits with a message.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "sparse-MLA prefill TFLOP/s + decode µs/step & KV GB/s, fraction of roofline"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA (5.0 PFLOP/s)


def mixed_peak(d_qk, d_v):
    """Peak of the fp8 compute mode: QK (2 d_qk flop per pair) on fp8 MFMA, PV (2 d_v) on
    bf16 MFMA, each at its own dense peak."""
    return (d_qk + d_v) / (d_qk / PEAK_FP8_TFLOPS + d_v / PEAK_BF16_TFLOPS)


def algorithmic(p):
    """(flops, gathered KV bytes, valid entries) the method must do for this input."""
    def valid_mask(pool, idx):
        return (idx >= 0) & (idx.astype(np.int64) < pool.num_slots)

    nv = int(valid_mask(p.kv, p.indices).sum())
    row = {"fp8": p.d_qk + 4 * (p.d_qk // 64), "bf16": 2 * p.d_qk}
    byts = nv * row[p.kv.dtype]
    if p.extra is not None:
        ne = int(valid_mask(p.extra, p.extra_indices).sum())
        byts += ne * row[p.extra.dtype]
        nv += ne
    return 2.0 * p.h * (p.d_qk + p.d_v) * nv, float(byts), nv


def time_calls(fn, iters, warmup, flush=None):
    """Mean and median ms per call of fn, with HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(iters):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return float(np.mean(times)), float(np.median(times))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, budget_s=20.0):
    """Time the oracle on a bounded sample of tokens on the host cores.

    Workers: the cores this process may run on, at most 16 (the host's CPU share per GPU on
    a shared machine, whatever os.cpu_count() reports); both counts and the CPU model are
    reported."""
    from oracle import sparse_mla_reference, sparse_mla_reference_parallel
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = max(1, min(int(cores or 1), 16))
    # probe the per-token cost on 2 tokens, then size the sample to the budget
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        t0 = time.perf_counter()
        sparse_mla_reference(p, np.arange(2))
        per_tok = (time.perf_counter() - t0) / 2
    n = int(max(cores, min(p.T, budget_s * cores / max(per_tok, 1e-6))))
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(p.T, size=min(n, p.T), replace=False))
    t0 = time.perf_counter()
    _, _, used = sparse_mla_reference_parallel(p, toks, workers=cores)
    dt = time.perf_counter() - t0
    frac = len(toks) / p.T
    flops, _, _ = algorithmic(p)
    return {"value": flops * frac / dt / 1e12, "unit": "TFLOP/s", "cores": used,
            "kind": "oracle",
            "sample": f"{len(toks)} of {p.T} query tokens (seeded), fp64 NumPy, {dt:.1f} s",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def traffic_record(kernel_srcs, workload):
    """HBM bytes per launch from the committed counter summary, or None.

    The summary under profiles/ carries the FETCH_SIZE and WRITE_SIZE sums (scaled by a
    plain copy of known size) and the sha256 of the kernel source and of the host code that
    sets the launch shape, taken together; a change to either makes the figure stale, and
    then no figure is reported.
    """
    import glob
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for src in kernel_srcs:
        h.update(open(src, "rb").read())
    sha = h.hexdigest()
    for path in glob.glob(os.path.join(here, "profiles", "traffic_*.md")):
        for line in open(path):
            if "traffic-record" not in line:
                continue
            rec = json.loads(line.split("traffic-record", 1)[1].rsplit("-->", 1)[0])
            if rec["workload"] == workload and rec.get("src_sha256") == sha:
                return float(rec["fetch_bytes"] + rec["write_bytes"])
    return None


def time_graph(call, iters, warmup, flush=None):
    """Mean and median ms per replay of call captured once in a HIP graph.

    The library enqueues only kernels (no allocation, no synchronisation, no memset), so a
    call with preallocated outputs and workspace can be captured; replay removes the host
    cost of argument marshalling and launches, which dominates a call of a few µs.
    """
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return time_calls(g.replay, iters, warmup, flush)


def make_call(name, decode=False, compute_mode=0):
    """(problem, device tensors, seconds to generate, call) for one workload: call() enqueues
    one step of the library on the current stream with preallocated outputs (and workspace)."""
    import torch
    import sparse_top_mla_prefill_amd as smla
    from workloads import WORKLOADS
    from workloads.device import to_device
    t0 = time.perf_counter()
    p = WORKLOADS[name]()
    d = to_device(p)
    gen_s = time.perf_counter() - t0
    out = d.new_out()
    if decode:
        nbytes = smla.sparse_mla_workspace_size(d.q, d.kv, d.indices, d.sm_scale, out, True,
                                                **d.kwargs())
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        call = lambda: smla.sparse_mla_decode(d.q, d.kv, d.indices, d.sm_scale,  # noqa: E731
                                              out=out, workspace=ws, **d.kwargs())
    else:
        call = lambda: smla.sparse_mla_prefill(d.q, d.kv, d.indices, d.sm_scale,  # noqa: E731
                                               out=out, compute_mode=compute_mode,
                                               **d.kwargs())
    return p, d, gen_s, call


def flusher():
    """A call that evicts L2 and the 256 MB MALL: a fill of a 1 GiB buffer."""
    import torch
    junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    return lambda: junk.fill_(1)


def bench_workload(name, steps, warmup, decode=False, cold=False, graph=False, compute_mode=0):
    p, d, gen_s, call = make_call(name, decode, compute_mode)
    flush = flusher() if cold else None
    if graph:
        mean_ms, med_ms = time_graph(call, steps, warmup, flush)
    else:
        mean_ms, med_ms = time_calls(call, steps, warmup, flush)
    flops, kv_bytes, nv = algorithmic(p)
    return p, d, {"workload": p.name, "decode": decode, "cold": cold, "graph": graph,
                  "compute": "fp8" if compute_mode else "bf16",
                  "ms_mean": mean_ms,
                  "ms_median": med_ms, "tflops": flops / (mean_ms * 1e-3) / 1e12,
                  "kv_GBs": kv_bytes / (mean_ms * 1e-3) / 1e9, "valid_entries": nv,
                  "gen_s": round(gen_s, 1)}, call


def graph_steps_ms(call, steps, warmup=2):
    """ms per step of `steps` calls captured back to back in one HIP graph and replayed once
    between HIP events on the current stream (the stream the graph's kernels run on): the
    kernels' own time plus the gaps between them, without the host's cost per call."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(warmup, 1)):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / steps


def decode_object(steps):
    """The decode workload (32 sequences x 1 token, h=64, topk=512, fp8): warm time per step
    over a graph of `steps` back-to-back calls, cold graph replays (L2 and MALL evicted
    before each), and its HBM roofline on the gathered KV bytes."""
    p, d, gen_s, call = make_call("decode_fp8", decode=True)
    ms = graph_steps_ms(call, steps)
    cold_mean, cold_med = time_graph(call, 20, 3, flusher())
    flops, kv_bytes, nv = algorithmic(p)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    return {"workload": p.name, "T": p.T, "h": p.h, "topk": p.topk, "kv_dtype": p.kv.dtype,
            "us_per_step": ms * 1e3,
            "timing": f"HIP events around one replay of a graph of {steps} back-to-back "
                      "steps on the launch stream (warm)",
            "cold_graph_us_median": cold_med * 1e3,
            "kv_bytes_per_step": kv_bytes, "tflops": flops / (ms * 1e-3) / 1e12,
            "tokens_per_s": p.T / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS}}


# Cold kernel traces: each workload launched reps x per times with the 1 GiB fill before
# every launch, after 3 warm launches; read back by --summarize-trace.
TRACE_SHAPES = {"prefill_large": (5, 5), "prefill_tp2": (5, 100), "dual_window": (5, 100),
                "decode_fp8": (5, 100), "tiny_bf16": (5, 100)}
TRACE_WARM = 3


def trace_set(name, compute_mode=0):
    import torch
    decode = name.startswith("decode")
    reps, per = TRACE_SHAPES[name]
    p, d, _, call = make_call(name, decode, compute_mode)
    flush = flusher()
    for _ in range(TRACE_WARM):
        call()
    torch.cuda.synchronize()
    for _ in range(reps):
        for _ in range(per):
            flush()
            call()
        torch.cuda.synchronize()
    print(json.dumps({"trace_set": name, "compute": "fp8" if compute_mode else "bf16",
                      "warm": TRACE_WARM, "reps": reps, "per": per}), flush=True)


def summarize_trace(db, name, skip, reps):
    """Per-kernel durations from a rocprofv3 database (its `kernels` view), the fills that
    evict the caches left out: the first `skip` dispatches of each kernel are dropped, the
    rest cut into `reps` runs; prints the median over all, the spread of the runs' medians,
    the mean, and the roofline fraction of the workload's algorithmic work per step."""
    import sqlite3
    from workloads import WORKLOADS
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration, grid_x, workgroup_x, vgpr_count, "
                       "accum_vgpr_count, sgpr_count, lds_size, scratch_size from kernels "
                       "order by start").fetchall()
    per_kernel = {}
    for r in rows:
        if "Fill" in r[0] or "fill" in r[0]:
            continue
        per_kernel.setdefault(r[0], []).append(r)
    p = WORKLOADS[name]()
    flops, kv_bytes, nv = algorithmic(p)
    decode = name.startswith("decode")
    print(f"workload {p.name}: {nv} valid (token, index) pairs, {flops:.4e} flop, "
          f"{kv_bytes:.4e} gathered KV bytes per step")
    step_ms = 0.0
    for kname, rs in per_kernel.items():
        d = np.array([r[1] for r in rs[skip:]], dtype=np.float64) / 1e6  # ms
        if d.size == 0:
            continue
        runs = [np.median(c) for c in np.array_split(d, max(1, min(reps, d.size)))]
        med = float(np.median(d))
        step_ms += med
        r0 = rs[0]
        print(f"- `{kname}`")
        print(f"  dispatches {len(rs)} (first {skip} dropped), {r0[2] // max(r0[3], 1)} "
              f"workgroups of {r0[3]} threads, "
              f"VGPR {r0[4]} AGPR {r0[5]} SGPR {r0[6]}, LDS {r0[7]} B, scratch {r0[8]} B")
        print(f"  median {med * 1e3:.2f} us, runs' medians {min(runs) * 1e3:.2f}-"
              f"{max(runs) * 1e3:.2f} us, mean {d.mean() * 1e3:.2f} us, min "
              f"{d.min() * 1e3:.2f} us, max {d.max() * 1e3:.2f} us")
    if decode:
        gbs = kv_bytes / (step_ms * 1e-3) / 1e9
        print(f"step (sum of the kernels' medians) {step_ms * 1e3:.2f} us: {gbs:.1f} GB/s of "
              f"gathered KV = {gbs / PEAK_HBM_GBS:.4f} of the {PEAK_HBM_GBS:.0f} GB/s HBM peak")
    else:
        tf = flops / (step_ms * 1e-3) / 1e12
        print(f"step (sum of the kernels' medians) {step_ms:.4f} ms: {tf:.1f} TFLOP/s = "
              f"{tf / PEAK_BF16_TFLOPS:.4f} of the {PEAK_BF16_TFLOPS} TFLOP/s bf16 MFMA peak")


CROSSOVER_TOKENS = (1, 2, 4, 8, 16, 24, 32, 48, 64)
CROSSOVER_CONFIGS = (
    # d_qk, kv dtype, extra dtype, h, topk, topk_extra
    *[(576, "fp8", None, h, k, 0) for h in (16, 32, 64, 128) for k in (128, 512, 2048)],
    (576, "bf16", None, 64, 512, 0),
    (1088, "fp8", "bf16", 64, 512, 128),
    (1088, "fp8", None, 128, 1024, 0),
)


PACK_ROWS = 32 * 18432  # every slot of the decode workload's pool


def bench_pack(steps=20, warmup=3, n=PACK_ROWS, d_qk=576):
    """The packing kernel on n bf16 rows (N(0,1), seeded device generator) into an fp8
    inline pool of n slots, written in a random slot order. Algorithmic bytes per row: the
    bf16 row and its slot id read, the e4m3 payload and the fp32 scales written."""
    import torch
    import sparse_top_mla_prefill_amd as smla
    from workloads import synth as S
    from workloads.device import pool_to_device
    pool = S.pack_pool(np.zeros((n, d_qk), np.uint8), np.ones((n, d_qk // 64), np.float32),
                       "fp8", d_qk)
    dev = pool_to_device(pool, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(2200)
    rows = torch.randn(n, d_qk, device="cuda", generator=g).to(torch.bfloat16)
    slots = torch.randperm(n, device="cuda", generator=g).to(torch.int32)
    call = lambda: smla.sparse_mla_pack_kv(rows, slots, dev)  # noqa: E731
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # steps launches back to back between two events on the launch stream: the mean is the
    # kernel's own time (a single eager call would add the host's argument marshalling)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / steps
    row_bytes = 2 * d_qk + 4 + d_qk + 4 * (d_qk // 64)
    gbs = n * row_bytes / (ms * 1e-3) / 1e9
    return {"workload": f"pack_kv_fp8_n{n}_d{d_qk}", "rows": n, "bytes_per_row": row_bytes,
            "ms_per_launch": ms, "GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}


def split_chunks(ws_bytes, T, h, d_v):
    """Index chunks per token of a decode-form plan, from its workspace size."""
    if ws_bytes == 0:
        return 1
    for nc in range(2, 257):
        rows = T * nc * h
        if -(-rows * d_v * 2 // 256) * 256 + rows * 8 == ws_bytes:
            return nc
    return -1


def crossover(iters=10, warmup=2):
    """Decode form against prefill form, per (geometry, h, topk, pool dtypes) and T.

    Each call runs cold (a 1 GiB fill evicts L2 and the MALL before it) and is replayed
    from a HIP graph. Indices are distinct random slots of a 65536-slot pool. The decode
    form counts as faster at T when it takes at most 0.95 of the prefill form's time;
    decode_max_tokens is the largest probed T where it does. One JSON line per config.
    """
    import torch
    import sparse_top_mla_prefill_amd as smla
    from workloads import synth as S
    from workloads.device import pool_to_device
    junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush = lambda: junk.fill_(1)  # noqa: E731
    rng = np.random.default_rng(2024)
    pools = {}

    def pool(d_qk, dt, pages):
        key = (d_qk, dt, pages)
        if key not in pools:
            pools[key] = pool_to_device(S.draw_pool(rng, dt, d_qk, pages), "cuda")
        return pools[key]

    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for d_qk, kvd, exd, h, topk, tke in CROSSOVER_CONFIGS:
        d_v = S.GEOMETRIES[d_qk]
        kv = pool(d_qk, kvd, 1024)
        ex = pool(d_qk, exd, 32) if exd else None
        sink = torch.randn(h, device="cuda", generator=gen)
        rows = []
        for T in CROSSOVER_TOKENS:
            q = torch.randn(T, h, d_qk, device="cuda", generator=gen).to(torch.bfloat16)
            idx = torch.rand(T, kv.num_pages * 64, device="cuda", generator=gen).argsort(
                dim=1)[:, :topk].to(torch.int32).contiguous()
            kw = dict(attn_sink=sink)
            if ex is not None:
                kw.update(extra=ex, extra_indices=torch.rand(
                    T, ex.num_pages * 64, device="cuda", generator=gen).argsort(
                    dim=1)[:, :tke].to(torch.int32).contiguous())
            out = torch.empty(T, h, d_v, dtype=torch.bfloat16, device="cuda")
            scale = 1.0 / math.sqrt(d_qk)
            nb = smla.sparse_mla_workspace_size(q, kv, idx, scale, out, True, **kw)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
            dec = lambda: smla.sparse_mla_decode(q, kv, idx, scale, out=out,  # noqa: E731
                                                 workspace=ws, **kw)
            pre = lambda: smla.sparse_mla_prefill(q, kv, idx, scale, out=out, **kw)  # noqa
            t_dec = time_graph(dec, iters, warmup, flush)[1]
            t_pre = time_graph(pre, iters, warmup, flush)[1]
            rows.append((T, t_dec, t_pre, split_chunks(nb, T, h, d_v)))
        wins = [r[0] for r in rows if r[1] <= 0.95 * r[2]]
        res = {"d_qk": d_qk, "kv": kvd, "extra": exd, "h": h, "topk": topk, "topk_extra": tke,
               "T": [r[0] for r in rows], "decode_us": [round(r[1] * 1e3, 1) for r in rows],
               "prefill_us": [round(r[2] * 1e3, 1) for r in rows],
               "decode_chunks": [r[3] for r in rows],
               "decode_max_tokens": max(wins) if wins else 0}
        print(json.dumps({"crossover": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_large")
    ap.add_argument("--compute", choices=["bf16", "fp8"], default="bf16",
                    help="compute mode of the main workload's calls (fp8: q in e4m3, QK on "
                         "fp8 MFMA; prefill workloads only)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES per step (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--pack", action="store_true",
                    help="only time the packing kernel (bf16 rows -> fp8 pool) and exit")
    ap.add_argument("--crossover", action="store_true",
                    help="only measure the decode form against the prefill form per config "
                         "and T (cold, graph replay), print one JSON line per config, and exit")
    ap.add_argument("--trace-set", metavar="WORKLOAD",
                    help="only launch WORKLOAD cold (the 1 GiB fill before each launch), "
                         "reps x per times after 3 warm launches, for a rocprofv3 kernel trace")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="summarise a rocprofv3 database of --workload's launches (no GPU)")
    ap.add_argument("--skip", type=int, default=TRACE_WARM,
                    help="dispatches per kernel dropped at the start by --summarize-trace")
    ap.add_argument("--reps", type=int, default=5,
                    help="runs the dispatches are cut into by --summarize-trace")
    args = ap.parse_args()
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.skip, args.reps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs a single device and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": args.steps}), flush=True)
        return

    if args.crossover:
        crossover()
        return
    if args.pack:
        print(json.dumps({"pack": bench_pack(args.steps, args.warmup)}), flush=True)
        return
    if args.trace_set:
        trace_set(args.trace_set, 1 if args.compute == "fp8" else 0)
        return

    decode = args.workload.startswith("decode")
    print(f"[bench] workload {args.workload} steps {args.steps} warmup {args.warmup}",
          file=sys.stderr, flush=True)
    p, d, gen_s, call = make_call(args.workload, decode, int(args.compute == "fp8"))
    # The timed region: exactly K steps between synchronisations, back to back on the
    # launch stream (torch's current stream, which the binding launches on).
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        call()
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    flops, kv_bytes, _ = algorithmic(p)
    value = flops / (ms_step * 1e-3) / 1e12
    print(f"[bench] {ms_step:.3f} ms/step, {value:.1f} TFLOP/s (wall {wall_ms:.1f} ms)",
          file=sys.stderr, flush=True)

    # Roofline of the dominant kernel. A prefill step is one launch of the attention kernel,
    # so its average launch duration is the timed region's time per step (HIP events on the
    # launch stream). A decode step may be two kernels (attention, then the split-K merge);
    # its line is then bound by HBM on the gathered KV bytes over the whole step.
    if decode:
        roof = {"bound": "hbm", "achieved": kv_bytes / (ms_step * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": value,
                "peak": (mixed_peak(p.d_qk, p.d_v) if args.compute == "fp8"
                         else PEAK_BF16_TFLOPS), "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    import sparse_top_mla_prefill_amd as smla_pkg
    # the stored counter record belongs to the bf16-mode kernel of the large prefill (the
    # role-split kernel: its source, the helpers it includes, and the host code that sets
    # its launch)
    csrc = os.path.join(os.path.dirname(smla_pkg.__file__), "csrc")
    roof["traffic"] = None if args.compute == "fp8" else traffic_record(
        [os.path.join(csrc, f) for f in ("roles.hip", "walk.h", "dkern.h", "smla_internal.h",
                                         "api.cpp")], p.name)
    roof["kernel_ms"] = ms_step
    del d, call
    torch.cuda.empty_cache()

    dec = None
    if not decode and not args.no_secondary:
        dec = decode_object(args.steps)
        print(f"[bench] decode {json.dumps(dec)}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    secondary = []
    if not args.no_secondary:
        for name, dec_, cold, graph, cm in [("prefill_tp2", False, False, False, 0),
                                            ("prefill_tp2", False, True, False, 0),
                                            ("dual_window", False, False, False, 0),
                                            ("dual_window", False, True, False, 0),
                                            ("prefill_large", False, True, False, 0),
                                            ("prefill_tp2", False, False, False, 1)]:
            if name == args.workload and dec_ == decode and cm == 0 and not cold:
                continue
            _, _, res, _ = bench_workload(name, 20 if not cold else 10, 3, decode=dec_,
                                          cold=cold, graph=graph, compute_mode=cm)
            if dec_:
                res["hbm_frac_on_kv"] = res["kv_GBs"] / PEAK_HBM_GBS
            elif cm:
                res["mfma_frac"] = res["tflops"] / mixed_peak(576, 512)
            else:
                res["mfma_frac"] = res["tflops"] / PEAK_BF16_TFLOPS
            secondary.append(res)
            print(f"[bench] secondary {json.dumps(res)}", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        res = bench_pack()
        secondary.append(res)
        print(f"[bench] secondary {json.dumps(res)}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(p)

    line = {
        "metric": METRIC,
        "value": (kv_bytes / (ms_step * 1e-3) / 1e9) if decode else value,
        "unit": "GB/s" if decode else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16" if args.compute == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "T": p.T, "h": p.h, "topk": p.topk,
                   "topk_extra": p.topk_extra, "d_qk": p.d_qk, "d_v": p.d_v,
                   "kv_dtype": p.kv.dtype, "tokens_per_s": p.T / (ms_step * 1e-3)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": dec,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
