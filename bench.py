#!/usr/bin/env python3
"""Throughput of exact tiled attention, forward + backward, on one MI355X.

One step = the whole hot path over one batch: fa_fwd, fa_bwd_preprocess,
fa_bwd_dkdv, fa_bwd_dq (C ABI of libfa.so) on inputs already resident in HBM.
Default workload: batch*heads = 32, N = 8192, d = 128, bf16, causal.

Counted FLOPs per head (the metric's convention): forward 4 N^2 d, backward
10 N^2 d, both halved when causal.  With --window W (causal sliding window)
N^2 / 2 becomes the exact count of visible (query, key) pairs,
N W - W (W - 1) / 2.  Prints one JSON line (rank 0).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 (256 CU x 2.4 GHz x 4096 flop/clk)
MFMA_FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
METRIC = "fwd+bwd attention TFLOPS (bf16, causal, N=8192, d=128) + % of MFMA peak"


def score_pairs(n, causal, window=0):
    """(query, key) pairs whose scores the method needs, per head: N^2, N^2 / 2
    when causal (the metric's convention), and with a causal window of W < N
    keys the exact band count N W - W (W - 1) / 2."""
    if causal and 0 < window < n:
        return n * window - window * (window - 1) / 2
    return n * n * (0.5 if causal else 1.0)


def counted_flops(bh, n, d, causal, window=0):
    pairs = score_pairs(n, causal, window)
    fwd = 4.0 * pairs * d * bh
    bwd = 10.0 * pairs * d * bh
    return fwd, bwd


def kernel_flops(bh, n, d, causal, window=0):
    """Algorithmic MFMA flops per launch of each kernel (the contractions it
    must perform over the needed score pairs): fwd S and PV (4 N^2 d); dK/dV
    kernel S, dP, dV, dK (8 N^2 d); dQ kernel S, dP, dQ (6 N^2 d)."""
    u = 2.0 * score_pairs(n, causal, window) * d * bh
    # the single-kernel backward runs S, dP, dV, dK and dQ once each
    return {"fwd": 2 * u, "dkdv": 4 * u, "dq": 3 * u, "bwd_fused": 5 * u}


def kernel_bytes(bh, n, d, elt):
    """Algorithmic HBM bytes per launch (each input read once, each output
    written once)."""
    t = bh * n * d * elt
    r = bh * n * 4
    # the single-kernel backward also clears, accumulates and rounds an fp32 dQ
    return {"fwd": 4 * t + r, "preprocess": 2 * t + r, "dkdv": 6 * t + 2 * r, "dq": 5 * t + 2 * r,
            "bwd_fused": 8 * t + 2 * r + 3 * bh * n * d * 4}


TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "attention_kernels_headline_8192_d128_causal_bf16.md")
KERNEL_SOURCES = {
    "fwd": ("fa_fwd_bf16.hip", "fa_common.h"),
    "dkdv": ("fa_bwd_bf16.hip", "fa_common.h"),
    "dq": ("fa_bwd_bf16.hip", "fa_common.h"),
    "preprocess": ("fa_f32.hip",),
}


def strip_comments(src: str) -> str:
    """C++ source without comments and blank lines (string literals in these
    kernels hold no comment markers)."""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def source_hash(kernel):
    """SHA-1 (12 hex digits) of the kernel's source files with comments
    removed, so that editing a comment keeps the recorded counters valid."""
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_tiled_attention_26_amd", "csrc", f)) as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:12]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (headline workload, default tilings), or None when the kernel's sources
    have changed since the counters were taken."""
    try:
        with open(TRAFFIC_TABLE) as fh:
            for line in fh:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                if len(cells) >= 5 and cells[0] == kernel and cells[1] == source_hash(kernel):
                    return int(cells[4])
    except OSError:
        pass
    return None


def cpu_baseline(bh, n, d, causal, budget_s=25.0, window=0):
    """The fp64 oracle timed on host cores on a bounded sample of the same
    workload: whole heads (forward + backward) until about `budget_s`."""
    import numpy as np

    import oracle
    from workloads import cast_io, make_inputs, to_f64

    cores = len(os.sched_getaffinity(0))
    rng_inputs = make_inputs(1, n, d, seed=0)
    q, k, v, do = (to_f64(t)[0] for t in cast_io(rng_inputs, "bf16"))
    heads = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention_forward(q, k, v, causal=causal, window=window)
        oracle.attention_backward(q, k, v, do, causal=causal, window=window)
        heads += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / heads * (heads + 1) > budget_s * 1.5:
            break
    fwd, bwd = counted_flops(heads, n, d, causal, window)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:
        pass
    return {
        "value": (fwd + bwd) / el / 1e12,
        "unit": "TFLOPS",
        "cores": threads or cores,
        "kind": "oracle",
        "sample": f"{heads} of {bh} heads (N={n}, d={d}, {'causal' if causal else 'non-causal'}"
                  f"{f', window {window}' if window else ''}), "
                  f"fp64 fwd+bwd, {el:.1f} s; host cores available: {cores}",
        "seconds": el,
    }


def rocprof_summary(paths):
    """Print a short text summary of rocprofv3 result databases (rocpd
    SQLite): per-kernel dispatch count and duration statistics from a
    --kernel-trace run, per-kernel counter averages from a --pmc run."""
    import sqlite3
    for path in paths:
        con = sqlite3.connect(path)
        print(f"## {os.path.basename(os.path.dirname(path))}/{os.path.basename(path)}")
        rows = con.execute(
            "select name, count(*), avg(end - start), min(end - start), max(end - start) "
            "from kernels group by name order by sum(end - start) desc").fetchall()
        if rows:
            # last_us: mean of the last `timed` dispatches of the kernel (a
            # default bench.py run times its last 20 steps, one dispatch each)
            timed = 20
            print(f"{'calls':>5} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'median_us':>10} "
                  f"{'last_us':>10}  kernel (last_us: mean of the last {timed} dispatches)")
            for name, cnt, avg, mn, mx in rows:
                ds = [r[0] for r in con.execute(
                    "select end - start from kernels where name = ? order by start", (name,))]
                med = sorted(ds)[len(ds) // 2]
                last = ds[-timed:]
                print(f"{cnt:5d} {avg / 1e3:10.1f} {mn / 1e3:10.1f} {mx / 1e3:10.1f} {med / 1e3:10.1f} "
                      f"{sum(last) / len(last) / 1e3:10.1f}  {name[:100]}")
        try:
            pm = con.execute("select name, counter_name, avg(counter_value), count(*) from pmc_events "
                             "group by name, counter_name order by name").fetchall()
        except sqlite3.OperationalError:
            pm = []
        if pm:
            print(f"{'counter':>12} {'avg_KiB':>14} {'dispatches':>10}  kernel")
            for name, cn, val, cnt in pm:
                print(f"{cn:>12} {val:14.1f} {cnt:10d}  {name[:100]}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline_8192_d128")
    ap.add_argument("--non-causal", action="store_true")
    ap.add_argument("--window", type=int, default=0,
                    help="causal sliding window of this many keys (0: none)")
    ap.add_argument("--fused-bwd", action="store_true",
                    help="time the single-kernel backward (fa_bwd_fused, atomic dQ) instead of "
                         "fa_bwd_dkdv + fa_bwd_dq")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--fwd-tiles", default="0,0")
    ap.add_argument("--dkdv-tiles", default="0,0")
    ap.add_argument("--dq-tiles", default="0,0")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times); used to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="DB",
                    help="only print a text summary of rocprofv3 result databases")
    args = ap.parse_args()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the path has no multi-GPU mode (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); heads would shard across GPUs with no communication.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_26_amd as fa
    from workloads import WORKLOADS, cast_io, make_inputs

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": 3}))
        return

    w = WORKLOADS[args.workload]
    causal = not args.non_causal
    window = args.window
    if window and not causal:
        ap.error("--window needs causal attention")
    bh, n, d = w.bh, w.n, w.d
    elt = 2 if w.dtype == "bf16" else 4
    ft = tuple(int(x) for x in args.fwd_tiles.split(","))
    kt = tuple(int(x) for x in args.dkdv_tiles.split(","))
    qt = tuple(int(x) for x in args.dq_tiles.split(","))
    print(f"# workload {w.name}: bh={bh} n={n} d={d} {w.dtype} causal={causal} window={window}",
          file=sys.stderr, flush=True)

    q, k, v, do = cast_io(make_inputs(bh, n, d, seed=0), w.dtype, "cuda")
    o = torch.empty_like(q)
    lse = torch.empty((bh, n), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    names = ("fwd", "preprocess", "bwd_fused") if args.fused_bwd else ("fwd", "preprocess", "dkdv", "dq")
    ws = None
    if args.fused_bwd:
        nbytes = fa.fa_bwd_fused_workspace_bytes(bh, n, d, fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32)
        ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda") if nbytes else None

    if window:
        def fwd_call():
            fa.fa_fwd_rect(q, k, v, o, lse, causal, None, *ft, stream=sptr, window=window)

        def dkdv_call():
            fa.fa_bwd_dkdv_rect(q, k, v, do, lse, delta, dk, dv, causal, None, *kt, stream=sptr,
                                window=window)

        def dq_call():
            fa.fa_bwd_dq_rect(q, k, v, do, lse, delta, dq, causal, None, *qt, stream=sptr, window=window)
    else:
        def fwd_call():
            fa.fa_fwd(q, k, v, o, lse, causal, None, *ft, stream=sptr)

        def dkdv_call():
            fa.fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, causal, None, *kt, stream=sptr)

        def dq_call():
            fa.fa_bwd_dq(q, k, v, do, lse, delta, dq, causal, None, *qt, stream=sptr)

    def fused_call():
        fa.fa_bwd_fused(q, k, v, do, lse, delta, dq, dk, dv, ws, causal, None, *kt, stream=sptr, window=window)

    calls = [fwd_call, lambda: fa.fa_bwd_preprocess(o, do, delta, stream=sptr)]
    calls += [fused_call] if args.fused_bwd else [dkdv_call, dq_call]

    def step(ev=None):
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_kernel = {nm: [] for nm in names}
    step_ms = []
    for ev in events:
        for j, nm in enumerate(names):
            per_kernel[nm].append(ev[j].elapsed_time(ev[j + 1]))
        step_ms.append(ev[0].elapsed_time(ev[len(names)]))
    avg = {nm: sum(x) / len(x) for nm, x in per_kernel.items()}
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = sum(step_ms) / len(step_ms)

    fwd_fl, bwd_fl = counted_flops(bh, n, d, causal, window)
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    tflops = (fwd_fl + bwd_fl) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = fwd_fl / (avg["fwd"] * 1e-3) / 1e12
    bwd_ms = sum(avg[nm] for nm in names if nm != "fwd")
    bwd_tf = bwd_fl / (bwd_ms * 1e-3) / 1e12

    kfl = kernel_flops(bh, n, d, causal, window)
    kby = kernel_bytes(bh, n, d, elt)
    dom = max((nm for nm in names if nm != "preprocess"), key=lambda nm: avg[nm])
    achieved = kfl[dom] / (avg[dom] * 1e-3) / 1e12
    roofline = {
        "kernel": dom,
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": (measured_traffic(dom)
                    if (w.name == "headline_8192_d128" and causal and not window and ft == (0, 0)
                        and kt == (0, 0) and qt == (0, 0) and not args.fused_bwd) else None),
        "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
        "avg_launch_ms": round(avg[dom], 4),
        "algorithmic_flops_per_launch": kfl[dom],
    }
    kernels = {}
    for nm in names:
        ent = {"avg_ms": round(avg[nm], 4)}
        if nm in kfl:
            ent["tflops"] = round(kfl[nm] / (avg[nm] * 1e-3) / 1e12, 1)
            ent["frac_mfma_peak"] = round(kfl[nm] / (avg[nm] * 1e-3) / 1e12 / peak, 4)
        ent["hbm_gbs"] = round(kby[nm] / (avg[nm] * 1e-3) / 1e9, 1)
        kernels[nm] = ent

    base = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        base = cpu_baseline(bh, n, d, causal, args.cpu_budget, window)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) Q, K, V, dO (numpy default_rng(0), cast to bf16)",
        "config": {"workload": w.name, "batch_heads": bh, "seq_len": n, "head_dim": d,
                   "causal": causal, "window": window,
                   "backward": "fused (fa_bwd_fused)" if args.fused_bwd else "two-kernel", "tiles": {"fwd": list(ft), "dkdv": list(kt), "dq": list(qt)}},
        "pct_of_mfma_peak": round(100 * tflops / peak, 2),
        "fwd_tflops": round(fwd_tf, 1),
        "fwd_pct_of_peak": round(100 * fwd_tf / peak, 2),
        "bwd_tflops": round(bwd_tf, 1),
        "bwd_pct_of_peak": round(100 * bwd_tf / peak, 2),
        "event_ms_per_step": round(ev_ms, 4),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": base,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
