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
    "fwd": ("fa_fwd_bf16.hip", "fa_common.h", "fa_order.h", "fa_order.cpp"),
    "dkdv": ("fa_bwd_bf16.hip", "fa_common.h", "fa_order.h", "fa_order.cpp"),
    "dq": ("fa_bwd_bf16.hip", "fa_common.h", "fa_order.h", "fa_order.cpp"),
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


def _oracle_seconds(q, k, v, do, causal, window):
    """Wall seconds of the oracle's forward and backward on one head."""
    import oracle
    t0 = time.perf_counter()
    oracle.attention_forward(q, k, v, causal=causal, window=window)
    t1 = time.perf_counter()
    oracle.attention_backward(q, k, v, do, causal=causal, window=window)
    return t1 - t0, time.perf_counter() - t1


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:
        return None


def cpu_oracle_run(name, causal, heads=None, window=0, budget_s=None):
    """The fp64 oracle (as it stands) timed on the host, forward and backward
    separately, one head after another on the workload's own seeded inputs:
    every head, the first `heads` heads, or heads until about `budget_s`."""
    from workloads import WORKLOADS, cast_io, make_inputs, to_f64

    w = WORKLOADS[name]
    arrays = make_inputs(w.bh, w.n, w.d, seed=0)
    q, k, v, do = (to_f64(t) for t in cast_io(arrays, w.dtype))
    todo = w.bh if heads is None else min(heads, w.bh)
    fwd_s = bwd_s = 0.0
    done = 0
    for h in range(todo):
        a, b = _oracle_seconds(q[h], k[h], v[h], do[h], causal, window)
        fwd_s, bwd_s, done = fwd_s + a, bwd_s + b, done + 1
        el = fwd_s + bwd_s
        if budget_s is not None and (el >= budget_s or el / done * (done + 1) > budget_s * 1.5):
            break
    fwd_fl, bwd_fl = counted_flops(done, w.n, w.d, causal, window)
    return {"workload": name, "batch_heads": w.bh, "seq_len": w.n, "head_dim": w.d, "dtype": w.dtype,
            "causal": causal, "heads_timed": done, "fwd_s": round(fwd_s, 3), "bwd_s": round(bwd_s, 3),
            "fwd_tflops": fwd_fl / fwd_s / 1e12, "bwd_tflops": bwd_fl / bwd_s / 1e12,
            "tflops": (fwd_fl + bwd_fl) / (fwd_s + bwd_s) / 1e12}


# the oracle timed per configuration: every head of the first four, two heads
# of the long-context one
CPU_ORACLE_CONFIGS = (("gradcheck_48", (False, True), None), ("tile_sweep_256", (False, True), None),
                      ("bf16_2048_d64", (True,), None), ("headline_8192_d128", (True, False), None),
                      ("long_32768_d128", (True,), 2))


def cpu_baseline(w, causal, window=0, scope="all", budget_s=25.0):
    """The contract's cpu_baseline object (the oracle on the timed workload)
    and, with scope "all", the per-configuration oracle table."""
    cores = len(os.sched_getaffinity(0))
    threads = _blas_threads() or cores
    table = []
    main = None
    if scope == "all":
        for name, modes, heads in CPU_ORACLE_CONFIGS:
            for c in modes:
                print(f"# oracle: {name} causal={c}", file=sys.stderr, flush=True)
                r = cpu_oracle_run(name, c, heads)
                table.append(r)
                if name == w.name and c == causal and not window:
                    main = r
    if main is None:
        print(f"# oracle: {w.name} causal={causal} window={window} (sample)", file=sys.stderr, flush=True)
        main = cpu_oracle_run(w.name, causal, window=window, budget_s=budget_s)
    base = {
        "value": main["tflops"],
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{main['heads_timed']} of {w.bh} heads (N={w.n}, d={w.d}, "
                  f"{'causal' if causal else 'non-causal'}{f', window {window}' if window else ''}), "
                  f"fp64 forward {main['fwd_s']:.1f} s + backward {main['bwd_s']:.1f} s; "
                  f"host cores available: {cores}, BLAS threads: {threads}",
        "seconds": main["fwd_s"] + main["bwd_s"],
    }
    if table:
        base["by_config"] = [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()} for r in table]
    return base


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


def metric_name(dtype, causal, window, n, d):
    mode = ("causal" + (f", window {window}" if window else "")) if causal else "non-causal"
    return f"fwd+bwd attention TFLOPS ({dtype}, {mode}, N={n}, d={d}) + % of MFMA peak"


def _stats(xs):
    ys = sorted(xs)
    return {"avg_ms": round(sum(xs) / len(xs), 4), "median_ms": round(ys[len(ys) // 2], 4), "min_ms": round(ys[0], 4)}


def measure(fa, torch, w, causal, window, tiles, fused, steps, warmup):
    """Time `steps` whole steps (forward, preprocess, dK/dV, dQ, or the fused
    backward) on the workload's seeded inputs, after `warmup` untimed ones:
    the wall time per step over one pass with nothing between the calls, and
    per-kernel HIP-event times over a second pass (every event recorded on
    the stream the kernels are launched on)."""
    from workloads import cast_io, make_inputs

    bh, n, d = w.bh, w.n, w.d
    ft, kt, qt = tiles
    q, k, v, do = cast_io(make_inputs(bh, n, d, seed=0), w.dtype, "cuda")
    o = torch.empty_like(q)
    lse = torch.empty((bh, n), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    names = ("fwd", "preprocess", "bwd_fused") if fused else ("fwd", "preprocess", "dkdv", "dq")
    ws = None
    if fused:
        nbytes = fa.fa_bwd_fused_workspace_bytes(bh, n, d, fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32)
        ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda") if nbytes else None
    if window:
        calls = [lambda: fa.fa_fwd_rect(q, k, v, o, lse, causal, None, *ft, stream=sptr, window=window)]
    else:
        calls = [lambda: fa.fa_fwd(q, k, v, o, lse, causal, None, *ft, stream=sptr)]
    calls.append(lambda: fa.fa_bwd_preprocess(o, do, delta, stream=sptr))
    if fused:
        calls.append(lambda: fa.fa_bwd_fused(q, k, v, do, lse, delta, dq, dk, dv, ws, causal, None, *kt,
                                             stream=sptr, window=window))
    elif window:
        calls.append(lambda: fa.fa_bwd_dkdv_rect(q, k, v, do, lse, delta, dk, dv, causal, None, *kt, stream=sptr,
                                                 window=window))
        calls.append(lambda: fa.fa_bwd_dq_rect(q, k, v, do, lse, delta, dq, causal, None, *qt, stream=sptr,
                                               window=window))
    else:
        calls.append(lambda: fa.fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, causal, None, *kt, stream=sptr))
        calls.append(lambda: fa.fa_bwd_dq(q, k, v, do, lse, delta, dq, causal, None, *qt, stream=sptr))

    def step(ev=None):
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the wall clock over `steps` whole steps, with nothing between the calls
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel HIP events in a second pass (the event records add a little
    # time of their own between the kernels)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    per_kernel = {nm: [ev[j].elapsed_time(ev[j + 1]) for ev in events] for j, nm in enumerate(names)}
    return {"names": names, "ms_per_step": wall * 1e3 / steps,
            "event_ms_per_step": sum(ev[0].elapsed_time(ev[len(names)]) for ev in events) / steps,
            "per_kernel": per_kernel, "step": step}


def summarize(w, causal, window, m, peak):
    """TFLOPS and fractions of the MFMA peak for one measured workload."""
    bh, n, d = w.bh, w.n, w.d
    elt = 2 if w.dtype == "bf16" else 4
    names = m["names"]
    stats = {nm: _stats(m["per_kernel"][nm]) for nm in names}
    fwd_fl, bwd_fl = counted_flops(bh, n, d, causal, window)
    kfl = kernel_flops(bh, n, d, causal, window)
    kby = kernel_bytes(bh, n, d, elt)
    fwd_ms = stats["fwd"]["avg_ms"]
    bwd_ms = sum(stats[nm]["avg_ms"] for nm in names if nm != "fwd")
    kernels = {}
    for nm in names:
        ent = dict(stats[nm])
        if nm in kfl:
            tf = kfl[nm] / (ent["avg_ms"] * 1e-3) / 1e12
            ent["tflops"] = round(tf, 1)
            ent["frac_mfma_peak"] = round(tf / peak, 4)
        ent["hbm_gbs"] = round(kby[nm] / (ent["avg_ms"] * 1e-3) / 1e9, 1)
        kernels[nm] = ent
    tflops = (fwd_fl + bwd_fl) / (m["ms_per_step"] * 1e-3) / 1e12
    return {
        "ms_per_step": round(m["ms_per_step"], 4),
        "tflops": round(tflops, 2),
        "pct_of_mfma_peak": round(100 * tflops / peak, 2),
        "fwd_tflops": round(fwd_fl / (fwd_ms * 1e-3) / 1e12, 1),
        "fwd_pct_of_peak": round(100 * fwd_fl / (fwd_ms * 1e-3) / 1e12 / peak, 2),
        "bwd_tflops": round(bwd_fl / (bwd_ms * 1e-3) / 1e12, 1),
        "bwd_pct_of_peak": round(100 * bwd_fl / (bwd_ms * 1e-3) / 1e12 / peak, 2),
        "event_ms_per_step": round(m["event_ms_per_step"], 4),
        "kernels": kernels,
    }


def sample_clock(step, seconds=3.0, settle=1.5):
    """Shader (GFX) clock while the timed step runs back to back for about
    `seconds`: the mean over the GPU's XCDs of amdsmi's current_gfxclks,
    sampled every 10 ms, keeping the samples taken after `settle` seconds
    (the metrics table trails the load by up to about a second).  Returns
    None where amdsmi is not available."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:   # no SMI library or no access: the field stays null
        print(f"# clock sampling unavailable: {e!r}", file=sys.stderr, flush=True)
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                clks = [c for c in amdsmi.amdsmi_get_gpu_metrics_info(handle)["current_gfxclks"] if isinstance(c, int)]
                if clks:
                    samples.append((time.perf_counter(), sum(clks) / len(clks)))
            except Exception:
                pass
            time.sleep(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    t1 = time.perf_counter()
    kept = [c for t, c in samples if t >= t0 + settle]
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not kept:
        return None
    kept.sort()
    return {"mhz_median": round(kept[len(kept) // 2], 1), "mhz_min": round(kept[0], 1), "mhz_max": round(kept[-1], 1),
            "samples": len(kept), "source": f"amdsmi current_gfxclks (mean over XCDs), sampled every 10 ms while "
                                            f"the timed step ran back to back for {seconds:.0f} s, after the first "
                                            f"{settle:.1f} s"}


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
    ap.add_argument("--cpu-scope", choices=("all", "sample"), default="all",
                    help="all: the oracle on every configuration (about two minutes); sample: on the timed "
                         "workload only, about --cpu-budget seconds")
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the non-causal headline and long-context sub-records and the clock sampling")
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
    from workloads import WORKLOADS

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
    tiles = tuple(tuple(int(x) for x in a.split(",")) for a in (args.fwd_tiles, args.dkdv_tiles, args.dq_tiles))
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    default_run = (w.name == "headline_8192_d128" and causal and not window and not args.fused_bwd
                   and tiles == ((0, 0), (0, 0), (0, 0)))
    print(f"# workload {w.name}: bh={w.bh} n={w.n} d={w.d} {w.dtype} causal={causal} window={window}",
          file=sys.stderr, flush=True)

    m = measure(fa, torch, w, causal, window, tiles, args.fused_bwd, args.steps, args.warmup)
    print(f"# timed {args.steps} steps", file=sys.stderr, flush=True)
    res = summarize(w, causal, window, m, peak)
    clock = None
    if not args.no_extra:
        clock = sample_clock(m["step"])
    del m
    torch.cuda.empty_cache()

    kfl = kernel_flops(w.bh, w.n, w.d, causal, window)
    dom = max((nm for nm in res["kernels"] if nm != "preprocess"), key=lambda nm: res["kernels"][nm]["avg_ms"])
    dom_ms = res["kernels"][dom]["avg_ms"]
    achieved = kfl[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {
        "kernel": dom,
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(dom) if default_run else None,
        "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
        "avg_launch_ms": dom_ms,
        "algorithmic_flops_per_launch": kfl[dom],
    }
    device = {"name": torch.cuda.get_device_name(0),
              "compute_units": torch.cuda.get_device_properties(0).multi_processor_count,
              "gfx_clock_under_load": clock}
    if clock and w.dtype == "bf16":
        # the same fraction against the peak at the clock the chip actually ran at
        at_clock = device["compute_units"] * 4096 * clock["mhz_median"] * 1e6 / 1e12
        device["bf16_peak_at_that_clock_tflops"] = round(at_clock, 1)
        roofline["frac_at_achieved_clock"] = round(achieved / at_clock, 4)

    extra = {}
    if default_run and not args.no_extra:
        for key, name, c in (("headline_non_causal", "headline_8192_d128", False),
                             ("long_context_causal", "long_32768_d128", True)):
            ws_ = WORKLOADS[name]
            print(f"# sub-record {key}: {name} causal={c}", file=sys.stderr, flush=True)
            mm = measure(fa, torch, ws_, c, 0, tiles, False, args.steps, args.warmup)
            sub = summarize(ws_, c, 0, mm, peak)
            del mm
            torch.cuda.empty_cache()
            sub = {"config": {"workload": name, "batch_heads": ws_.bh, "seq_len": ws_.n, "head_dim": ws_.d,
                              "causal": c}, **sub}
            extra[key] = sub

    base = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        base = cpu_baseline(w, causal, window, scope=args.cpu_scope if default_run else "sample",
                            budget_s=args.cpu_budget)

    out = {
        "metric": metric_name(w.dtype, causal, window, w.n, w.d),
        "value": res["tflops"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic: seeded N(0,1) Q, K, V, dO (numpy default_rng(0), cast to {w.dtype})",
        "config": {"workload": w.name, "batch_heads": w.bh, "seq_len": w.n, "head_dim": w.d,
                   "causal": causal, "window": window,
                   "backward": "fused (fa_bwd_fused)" if args.fused_bwd else "two-kernel",
                   "tiles": {"fwd": list(tiles[0]), "dkdv": list(tiles[1]), "dq": list(tiles[2])}},
        **{k: v for k, v in res.items() if k not in ("ms_per_step", "tflops")},
        "device": device,
        "roofline": roofline,
        "cpu_baseline": base,
        **extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
