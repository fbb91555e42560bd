#!/usr/bin/env python3
"""Benchmark of the gfx950 exact-attention forward on one MI355X.

A step is one forward call (tiled QK^T, masked online softmax, P V, O and LSE
epilogue) over the named workload with inputs resident in HBM. The line printed
on stdout is one JSON object: TFLOP/s with FLOPs = 4 B H N^2 D (halved for a
causal mask), the roofline of the forward kernel measured with HIP events on
the stream it runs on, and the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --extra      # also write fwd/bwd lines for every workload

Only one GPU is used: --gpus N with N > 1 exits with a message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd/bwd TFLOPS bf16 (B2 H8 N4096 D128) + % of MFMA peak, 1 MI355X"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_b2h8n4096d128.json")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_io_aware_35_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_common.h", "fa_params.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def fwd_flops(w, causal=None):
    c = w.causal if causal is None else causal
    f = 4.0 * w.batch * w.heads * w.seqlen * w.seqlen * w.headdim
    return f / 2 if c else f


def algorithmic_bytes(w):
    """Compulsory HBM bytes of one forward: read Q, K, V; write O and LSE."""
    esz = 2 if w.dtype == "bf16" else 4
    n = w.batch * w.seqlen * w.heads * w.headdim
    return 4 * n * esz + w.batch * w.heads * w.seqlen * 4


def time_gpu(fn, steps, warmup):
    """Mean milliseconds per call of fn() between HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def per_launch_ms(fn, launches):
    """Per-launch durations from an event pair around each launch (median)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return t[len(t) // 2], sum(t) / len(t)


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, seconds):
    """The fp64 oracle on (batch, head) slices of the same inputs until about
    `seconds` of CPU time have passed; returns TFLOP/s over the slices done."""
    import numpy as np
    import threadpoolctl
    from exact_io_aware_35_amd.inputs import make_inputs
    from oracle import attention_forward
    d = make_inputs(w, 0)
    q, k, v = (d[x].float().numpy() for x in ("q", "k", "v"))
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    done, t0 = 0, time.perf_counter()
    flops_per_head = fwd_flops(w) / (w.batch * w.heads)
    for b in range(w.batch):
        for h in range(w.heads):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1), slice(None))
            attention_forward(np.ascontiguousarray(q[sl]), np.ascontiguousarray(k[sl]),
                              np.ascontiguousarray(v[sl]), w.softmax_scale, w.causal, w.window)
            done += 1
            if time.perf_counter() - t0 > seconds:
                break
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done * flops_per_head / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.batch * w.heads} (batch, head) slices, all {w.seqlen} "
                      f"query rows each, fp64 numpy; {dt:.1f} s"}


def run_workload(w, steps, warmup, backward=False):
    """(fwd ms, bwd ms or None) for workload w on cuda:0."""
    import torch
    import exact_io_aware_35_amd as fa
    from exact_io_aware_35_amd.inputs import make_inputs
    d = make_inputs(w, 0)
    dev = torch.device("cuda:0")
    q, k, v = (d[x].to(dev) for x in ("q", "k", "v"))
    sk = d["seqlens_k"].to(dev) if d["seqlens_k"] is not None else None
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.seqlen), dtype=torch.float32, device=dev)
    kw = dict(causal=w.causal, window=w.window, softmax_scale=w.softmax_scale, seqlens_k=sk)
    fwd = lambda: fa.forward(q, k, v, out=out, lse=lse, **kw)
    t_f = time_gpu(fwd, steps, warmup)
    t_b = None
    if backward:
        do = d["dout"].to(dev) if d["dout"] is not None else torch.randn_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.workspace_size(w.batch, w.heads, w.seqlen, w.headdim),
                         dtype=torch.uint8, device=dev)
        bwd = lambda: fa.backward(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
        t_b = time_gpu(bwd, steps, warmup)
    return t_f, t_b, (fwd, q)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--extra", action="store_true",
                    help="also time fwd/bwd of every workload; lines go to stderr")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build measures the single-GPU kernel "
              "(heads and batch shard across GPUs with no exchange); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_io_aware_35_amd.inputs import METRIC_WORKLOAD, WORKLOADS
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = WORKLOADS[args.workload or METRIC_WORKLOAD]
    print(f"bench: workload {w.name}, steps {args.steps}, warmup {args.warmup}",
          file=sys.stderr, flush=True)

    ms, _, (fwd, q) = run_workload(w, args.steps, args.warmup)
    med_ms, mean_ms = per_launch_ms(fwd, min(args.steps, 100))
    flops = fwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    # One kernel per step: its average launch duration is the timed region's
    # mean; the per-launch event pairs are reported beside it.
    kernel_tflops = flops / (ms * 1e-3) / 1e12
    traffic = load_traffic()
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seqlen": w.seqlen,
                   "headdim": w.headdim, "causal": w.causal, "window": list(w.window),
                   "flops_per_step": flops, "pass": "forward"},
        "frac_of_mfma_peak": round(tflops / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(kernel_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / peak, 4),
                     "traffic": traffic, "kernel": "fwd_bf16_kernel",
                     "launch_ms_mean": round(mean_ms, 5), "launch_ms_median": round(med_ms, 5),
                     "algorithmic_bytes": algorithmic_bytes(w)},
        "cpu_baseline": None,
    }
    if args.extra:
        for name, wk in WORKLOADS.items():
            tf, tb, _ = run_workload(wk, 20, 3, backward=wk.backward or name == METRIC_WORKLOAD)
            ff = fwd_flops(wk)
            rec = {"workload": name, "fwd_ms": round(tf, 4), "fwd_tflops": round(ff / tf / 1e9, 2)}
            if tb is not None:
                rec.update(bwd_ms=round(tb, 4), bwd_tflops=round(2.5 * ff / tb / 1e9, 2))
            print("extra: " + json.dumps(rec), file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
