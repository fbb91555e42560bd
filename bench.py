#!/usr/bin/env python3
"""Benchmark of the gfx950 exact-attention forward on one MI355X.

A step is one forward call (tiled QK^T, masked online softmax, P V, O and LSE
epilogue) over the named workload with inputs resident in HBM. The line printed
on stdout is one JSON object: TFLOP/s with FLOPs = 4 B H N^2 D (halved for a
causal mask), the roofline of the forward kernel measured with HIP events on
the stream it runs on, the fp64 CPU oracle timed on a bounded sample, and the
same shape's backward (timed separately, FLOPs counted as 2.5x the forward's).
Before the W warm-up launches the forward runs back to back for 2 s while the
shader clock is sampled (the line's "clock" object), so the warm-up and the K
timed launches run at the clock this load holds, not inside its ramp.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --extra      # also write fwd/bwd lines for every workload
    python bench.py --copy-mib 256   # also run a plain 256 MiB device copy (counter calibration)
    python bench.py --oracle-all 8   # host only: the fp64 oracle's rate on every workload
    python bench.py --summarize DIR_FETCH DIR_WRITE DIR_STATS   # write profiles/ summaries

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
METRIC_WORKLOAD_NAME = "fwd_bf16_b2h8n4096d128"
STATS_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -- python bench.py "
             "--workload {workload} --steps 200 --warmup 500 --no-cpu-baseline --no-clock")
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "fp8": 5000.0}
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
    n = w.batch * w.seqlen * w.heads * w.headdim
    if w.dtype == "fp8":  # e4m3 inputs, bf16 output
        return 3 * n + 2 * n + w.batch * w.heads * w.seqlen * 4
    esz = 4 if w.dtype == "f32" else 2
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
    return t[len(t) // 2], sum(t) / len(t), t[0]


MI355X_CUS = 256
BF16_FLOP_PER_CLK_PER_CU = 4096   # dense 32x32x16 bf16 MFMA rate: 2.5 PF/s at 2.4 GHz


def sample_gfx_clock(fn, seconds=2.0, period_s=0.004):
    """Shader clock while fn() runs back to back for about `seconds`.

    The GPU's own telemetry is read through amdsmi from a host thread while
    the launches run: the gpu_metrics table's per-XCD current graphics clocks
    (falling back to the driver's current GFX clock). The table changes only
    a few times a second and lags the clock: after an idle spell its first
    values are the idle clock and then points of the ramp. The value read
    last, after `seconds` of back-to-back launches, is the one reported;
    every change of value is listed with the time it was first read. Returns
    None with a reason if the telemetry is not readable here."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # noqa: BLE001 - report, never fail the bench on telemetry
        return {"mhz": None, "why": f"amdsmi unavailable: {type(e).__name__}: {e}"[:200]}

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))
                  and 0 < c < 10000]
            if xs:
                return sum(xs) / len(xs), "gpu_metrics current_gfxclks (mean over XCDs)"
        except Exception:  # noqa: BLE001
            pass
        c = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
        return float(c["clk"]), "amdsmi_get_clock_info GFX clk"

    samples, src, stop = [], [None], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                v, src[0] = read()
                samples.append((time.perf_counter() - t0, v))
            except Exception:  # noqa: BLE001
                pass
            stop.wait(period_s)

    for _ in range(50):  # clock up before sampling starts
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=2.0)
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if not samples:
        return {"mhz": None, "why": "no telemetry sample could be read"}
    changes = [[round(t, 3), v] for i, (t, v) in enumerate(samples)
               if i == 0 or v != samples[i - 1][1]]
    return {"mhz": samples[-1][1], "samples": len(samples),
            "changes_s_mhz": changes[-8:], "source": src[0],
            "how": f"read every {period_s * 1e3:.0f} ms from a host thread while the "
                   f"forward ran back to back for {seconds:.1f} s; the last value read"}


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


def plain_copy(mib, reps=5):
    """A plain device-to-device copy of `mib` MiB, the calibration kernel for
    the HBM byte counters (its bytes moved are known exactly)."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_means(csv_path, counter):
    """Per-dispatch mean of `counter` for each kernel name in a rocprofv3
    counter_collection.csv."""
    import csv
    acc = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize(fetch_dir, write_dir, stats_dir, copy_mib, cmds):
    """Turn rocprofv3 outputs into the committed profile summaries."""
    import glob
    fcsv = glob.glob(os.path.join(fetch_dir, "**", "*counter_collection.csv"), recursive=True)[0]
    wcsv = glob.glob(os.path.join(write_dir, "**", "*counter_collection.csv"), recursive=True)[0]
    fetch = _counter_means(fcsv, "FETCH_SIZE")
    write = _counter_means(wcsv, "WRITE_SIZE")
    attn = [k for k in fetch if "fwd_h16_kernel" in k][0]
    copy = [k for k in fetch if "fwd_h16_kernel" not in k and "opy" in k or "elementwise" in k]
    copy = max(copy, key=lambda k: fetch[k])
    known = copy_mib * (1 << 20)
    f_scale = known / (fetch[copy] * 1024.0)
    w_scale = known / (write[copy] * 1024.0)
    hbm_read = fetch[attn] * 1024.0 * f_scale
    hbm_write = write[attn] * 1024.0 * w_scale
    out = {"kernel": attn, "workload": "fwd_bf16_b2h8n4096d128",
           "kernel_source_hash": kernel_source_hash(),
           "fetch_size_kib_per_dispatch": fetch[attn], "write_size_kib_per_dispatch": write[attn],
           "copy_kernel": copy, "copy_bytes": known,
           "copy_fetch_kib": fetch[copy], "copy_write_kib": write[copy],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": hbm_read, "hbm_write_bytes_per_launch": hbm_write,
           "hbm_bytes_per_launch": hbm_read + hbm_write,
           "commands": cmds}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    stats_summary(stats_dir, "fwd_bf16_b2h8n4096d128", cmds["stats"])
    print(json.dumps(out, indent=1))


def pretty_kernel(name):
    """Readable form of this library's kernel names. The profiler leaves names
    whose template arguments are the extended float types (__bf16, _Float16)
    mangled; e.g. _ZN2fa14fwd_h16_kernelILi128ELb0EDF16bEEvNS_9FwdParamsE
    becomes fa::fwd_h16_kernel<128, false, bf16>."""
    import re
    m = re.match(r"_ZN2fa(\d+)(\w+?)I(.*)EEvNS_\d+\w+E", name)
    if not m or int(m.group(1)) != len(m.group(2)):
        return name
    args = re.findall(r"Li(\d+)E|Lb([01])E|DF16(b|_)", m.group(3))
    out = []
    for i, b, f in args:
        out.append(i if i else ("true" if b == "1" else "false") if b else
                   ("bf16" if f == "b" else "fp16"))
    return f"fa::{m.group(2)}<{', '.join(out)}>"


def stats_summary(stats_dir, workload, cmd):
    """Copy a rocprofv3 --stats table into profiles/kernel_stats_<workload>.txt."""
    import glob
    scsv = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    lines = open(scsv).read().strip().splitlines()
    # Steady state from the per-dispatch trace: the mean of each kernel's last
    # 100 launches (the table's averages include the cold warm-up launches).
    import csv
    tcsv = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    durs = {}
    for r in csv.DictReader(open(tcsv)):
        durs.setdefault(r["Kernel_Name"], []).append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    with open(os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.txt"), "w") as f:
        f.write(f"rocprofv3 --kernel-trace --stats summary of bench.py on {workload} "
                "(forward and backward kernels)\n")
        f.write("command: " + cmd + "\n\n")
        f.write("Table from the --stats output (averages over every launch, warm-up included):\n")
        rows = [r for r in lines[1:] if r.startswith('"_ZN2fa') or "fa::" in r.split('",')[0]]
        f.write("\n".join(lines[:1] + rows) + "\n")
        if len(lines) - 1 > len(rows):
            f.write(f"({len(lines) - 1 - len(rows)} other kernels, from setting up the inputs, "
                    "left out)\n")
        f.write("\n")
        f.write("Steady state from the kernel trace (mean / median of the last 100 launches, us):\n")
        for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            if "fa::" not in name and not name.startswith("_ZN2fa"):
                continue
            tail = sorted(d[-100:])
            f.write(f"  {pretty_kernel(name)}: mean {sum(tail) / len(tail) / 1e3:.2f}  "
                    f"median {tail[len(tail) // 2] / 1e3:.2f}  (launches {len(d)})\n")


# Counter passes for --pmc-summary: each fits the per-block limits of one
# rocprofv3 --pmc run (at most 8 SQ and 2 GRBM counters).
PMC_PASSES = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_WAIT_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
    "SQ_INSTS_SALU SQ_ACTIVE_INST_MISC GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_SCA SQ_INST_LEVEL_LDS SQ_LEVEL_WAVES "
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SMEM SQ_INSTS_BRANCH SQ_WAVES",
]
PMC_CMD = ("rocprofv3 --pmc {counters} --output-format csv -- python bench.py --workload "
           "{workload} --steps 5 --warmup 1 --no-cpu-baseline --no-clock")


def pmc_summary(dirs, workload, out_dir=None):
    """Per-kernel counter means (one dispatch) from one rocprofv3 --pmc output
    directory per pass of PMC_PASSES -> <out_dir or profiles>/pmc_<workload>.txt."""
    import csv
    import glob
    vals, durs = {}, {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if "fa::" not in r["Kernel_Name"] and not r["Kernel_Name"].startswith("_ZN2fa"):
                    continue
                name = pretty_kernel(r["Kernel_Name"])
                vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    durs.setdefault(name, []).append(
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"pmc_{workload}.txt"), "w") as f:
        f.write(f"rocprofv3 counter summary of bench.py on {workload}: per kernel, the mean of "
                "each counter over its dispatches (one dispatch's total). For dispatches of "
                "100 us or more, the clock they ran at (GRBM_GUI_ACTIVE / 8 XCDs over the "
                "dispatch's timestamps) and the MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES "
                "over 1024 SIMDs x those cycles).\n")
        for i, c in enumerate(PMC_PASSES):
            f.write(f"pass {i + 1}: " + PMC_CMD.format(counters=c, workload=workload) + "\n")
        for name, cs in vals.items():
            m = {c: sum(v) / len(v) for c, v in cs.items()}
            f.write(f"\n{name}\n")
            for c in sorted(m):
                f.write(f"  {c:28s} {m[c]:.4g}\n")
            try:
                f.write(f"  -> per wave-cycle: VALU issuing {m['SQ_ACTIVE_INST_VALU'] / m['SQ_WAVE_CYCLES']:.3f}, "
                        f"LDS issuing {m['SQ_ACTIVE_INST_LDS'] / m['SQ_WAVE_CYCLES']:.3f}, "
                        f"waiting {m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f}\n")
                f.write(f"  -> per MFMA: {m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f} VALU, "
                        f"{m['SQ_INSTS_VALU_TRANS_F32'] / m['SQ_INSTS_MFMA']:.2f} transcendental, "
                        f"{m['SQ_INSTS_LDS'] / m['SQ_INSTS_MFMA']:.2f} LDS instructions; "
                        f"LDS bank conflicts {m['SQ_LDS_BANK_CONFLICT']:.0f}\n")
            except (KeyError, ZeroDivisionError):
                pass
            try:
                # GRBM_GUI_ACTIVE counts the cycles of each of the 8 XCDs, summed;
                # SQ_VALU_MFMA_BUSY_CYCLES sums every MFMA's cycles over the 1024
                # SIMDs (it equals the MFMA count x 32 for 32x32x16 bf16). The
                # GRBM count also takes in cycles outside the dispatch's own
                # timestamps, a few microseconds' worth, so the two ratios are
                # written only for dispatches of 100 us or more.
                cyc = m["GRBM_GUI_ACTIVE"] / 8
                ns = sum(durs[name]) / len(durs[name])
                if ns < 100e3 or not m.get("SQ_INSTS_MFMA"):
                    raise KeyError(name)
                f.write(f"  -> clock {cyc / ns:.2f} GHz (GRBM_GUI_ACTIVE / 8 over the dispatch's "
                        f"{ns / 1e3:.1f} us); MFMA busy "
                        f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 4 * MI355X_CUS):.3f} of the "
                        f"SIMD-cycles\n")
            except (KeyError, ZeroDivisionError):
                pass


def cpu_baseline(w, seconds):
    """The fp64 oracle on (batch, head) slices of the same inputs until about
    `seconds` of CPU time have passed; returns TFLOP/s over the slices done."""
    import numpy as np
    import threadpoolctl
    from exact_io_aware_35_amd.inputs import make_inputs
    from oracle import attention_forward
    from oracle.fp8 import attention_forward_fp8
    d = make_inputs(w, 0)
    if w.dtype == "fp8":
        q, k, v = (d[x].numpy() for x in ("q", "k", "v"))
        ds = d["descale"]
        attention_forward = lambda q_, k_, v_, *a: attention_forward_fp8(  # noqa: E731
            q_, k_, v_, ds["q"], ds["k"], ds["v"], *a)
    else:
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
    import torch
    return {"value": round(done * flops_per_head / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "torch_threads": torch.get_num_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{done} of {w.batch * w.heads} (batch, head) slices, all {w.seqlen} "
                      f"query rows each, fp64 numpy; {dt:.1f} s"}


def _visible_keys(w, kl, rows):
    """Visible keys of each query row in ``rows`` (key length kl)."""
    import numpy as np
    r = np.asarray(rows, dtype=np.int64)
    lo = np.zeros_like(r)
    hi = np.full_like(r, kl - 1)
    if w.causal:
        hi = np.minimum(hi, r)
    if w.window[0] >= 0:
        lo = np.maximum(lo, r - w.window[0])
    if w.window[1] >= 0:
        hi = np.minimum(hi, r + w.window[1])
    return np.clip(hi - lo + 1, 0, None)


def oracle_rates(w, seconds):
    """Rates of the fp64 oracle on workload w, one record per leg: the forward,
    and the backward on workloads that have one. Each leg walks the (batch,
    head) slices until about `seconds` of CPU time have passed. On workloads
    whose oracle checks sampled query rows, the forward leg runs those rows
    only. FLOPs follow the metric's count (4 B H N^2 D, halved for causal;
    2.5x that for the backward); a sampled-row leg counts 4 D per visible
    (row, key) pair."""
    import numpy as np
    import threadpoolctl
    from exact_io_aware_35_amd.inputs import make_inputs
    from oracle import attention_backward, attention_forward, attention_forward_rows
    from oracle.fp8 import dequantise
    d = make_inputs(w, 0)
    if w.dtype == "fp8":
        ds = d["descale"]
        q, k, v = dequantise(d["q"].numpy(), d["k"].numpy(), d["v"].numpy(),
                             ds["q"], ds["k"], ds["v"])
    else:
        q, k, v = (d[x].float().numpy() for x in ("q", "k", "v"))
    sk = d["seqlens_k"].numpy() if d["seqlens_k"] is not None else None
    do = d["dout"].float().numpy() if d["dout"] is not None else None
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    per_slice = fwd_flops(w) / (w.batch * w.heads)
    legs = [("forward_rows" if w.sample_rows else "forward")]
    if w.backward:
        legs.append("backward")
    out = []
    for leg in legs:
        done, flops, t0 = 0, 0.0, time.perf_counter()
        for b in range(w.batch):
            for h in range(w.heads):
                sl = (slice(b, b + 1), slice(None), slice(h, h + 1), slice(None))
                qs, ks, vs = (np.ascontiguousarray(x[sl]) for x in (q, k, v))
                skb = None if sk is None else sk[b:b + 1]
                kw = dict(softmax_scale=w.softmax_scale, causal=w.causal, window=w.window,
                          seqlens_k=skb)
                if leg == "forward":
                    attention_forward(qs, ks, vs, **kw)
                    flops += per_slice
                elif leg == "forward_rows":
                    rows = d["rows"][h].numpy()
                    attention_forward_rows(qs, ks, vs, rows, **kw)
                    kl = w.seqlen if skb is None else int(skb[0])
                    flops += 4.0 * w.headdim * float(_visible_keys(w, kl, rows).sum())
                else:
                    attention_backward(qs, ks, vs, np.ascontiguousarray(do[sl]), **kw)
                    flops += 2.5 * per_slice
                done += 1
                if time.perf_counter() - t0 > seconds:
                    break
            if time.perf_counter() - t0 > seconds:
                break
        dt = time.perf_counter() - t0
        what = (f"{w.sample_rows + len(w.extra_rows)} sampled query rows of each slice"
                if leg == "forward_rows" else f"all {w.seqlen} query rows of each slice")
        out.append({"workload": w.name, "leg": leg, "value": round(flops / dt / 1e12, 6),
                    "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                    "sample": f"{done} of {w.batch * w.heads} (batch, head) slices, {what}, "
                              f"fp64 numpy; {dt:.1f} s"})
    return out


def run_workload(w, steps, warmup, backward=False, variant=None, before=None):
    """(fwd ms, bwd ms or None) for workload w on cuda:0. variant: None, "alibi"
    (the usual geometric slopes per head) or "qkvpacked" (one packed input).
    before(fwd), if given, runs once the forward is built and before its
    warm-up launches."""
    import torch
    import exact_io_aware_35_amd as fa
    from exact_io_aware_35_amd.inputs import make_inputs
    d = make_inputs(w, 0)
    dev = torch.device("cuda:0")
    q, k, v = (d[x].to(dev) for x in ("q", "k", "v"))
    sk = d["seqlens_k"].to(dev) if d["seqlens_k"] is not None else None
    out = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "fp8" else q.dtype, device=dev)
    lse = torch.empty((w.batch, w.heads, w.seqlen), dtype=torch.float32, device=dev)
    kw = dict(causal=w.causal, window=w.window, softmax_scale=w.softmax_scale, seqlens_k=sk)
    if w.dtype == "fp8":
        ds = d["descale"]
        fwd = fa.prepare_forward_fp8(q, k, v, out, lse, ds["q"], ds["k"], ds["v"], **kw)
        if before is not None:
            before(fwd)
        return time_gpu(fwd, steps, warmup), None, (fwd, q)
    if variant is None:
        fwd = fa.prepare_forward(q, k, v, out, lse, **kw)
    elif variant == "alibi":
        kw["alibi_slopes"] = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.heads) for h in range(w.heads)],
                                          dtype=torch.float32, device=dev)
        fwd = lambda: fa.forward(q, k, v, out=out, lse=lse, **kw)
    else:
        qkv = torch.stack([q, k, v], dim=2).contiguous()
        fwd = lambda: fa.forward_qkvpacked(qkv, out=out, lse=lse, **kw)
    if before is not None:
        before(fwd)
    t_f = time_gpu(fwd, steps, warmup)
    t_b = None
    if backward:
        do = d["dout"].to(dev) if d["dout"] is not None else torch.randn_like(q)
        ws = torch.empty(fa.workspace_size(w.batch, w.heads, w.seqlen, w.headdim),
                         dtype=torch.uint8, device=dev)
        if variant == "qkvpacked":
            dqkv = torch.empty_like(qkv)
            bwd = lambda: fa.backward_qkvpacked(qkv, out, lse, do, dqkv=dqkv, workspace=ws, **kw)
        else:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            bwd = lambda: fa.backward(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws,
                                      **kw)
        t_b = time_gpu(bwd, steps, warmup)
    return t_f, t_b, (fwd, q)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed launches before the timed ones (after the clock sampling, "
                         "which already runs the forward back to back for 2 s)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock (amdsmi) before the warm-up")
    ap.add_argument("--extra", action="store_true",
                    help="also time fwd/bwd of every workload; lines go to stderr")
    ap.add_argument("--oracle-all", type=float, default=None, metavar="SECONDS",
                    help="time the fp64 oracle on every workload (forward, backward where the "
                         "workload has one; sampled rows for the long ones), each leg bounded "
                         "by SECONDS of CPU time; prints one 'oracle:' JSON line per leg")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB")
    ap.add_argument("--summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "STATS_DIR"),
                    help="write the profiles/ summaries from rocprofv3 output directories")
    ap.add_argument("--pmc-summary", nargs="+", metavar="ARG",
                    help="WORKLOAD DIR1 DIR2 DIR3: write profiles/pmc_WORKLOAD.txt from the "
                         "rocprofv3 --pmc output directories of the three counter passes")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_DIR", "WORKLOAD"),
                    help="write profiles/kernel_stats_WORKLOAD.txt from a --stats run of "
                         "bench.py --workload WORKLOAD")
    args = ap.parse_args()
    if args.oracle_all is not None:
        # Host-only: no GPU is touched.
        from exact_io_aware_35_amd.inputs import WORKLOADS
        for wk in WORKLOADS.values():
            for rec in oracle_rates(wk, args.oracle_all):
                print("oracle: " + json.dumps(rec), flush=True)
        return
    if args.summarize:
        pmc = "rocprofv3 {opts} -- python bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-clock --copy-mib 256"
        summarize(*args.summarize, copy_mib=256,
                  cmds={"fetch": pmc.format(opts="--pmc FETCH_SIZE --output-format csv"),
                        "write": pmc.format(opts="--pmc WRITE_SIZE --output-format csv"),
                        "stats": STATS_CMD.format(workload=METRIC_WORKLOAD_NAME)})
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[1:], args.pmc_summary[0])
        return
    if args.stats_summary:
        stats_summary(args.stats_summary[0], args.stats_summary[1],
                      STATS_CMD.format(workload=args.stats_summary[1]))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: it measures the single-GPU kernels "
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

    # The shader clock is sampled first, while the forward runs back to back
    # for 2 s: it reports the clock this load holds, and the warm-up and
    # timed launches that follow then run at that steady state instead of
    # inside the clock's ramp after an idle spell (about 400 launches, which
    # a short warm-up does not cover).
    clock = {}
    before = None if args.no_clock else (lambda fn: clock.update(sample_gfx_clock(fn)))
    # The backward is built for the 16-bit types.
    ms, bwd_ms, (fwd, q) = run_workload(w, args.steps, args.warmup,
                                        backward=w.dtype in ("bf16", "f16"), before=before)
    med_ms, mean_ms, min_ms = per_launch_ms(fwd, min(args.steps, 100))
    flops = fwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    # The forward is one kernel; its average launch duration comes from an
    # event pair around each launch on the stream it runs on (the timed
    # region's mean also holds the host-side launch gaps).
    kernel_tflops = flops / (mean_ms * 1e-3) / 1e12
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
                     "traffic": traffic if w.name == METRIC_WORKLOAD_NAME else None,
                     "kernel": {"bf16": "fwd_h16_kernel<bf16>", "f16": "fwd_h16_kernel<fp16>",
                                "f32": "fwd_f32_kernel", "fp8": "fwd_fp8_kernel"}[w.dtype],
                     "launch_ms_mean": round(mean_ms, 5), "launch_ms_median": round(med_ms, 5),
                     "launch_ms_min": round(min_ms, 5),
                     "algorithmic_bytes": algorithmic_bytes(w),
                     "hbm_gbs": round(algorithmic_bytes(w) / (mean_ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(algorithmic_bytes(w) / (mean_ms * 1e-3) / 1e9
                                       / PEAK_HBM_GBS, 4)},
        "cpu_baseline": None,
        # The same shape's backward (prep, dK/dV and dQ kernels), counted as
        # 2.5x the forward's FLOPs (five N x N x D products against two).
        "backward": None if bwd_ms is None else {
            "ms": round(bwd_ms, 5), "tflops": round(2.5 * flops / (bwd_ms * 1e-3) / 1e12, 2),
            "frac_of_mfma_peak": round(2.5 * flops / (bwd_ms * 1e-3) / 1e12 / peak, 4),
            "flops": 2.5 * flops},
    }
    if clock:
        if clock.get("mhz"):
            # The dtype's dense peak scales with the clock (bf16: 4096 FLOP per
            # clock per CU; the other dtypes in proportion to their peaks).
            peak_clk = (MI355X_CUS * BF16_FLOP_PER_CLK_PER_CU * clock["mhz"] * 1e6 / 1e12
                        * peak / PEAK_TFLOPS["bf16"])
            clock["peak_tflops_at_clock"] = round(peak_clk, 1)
            clock["frac_at_clock"] = round(kernel_tflops / peak_clk, 4)
        line["clock"] = clock
    if args.extra:
        for name, wk in WORKLOADS.items():
            tf, tb, _ = run_workload(wk, 20, 3, backward=wk.backward or name == METRIC_WORKLOAD)
            ff = fwd_flops(wk)
            rec = {"workload": name, "fwd_ms": round(tf, 4), "fwd_tflops": round(ff / tf / 1e9, 2)}
            if tb is not None:
                rec.update(bwd_ms=round(tb, 4), bwd_tflops=round(2.5 * ff / tb / 1e9, 2))
            print("extra: " + json.dumps(rec), file=sys.stderr, flush=True)
        for variant in ("alibi", "qkvpacked"):
            tf, tb, _ = run_workload(w, 20, 3, backward=True, variant=variant)
            rec = {"workload": w.name, "variant": variant, "fwd_ms": round(tf, 4),
                   "fwd_tflops": round(flops / tf / 1e9, 2), "bwd_ms": round(tb, 4),
                   "bwd_tflops": round(2.5 * flops / tb / 1e9, 2)}
            print("extra: " + json.dumps(rec), file=sys.stderr, flush=True)
    if args.copy_mib:
        plain_copy(args.copy_mib)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
