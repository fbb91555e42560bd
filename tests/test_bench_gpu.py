"""The benchmark's JSON line on the GPU: one short run of bench.py in a child
process, checked for the fields and the arithmetic that its readers rely on."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_has_the_contract_fields():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20",
                        "--warmup", "5", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert d["dtype"] == "bf16" and d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert d["config"]["workload"] == "fwd_bf16_b2h8n4096d128"
    # value is the timed region's rate: FLOPs per step over ms_per_step.
    flops = d["config"]["flops_per_step"]
    assert flops == 4.0 * 2 * 8 * 4096 ** 2 * 128
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["peak"] == 2500.0 and 0.0 < rl["frac"] < 1.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["launch_ms_min"] <= rl["launch_ms_median"] and rl["launch_ms_min"] <= rl["launch_ms_mean"]
    assert rl["algorithmic_bytes"] == 4 * 2 * 8 * 4096 * 128 * 2 + 2 * 8 * 4096 * 4
    assert d["backward"]["ms"] > 0.0
    clk = d.get("clock")
    assert clk is not None
    if clk.get("mhz"):
        assert 100.0 < clk["mhz"] < 3000.0
        assert 0.0 < clk["frac_at_clock"]
