"""Host-side parts of bench.py (no GPU): the oracle-rate legs and their FLOP
counts. The sampled-row count is checked against the closed-form visible-pair
count of the oracle on full rows."""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_io_aware_35_amd.inputs import WORKLOADS, Workload  # noqa: E402
from oracle import visible_pair_count  # noqa: E402


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (7, 0)),
                                           (False, (3, 5))])
def test_visible_keys_sum_to_the_visible_pair_count(causal, window):
    w = Workload("t", "bf16", 1, 1, 40, 64, causal=causal, window=window)
    for kl in (40, 23):
        got = int(bench._visible_keys(w, kl, np.arange(40)).sum())
        assert got == visible_pair_count(40, causal, window, np.array([kl]))


def test_oracle_rates_report_each_leg():
    recs = bench.oracle_rates(WORKLOADS["fwd_f32_b1h1n256d64"], 0.0)
    assert [r["leg"] for r in recs] == ["forward"]
    w = Workload("t", "bf16", 1, 2, 64, 64, causal=True, backward=True)
    recs = bench.oracle_rates(w, 0.0)
    assert [r["leg"] for r in recs] == ["forward", "backward"]
    for r in recs:
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
        assert r["sample"].startswith("1 of 2 ")  # stops after the first slice at 0 s
    w = Workload("t", "bf16", 1, 1, 128, 64, causal=True, sample_rows=5, extra_rows=(0, 127))
    (rec,) = bench.oracle_rates(w, 10.0)
    assert rec["leg"] == "forward_rows" and "7 sampled query rows" in rec["sample"]


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
