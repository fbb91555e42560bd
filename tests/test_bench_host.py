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


def test_pretty_kernel_names():
    assert bench.pretty_kernel("_ZN2fa14fwd_h16_kernelILi128ELb0EDF16bEEvNS_9FwdParamsE") == \
        "fa::fwd_h16_kernel<128, false, bf16>"
    assert bench.pretty_kernel("_ZN2fa14bwd_kvq_kernelILi64ELb1EDF16_EEvNS_9BwdParamsEii") == \
        "fa::bwd_kvq_kernel<64, true, fp16>"
    assert bench.pretty_kernel("not_mangled") == "not_mangled"


def _counter_csv(path, kernel, counters, dur_ns):
    import csv
    cols = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (name, val) in enumerate(counters.items()):
            w.writerow({"Correlation_Id": 1, "Dispatch_Id": 1, "Kernel_Name": kernel,
                        "Counter_Name": name, "Counter_Value": val,
                        "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur_ns})


def test_pmc_summary_derives_clock_and_mfma_busy(tmp_path):
    # 200000 cycles per XCD over 100 us is 2 GHz; MFMA busy half of 1024 SIMDs
    # x 200000 cycles is 0.5. A 50 us dispatch gets no derived line.
    long_k = "_ZN2fa14fwd_h16_kernelILi128ELb0EDF16bEEvNS_9FwdParamsE"
    short_k = "_ZN2fa14fwd_h16_kernelILi64ELb0EDF16bEEvNS_9FwdParamsE"
    for i, (k, ns) in enumerate(((long_k, 100000), (short_k, 50000))):
        d = tmp_path / f"pass{i}"
        d.mkdir()
        _counter_csv(d / "x_counter_collection.csv", k,
                     {"GRBM_GUI_ACTIVE": 8 * 2e5 * ns / 1e5, "SQ_INSTS_MFMA": 1000,
                      "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * 2e5 * ns / 1e5}, ns)
    bench.pmc_summary([str(tmp_path / "pass0"), str(tmp_path / "pass1")], "t", out_dir=str(tmp_path))
    text = (tmp_path / "pmc_t.txt").read_text()
    blocks = {b.split("\n")[0]: b for b in text.split("\n\n")[1:]}
    assert "clock 2.00 GHz" in blocks["fa::fwd_h16_kernel<128, false, bf16>"]
    assert "MFMA busy 0.500" in blocks["fa::fwd_h16_kernel<128, false, bf16>"]
    assert "clock" not in blocks["fa::fwd_h16_kernel<64, false, bf16>"]
