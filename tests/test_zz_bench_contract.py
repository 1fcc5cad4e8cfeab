"""The benchmark script's contract: one GPU only, and the JSON line it prints
(metric, whole-step value, the attention kernel's roofline with its committed
HBM traffic record, the causal form of the headline shape beside it).

The GPU case runs bench.py in a child process with a few steps and no CPU
baseline; it is named to be collected last."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_peaks_and_traffic_record_for_the_current_kernel():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.mfma_peak("fp8") == pytest.approx(5000.0)
    assert bench.mfma_peak("fp16") == pytest.approx(2.0 / (1 / 5000.0 + 1 / 2500.0))
    # the committed counter record belongs to the attention source as it stands
    rec = bench.traffic_record(bench.source_hash(bench.ATTN_SRC), "snippet_b2h32s4096d128", "fp8", False,
                               q_in_attn=True)
    assert rec is not None and rec["hbm_bytes_per_launch"] > 0
    # and a record is never reported for another source
    assert bench.traffic_record("0" * 16, "snippet_b2h32s4096d128", "fp8", False, q_in_attn=True) is None


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    r = subprocess.run([sys.executable, "-u", BENCH, "--steps", "3", "--warmup", "3", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 3 and d["unit"] == "TOPS"
    assert d["config"]["workload"] == "snippet_b2h32s4096d128"
    ops = 4.0 * 2 * 32 * 4096 * 4096 * 128
    assert d["value"] == pytest.approx(ops / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-2)
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == pytest.approx(5000.0)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    assert 0.0 < rf["frac"] < 1.0
    assert rf["traffic"] is not None and rf["traffic"] > 0
    c = d["causal_companion"]
    assert c["causal"] is True and 0.0 < c["frac"] < 1.0
    assert c["value"] == pytest.approx(ops / 2 / (c["ms_per_step"] * 1e-3) / 1e12, rel=1e-2)
