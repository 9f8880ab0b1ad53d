"""The benchmark's output contract on the GPU: a short `bench.py` run (one
timed step, no extra section, no CPU baseline) prints exactly one JSON line
on stdout with the fields the measurement reports rely on, consistent with
each other (the decode roofline's achieved rate is bytes over its mean
duration and below the peak; value is the step's KV bytes over its time)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_consistent_json_line():
    print("bench.py --steps 1 --warmup 1 --no-extra --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "1",
                        "--no-extra", "--no-cpu-baseline"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "decode_118750x48"
    # value: 48 layers x 118,750 cells x 816 B per step over the step's time
    step_bytes = 48 * 118750 * 816
    assert d["value"] == pytest.approx(step_bytes / (d["ms_per_step"] * 1e-3) / 1e9, rel=2e-3)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["bytes_per_launch"] == 118750 * 816
    assert rf["achieved"] == pytest.approx(rf["bytes_per_launch"] / (rf["mean_us"] * 1e-6) / 1e9, rel=2e-3)
    assert 0 < rf["frac"] < 1 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    # a decode launch cannot take longer than a layer's share of the step
    assert rf["mean_us"] * 48 <= d["ms_per_step"] * 1e3 * 1.3
    sp = rf["spread"]
    assert sp["launches"] == 96 and 0 < sp["p10_us"] <= sp["median_us"] <= sp["p90_us"]
    if rf["traffic"] is not None:
        assert rf["traffic_bytes_per_launch"] >= rf["bytes_per_launch"]
