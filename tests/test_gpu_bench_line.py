"""bench.py end to end on the GPU: a short run prints one JSON line with the fields the measurement contract
asks for (metric, value, roofline, the oracle's CPU baseline)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_complete_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--cpu-budget", "2", "--no-secondary", "--prewarm", "0.05"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["value"] > 0
    assert d["config"]["workload"] == "decode_qwen3_0p6b"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the measured traffic comes from the committed counter summary taken on the kernels' current code: a kernel
    # change without new counters leaves it null, and that is a failure (the counters must be taken again)
    assert roof["traffic"] is not None, "stale or missing HBM counter summary for the decode kernels"
    assert roof["traffic"] > roof["bytes_per_launch"] * 0.9
    # the roofline's kernel time is the attention call alone, which is part of the step
    assert roof["launch_ms"] <= d["ms_per_step"] * 1.02
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
