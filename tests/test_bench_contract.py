"""The benchmark's output contract: one JSON line with the metric, the roofline and the CPU
baseline fields, and a refusal (not a silent one-GPU run) when more than one GPU is asked for."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line_on_the_tiny_workload():
    cmd = [sys.executable, "-u", BENCH, "--config", "1", "--steps", "2", "--warmup", "1", "--no-extra",
           "--no-cpu-baseline", "--no-clock"]
    print("bench child:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny_4x8x8"
    assert d["cpu_baseline"] is None  # skipped on request
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["kernel"] == "attn_fwd_kernel<64,8,2> (dense)"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    # the committed memory counters belong to the 5 s workload: none for this one
    assert roof["traffic"] is None
    # achieved = algorithmic flops per launch / the launch's average duration
    flops = 4.0 * 1 * 2 * 256 * 256 * 64
    assert roof["per_launch_flops"] == flops
    assert abs(roof["achieved"] - flops / (roof["avg_launch_ms"] * 1e-3) / 1e12) < 1e-9 * roof["achieved"]
