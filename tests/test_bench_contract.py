"""bench.py's output contract: one JSON line with the fields the benchmark
driver reads, and a refusal of more than one GPU.

The benchmark runs as a child process (as the driver runs it); the GPU case
uses the tiny fp32 recipe and a few iterations so it takes seconds.
"""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line():
    cmd = [sys.executable, BENCH, "--workload", "tiny_f32", "--steps", "3", "--warmup", "1",
           "--cpu-batches", "1", "--baselines", "0", "--tol-run", "0"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["unit"] == "iter/s" and j["higher_is_better"] is True
    assert j["scaling"] == "weak" and j["vs_baseline"] is None
    assert j["dtype"] == "f32" and j["data"] == "synthetic"
    assert j["config"]["workload"].startswith("tiny_f32")
    assert j["value"] > 0 and j["ms_per_step"] > 0
    # value is iterations per second over the same timed region
    assert math.isclose(j["value"], 1e3 / j["ms_per_step"], rel_tol=1e-6)
    rf = j["roofline"]
    assert rf["bound"] in ("mfma", "hbm", "alu")
    assert rf["unit"] in ("TFLOP/s", "GB/s")
    assert rf["achieved"] > 0 and rf["peak"] > 0
    assert math.isclose(rf["frac"], rf["achieved"] / rf["peak"], rel_tol=1e-6)
    assert "traffic" in rf
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == "iter/s" and cb["sample"]
