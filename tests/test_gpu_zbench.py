"""bench.py's output contract on the GPU: one JSON line with the metric, the
step time, the roofline object and the CPU-oracle baseline (the tiny
workload, a few steps, in a child process)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line(gpu_lib):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "tiny_fp32", "--steps", "3",
           "--warmup", "1", "--cpu-budget", "1", "--no-read-probe"]
    print("case bench tiny_fp32 3 steps", flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "GB/s" and d["dtype"] == "fp32" and d["config"]["workload"] == "tiny_fp32"
    r = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] in ("hbm", "mfma") and r["achieved"] > 0
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)   # printed to 4 decimals
    c = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in c, k
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
