"""The benchmark's output contract on the GPU: one JSON line on stdout with the metric, the
whole-job value, the step count and warm-up, the roofline object (HBM-bound, achieved over
peak) and the CPU oracle baseline, for the default workload and the tree-attention path."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_default_line():
    d = bench("--steps", "5", "--warmup", "2", "--cpu-seconds", "1")
    assert d["metric"] == "tree verify+commit draft-nodes*heads/sec"
    assert d["unit"] == "nodes*heads/s" and d["n_gpus"] == 1
    assert d["steps"] == 5 and d["warmup"] == 2 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["B"] == 32 and d["config"]["H"] == 32 and d["config"]["N"] == 4
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert 0.0 < r["frac"] < 1.0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1


def test_attention_line():
    d = bench("--attention", "2048", "--steps", "5", "--warmup", "2", "--cpu-seconds", "0")
    assert d["steps"] == 5 and d["warmup"] == 2 and d["value"] > 0
    assert d["roofline"]["bound"] == "hbm" and 0.0 < d["roofline"]["frac"] < 1.0
