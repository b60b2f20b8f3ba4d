"""The benchmark's output contract on the GPU: one JSON line on stdout with the metric, the
whole-job value, the step count and warm-up, the roofline object (HBM-bound, achieved over
peak) and the CPU oracle baseline, for the default workload (configuration 3), for
configuration 4 with the store-all scheme timed beside it, and for the tree-attention path."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*args, timeout=480):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def check_line(d, steps, warmup):
    assert d["metric"] == "tree verify+commit draft-nodes*heads/sec"
    assert d["unit"] == "nodes*heads/s" and d["n_gpus"] == 1
    assert d["steps"] == steps and d["warmup"] == warmup and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert 0.0 < r["frac"] < 1.0
    # no kernel duration in the line is longer than the step it is part of
    assert all(0.0 < t <= d["ms_per_step"] * 1e3 for t in d["kernels_us"].values())
    assert r["launch_us"] <= d["ms_per_step"] * 1e3
    assert d["copy_gbs"] is None or 0.0 < d["copy_gbs"] < 16000.0


def test_default_line():
    # the default workload: B128 x H32, 64-node trees, 30 layers (the largest one-GPU workload)
    d = bench("--steps", "3", "--warmup", "2", "--cpu-seconds", "1")
    check_line(d, 3, 2)
    cfg = d["config"]
    assert (cfg["B"], cfg["H"], cfg["N"], cfg["layers"]) == (128, 32, 64, 30)
    assert "B128 x H32" in cfg["workload"] and "30 layers" in cfg["workload"]
    assert d["roofline"]["kernel"] == "treewy_commit_verify"
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert c["threads"] == c["cores"] and c["host_cores"] >= c["threads"]
    assert isinstance(c["cpu_model"], str) and c["cpu_model"]


def test_config4_line_times_snapshots_beside():
    # configuration 4: the store-all scheme is timed on the same inputs in the same run
    d = bench("--config", "4", "--steps", "3", "--warmup", "2", "--cpu-seconds", "0",
              "--copy-gib", "0")
    check_line(d, 3, 2)
    assert (d["config"]["B"], d["config"]["H"], d["config"]["N"]) == (256, 64, 32)
    s = d["snapshot"]
    assert s["ms_per_step"] > 0 and s["bytes_per_step"] > 0 and s["achieved_gbs"] > 0
    assert set(s["kernels_us"]) == {"treewy_verify_snapshot", "treewy_commit_snapshot"}
    # the snapshots alone are B*H*N states of 64 KiB, far more than TreeWY moves
    assert s["bytes_per_step"] > 256 * 64 * 32 * 65536
    assert s["bytes_vs_treewy"] > 5.0


def test_attention_line():
    d = bench("--attention", "2048", "--steps", "5", "--warmup", "2", "--cpu-seconds", "0")
    assert d["steps"] == 5 and d["warmup"] == 2 and d["value"] > 0
    assert d["roofline"]["bound"] == "hbm" and 0.0 < d["roofline"]["frac"] < 1.0
