"""The parts of bench.py that run without a GPU: the one-GPU rule, the
committed HBM-traffic record it reports, and the CPU oracle baseline leg."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_follows_the_kernel_source():
    path = os.path.join(bench.PROFILES, "traffic_training_T4096_H7168_K8_R64.json")
    rec = json.load(open(path)).get("dispatch:dispatch_scatter_kernel")
    got = bench.load_traffic("dispatch.hip", "dispatch:dispatch_scatter_kernel")
    if rec is not None and rec["source_sha"] == bench.kernel_source_sha("dispatch.hip"):
        # measured HBM bytes: the counters scaled by the plain-copy calibration
        exp = int(round((rec["fetch_kib"] * rec["fetch_scale"] +
                         rec["write_kib"] * rec["write_scale"]) * 1024))
        assert abs(got - exp) <= 2048
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None  # counters taken on other code are not reported
    assert bench.load_traffic("dispatch.hip", "no such kernel") is None


def test_cpu_baseline_leg():
    from gen import config_inputs, random_rows
    tr = config_inputs(1)
    dc = config_inputs(3)
    names = ["layout", "dispatch", "dispatch_cached", "combine", "ll_dispatch", "ll_combine"]
    # bytes of the size the bench uses: the rates are rounded to 1 MB/s, and
    # parallel test workers share the one core every leg pins itself to
    out = bench.cpu_baseline(tr, dc, x2_bits=random_rows(tr.T, tr.H, 0, tag=11), budget=0.01,
                             step_bytes=10**12, op_bytes={n: 10**12 for n in names},
                             workloads=(0,))
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["unit"] == "GB/s"
    assert out["value"] > 0 and "whole passes" in out["sample"]
    assert np.isfinite(out["value"])
    assert sorted(out["per_op"]) == sorted(names)
    assert all(v["median_ms"] > 0 and v["gbs"] > 0 for v in out["per_op"].values())
    assert list(out["per_workload"]) == ["tiny"]
    assert all(v > 0 for v in out["per_workload"]["tiny"].values())
    if hasattr(os, "sched_getaffinity"):
        assert len(os.sched_getaffinity(0)) >= 1  # the affinity is restored
