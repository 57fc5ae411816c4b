"""bench.py end to end on the GPU: a short run prints one JSON line that keeps
the reporting contract (every field present, with consistent values)."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_keeps_the_contract():
    sys.__stderr__.write("\n[gpu-test] bench.py --steps 3 --warmup 1 --cpu-seconds 0.5\n")
    sys.__stderr__.flush()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=115, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    b = json.loads(lines[0])

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["unit"] == "GB/s" and b["higher_is_better"] is True and b["data"] == "synthetic"
    assert b["dtype"] == "bf16" and b["vs_baseline"] is None
    cfg = b["config"]
    assert "workload" in cfg and (cfg["T"], cfg["H"], cfg["K"], cfg["R"]) == (4096, 7168, 8, 64)
    assert "model" not in cfg
    # value is the step's algorithmic bytes over its wall time
    assert b["value"] > 0 and b["ms_per_step"] > 0
    expect = cfg["step_bytes"] / (b["ms_per_step"] * 1e-3) / 1e9
    assert abs(b["value"] - expect) <= 0.01 * expect + 1.0

    roof = b["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    N = cfg["N"]
    algo = (4096 + N) * 7168 * 2 + N * 4 + 4096 * 8 * 12 + N * 8 * 12
    assert abs(roof["achieved"] - algo / roof["avg_us"] / 1e3) <= 0.01 * roof["achieved"] + 1.0
    if roof["traffic"] is not None:  # counters taken on the current pack source
        assert abs(roof["traffic"] - algo) <= 0.02 * algo

    # informational parts: the layout with its N readback, the other workloads
    assert b["next"]["layout_with_n_readback"]["avg_us"] > 0
    assert b["next"]["layout_with_n_readback"]["idle_stream_us"] > 0
    for name in ("skewed", "large"):
        wl = b["workloads"][name]
        assert wl["N"] > 0 and wl["combine_gbs"] > 0 and wl["dispatch_cached_gbs"] > 0
    ll = b["workloads"]["ll_large"]
    assert ll["T"] * ll["K"] > 4096 and ll["ll_dispatch_us"] > 0 and ll["ll_combine_us"] > 0
    # every operation beside its same-traffic probe
    ce = b["ceilings"]
    for op, probe in (("dispatch_cached", "pack_probe"), ("combine", "reduce_probe"),
                      ("ll_dispatch", "ll_copy_probe"), ("ll_combine", "ll_reduce_probe")):
        assert ce[op]["avg_us"] > 0 and ce[probe]["avg_us"] > 0
        frac = ce["frac_of_ceiling"][f"{op}_vs_{probe}"]
        assert abs(frac - ce[probe]["avg_us"] / ce[op]["avg_us"]) < 0.01
    assert ce["pack_probe"]["bytes"] == (4096 + N) * 7168 * 2
    for op in ("dispatch_cached", "combine", "ll_dispatch", "ll_combine"):
        assert b["ops"][op]["back_to_back_us"] == ce[op]["avg_us"]

    cpu = b["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["cores"] == 1
    assert cpu["value"] > 0 and cpu["sample"]
    assert sorted(cpu["per_workload"]) == ["large", "skewed", "tiny"]
