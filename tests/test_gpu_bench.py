"""bench.py end to end on the GPU, with few steps: one JSON line carrying the
fields of the benchmark contract (metric, value, roofline with its fraction
and traffic, the per-workload figures, the ceilings), with values that are
consistent with each other."""

import json
import os
import subprocess
import sys

import pytest

from conftest import REPO

pytestmark = pytest.mark.gpu


def test_bench_prints_one_contract_line():
    res = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--steps", "3", "--warmup", "2", "--reps",
                          "4", "--min-ms", "0", "--no-cpu-baseline"], capture_output=True, text=True, cwd=REPO,
                         timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "skinny", "workloads", "ceilings"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["unit"] == "TFLOP/s"
    assert d["higher_is_better"] is True and d["dtype"] == "f32" and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 157.3 and r["unit"] == "TFLOP/s"
    assert 0.0 < r["frac"] < 1.0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    # the step is the large-T launch plus the small-T one
    assert r["avg_launch_ms"] < d["ms_per_step"]
    names = [w["workload"] for w in d["workloads"]]
    assert len(names) == 7 and "q4_k_n14336_k4096_t4096" in names and "q4_k_n4096_k14336_t16" in names
    for w in d["workloads"]:
        assert w["avg_launch_us"] > 0 and 0.0 < w["binding_roof_frac"] < 1.0, w
        assert w["event_pairs"]["min_us"] <= w["event_pairs"]["median_us"], w
    c = d["ceilings"]
    assert c["mfma_f32_tflops"] > 100 and c["copy_gbs"] > 1000
    assert 0.0 <= c["mfma_f32_beside_valu"]["serial_frac"] <= 1.2
    # beside the step: the skinny kernel at T = 32 and 64, and the workspace
    # call against retro_out_prod on the 64-slab T = 16 shape
    assert [m["workload"] for m in d["mid_t"]] == ["q4_k_n4096_k14336_t32", "q4_k_n4096_k14336_t64"]
    for m in d["mid_t"]:
        assert m["kernel"] == "skinny" and 0.0 < m["f32_mfma_frac"] < 1.0, m
    sp = d["skinny_split"]
    assert sp["slabs_of_dst"] == 64 and sp["workspace_bytes"] > 0
    assert sp["speedup"] > 1.0 and sp["workspace"]["avg_launch_us"] < sp["skinny"]["avg_launch_us"]
