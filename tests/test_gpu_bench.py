"""bench.py's output contract on the GPU: a short run prints exactly one JSON
line on stdout with the fields and types the measurement protocol fixes, a
roofline whose fraction is its achieved rate over its peak, an oracle CPU
baseline, parity against the oracle, and the SGEMM record."""
import json
import os
import subprocess
import sys

import pytest

from xpose_testlib import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def record():
    say("bench.py --steps 3 --warmup 1 --no-ablation")
    out = subprocess.run(
        [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
         "--warmup", "1", "--no-ablation"],
        capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-3000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines[:3]
    return json.loads(lines[0])


def test_top_level_fields(record):
    r = record
    assert r["metric"] and r["unit"] == "GB/s"
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 1
    assert r["value"] > 0 and r["ms_per_step"] > 0
    assert r["higher_is_better"] is True and r["scaling"] in ("weak", "strong")
    assert r["vs_baseline"] is None
    assert r["dtype"] == "f32" and r["data"] == "synthetic"
    assert "workload" in r["config"] and "model" not in r["config"]
    assert r["config"]["rows"] == 8192 and r["config"]["cols"] == 8192
    # value is whole-job bytes over the wall clock of the timed steps
    assert r["value"] == pytest.approx(
        r["config"]["rw_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, rel=0.02)


def test_roofline(record):
    rf = record["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["achieved"] and rf["frac"] == pytest.approx(
        rf["achieved"] / rf["peak"], abs=1e-3)
    assert rf["traffic"] is None or rf["traffic"] > 0
    # achieved follows the average launch duration of the timed region
    avg = record["timing"]["region_avg_us"]
    assert rf["achieved"] == pytest.approx(
        record["config"]["rw_bytes"] / (avg * 1e-6) / 1e9, rel=2e-3)


def test_cold_roofline(record):
    rc, cold = record["roofline_cold"], record["cold"]
    assert rc["bound"] == "hbm" and rc["unit"] == "GB/s" and rc["peak"] == 8000.0
    assert rc["achieved"] == cold["transpose"]["median_GBps"]
    assert rc["copy"] == cold["copy"]["median_GBps"]
    assert rc["frac"] == pytest.approx(rc["achieved"] / rc["peak"], abs=1e-3)
    assert rc["frac_of_copy"] == pytest.approx(rc["achieved"] / rc["copy"],
                                               abs=1e-3)


def test_cpu_baseline_and_parity(record):
    cb = record["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == "GB/s" and cb["sample"]
    assert record["parity_vs_oracle"] is True


def test_sgemm_record(record):
    sg = record["sgemm"]
    assert sg["m"] == sg["n"] == sg["k"] == 4096
    assert sg["flops"] == 2 * 4096 ** 3
    assert sg["parity_vs_oracle"] is True
    rf = sg["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 157.3
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-3)
    assert sg["cpu_baseline"]["kind"] == "oracle"
    # the small-grid table: the library's split of k where 128 x 128 blocks
    # leave compute units idle, against no split and torch
    rows = {(r["m"], r["n"], r["k"]): r for r in sg["shapes"]}
    assert (1024, 1024, 1024) in rows and rows[(1024, 1024, 1024)]["splits"] > 1
    for r in rows.values():
        assert r["split_TFLOPs"] > 0 and r["no_split_TFLOPs"] > 0
        assert r["torch_addmm_TFLOPs"] > 0 and r["splits"] >= 1
        assert (r["workspace_MiB"] > 0) == (r["splits"] > 1)


def test_sweep_rows():
    """The default-kernel sweep: one row per shape, rates positive, the
    fractions the ratio of the transpose's rate to the copy's."""
    import torch
    import bench
    import lds_tiled_matrix_amd as X
    shapes = ((4, 1024, 2048), (2, 999, 777), (8, 513, 1000), (1, 2048, 4096))
    say(f"bench.bench_sweep {shapes}")
    rows = bench.bench_sweep(X, torch.cuda.Stream(), shapes=shapes, steps=3,
                             cold_reps=2)
    assert [(r["elem_bytes"], r["rows"], r["cols"]) for r in rows] == list(shapes)
    for r in rows:
        assert r["rw_bytes"] == 2 * r["elem_bytes"] * r["rows"] * r["cols"]
        assert r["hot_GBps"] > 0 and r["cold_GBps"] > 0
        assert 0 < r["hot_of_copy"] and 0 < r["cold_of_copy"]
        assert "x" in r["kernel"]
