"""bench.py's host-side contract, without a GPU: more than one GPU is
refused with a message, a host without a GPU is reported, and the traffic
summary it reads back parses."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    out = run("--gpus", "2")
    assert out.returncode == 2
    assert "one GPU" in out.stderr and not out.stdout.strip()


def test_bad_step_counts_are_rejected():
    out = run("--steps", "0")
    assert out.returncode != 0 and not out.stdout.strip()


def test_bad_sgemm_shapes_are_rejected():
    for bad in ("1024x1024", "0x5x5", "axbxc"):
        out = run("--sgemm-shapes", bad)
        assert out.returncode == 2 and "--sgemm-shapes" in out.stderr
        assert not out.stdout.strip()


def test_no_gpu_is_reported():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    out = run("--steps", "1", "--warmup", "0")
    assert out.returncode == 1 and "no GPU" in out.stderr


def test_traffic_summary_parses():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    t = bench.read_traffic()
    assert t is None or (isinstance(t, int) and t > 0)
    if t is not None:
        # HBM bytes of one 8192 x 8192 fp32 transpose: close to 2 x 256 MiB
        assert abs(t / (2 * 8192 * 8192 * 4) - 1) < 0.05


def test_traffic_needs_the_profiled_launch():
    """The summary counts only for the launch it was taken on: a config
    naming another tile, order or grid gets no traffic figure."""
    cfg = {"layout": "swizzle", "tile": "128x128", "threads": 256,
           "cache": "nt_store", "tile_order": "diagonal", "occupancy": 1,
           "workgroups": 4096}
    fields = {}
    with open(bench.TRAFFIC_FILE) as f:
        for ln in f:
            if ln.startswith("- ") and ":" in ln:
                k, v = ln[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    assert fields["plan"] == bench.plan_signature(cfg)
    assert bench.read_traffic(cfg) == bench.read_traffic()
    for key, other in (("tile", "256x128"), ("tile_order", "super-tiles 8x32"),
                       ("occupancy", 0), ("workgroups", 2048)):
        assert bench.read_traffic(dict(cfg, **{key: other})) is None, key
