"""LDS bank conflicts counted by the hardware, every run ("Shared Memory and
Bank Conflicts", section "see it on your own machine": read the profiler's
shared-memory conflict counter; zero is the target).

tests/lds_counter_run.py launches the default kernel of every workload and
the layout ablation once each, under ``rocprofv3 --pmc``.  The default
kernels must count zero bank conflicts (and zero address conflicts); the
unpadded layout must count conflicts on both the fp32 and the fp16 tile,
and the one-word pad must be conflict-free for fp32 (on the fp16 tile its
packed-pair writes conflict 2-way, which the count must show too)."""
import collections
import csv
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from xpose_testlib import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_INSTS_LDS")


def _rocprofv3():
    exe = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    return exe if os.path.exists(exe) else None


@pytest.fixture(scope="module")
def counts():
    exe = _rocprofv3()
    if exe is None:
        pytest.skip("rocprofv3 not installed")
    with tempfile.TemporaryDirectory(prefix="lds_pmc_") as tmp:
        env = dict(os.environ, TMPDIR="/tmp",
                   PYTHONPATH=os.path.dirname(HERE))
        cmd = ["timeout", "-s", "KILL", "150", exe, "--pmc", *COUNTERS,
               "--output-format", "csv", "-d", tmp, "-o", "lds", "--",
               sys.executable, os.path.join(HERE, "lds_counter_run.py")]
        say("rocprofv3 --pmc " + " ".join(COUNTERS) + " -- lds_counter_run.py")
        out = subprocess.run(cmd, capture_output=True, text=True, cwd="/tmp",
                             env=env, timeout=200)
        tags = [ln.split()[1:] for ln in out.stdout.splitlines()
                if ln.startswith("launch ")]
        files = glob.glob(os.path.join(tmp, "**", "*counter_collection.csv"),
                          recursive=True)
        assert out.returncode == 0 or (out.returncode == 139 and files and
                                       len(tags) == 10), out.stderr[-2000:]
        assert len(files) == 1, files
        per = collections.defaultdict(lambda: collections.Counter())
        names = {}
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                if "xpose::" not in r["Kernel_Name"]:
                    continue
                d = int(r["Dispatch_Id"])
                per[d][r["Counter_Name"]] += float(r["Counter_Value"])
                names[d] = r["Kernel_Name"]
    order = sorted(per)
    assert len(order) == len(tags), (len(order), tags)
    res = {}
    for d, t in zip(order, tags):
        tag = " ".join(t[:2])
        res[tag] = dict(per[d], kernel=names[d], kind=t[2])
        say(f"{tag:12s} {t[2]:5s} {t[3]:8s} " + " ".join(
            f"{c}={int(per[d][c])}" for c in COUNTERS))
    return res


def test_default_kernels_have_no_bank_conflicts(counts):
    for c in ("c1", "c2", "c3", "c4", "c5"):
        r = counts[f"{c} default"]
        assert r["SQ_INSTS_LDS"] > 0, c
        assert r["SQ_LDS_BANK_CONFLICT"] == 0, (c, r)
        assert r["SQ_LDS_ADDR_CONFLICT"] == 0, (c, r)


def test_layout_ablation_counts(counts):
    assert counts["c2 unpadded"]["SQ_LDS_BANK_CONFLICT"] > 0
    assert counts["c4 unpadded"]["SQ_LDS_BANK_CONFLICT"] > 0
    assert counts["c2 pad1"]["SQ_LDS_BANK_CONFLICT"] == 0
    assert counts["c2 swizzle"]["SQ_LDS_BANK_CONFLICT"] == 0
    assert counts["c4 pad1"]["SQ_LDS_BANK_CONFLICT"] > 0
