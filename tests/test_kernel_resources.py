"""Resource use of every compiled gfx950 kernel, from the compiler's own
per-kernel summary of a device-only build (no GPU needed): no kernel spills
registers to scratch memory, and each fits the compute unit's 160 KiB of
LDS.  A spill turns register-resident tiles and accumulators into memory
traffic inside the hot loops; an outlined helper that captures them by
reference does the same, so this also guards the forced inlining."""
import os
import re
import subprocess
import tempfile

import pytest

from lds_tiled_matrix_amd import build

SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


@pytest.fixture(scope="module")
def summaries():
    flags = [f for f in build.flags() if f not in ("-shared", "-fPIC")]
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = {}
        for src in SOURCES:
            asm = os.path.join(tmp, src.replace(".hip", ".s"))
            procs[src] = (asm, subprocess.Popen(
                [build.hipcc()] + flags + ["--cuda-device-only", "-S", "-o", asm,
                                           os.path.join(build.CSRC, src)],
                stdout=subprocess.DEVNULL, stderr=subprocess.PIPE))
        for src, (asm, p) in procs.items():
            _, err = p.communicate(timeout=900)
            assert p.returncode == 0, err.decode()[-2000:]
            with open(asm) as f:
                out[src] = f.read()
    return out


def kernels(text):
    """(name, fields) for every kernel in a gfx950 assembly listing."""
    res = []
    for m in re.finditer(r"^(_Z\S+):\s", text, re.M):
        i = text.find("; Kernel info:", m.end())
        if i < 0:
            continue
        lines = []
        for line in text[i:i + 4000].split("\n"):
            if not line.startswith(";"):
                break
            lines.append(line)
        block = "\n".join(lines)
        fields = {k: int(v) for k, v in
                  re.findall(r"; (\w+): (\d+)", block)}
        res.append((m.group(1), fields))
    return res


def test_every_source_has_kernels(summaries):
    for src, text in summaries.items():
        assert len(kernels(text)) > 10, src


def test_no_kernel_spills(summaries):
    for src, text in summaries.items():
        assert all("ScratchSize" in f for _, f in kernels(text)), src
    bad = [(src, name[:90], f["ScratchSize"])
           for src, text in summaries.items()
           for name, f in kernels(text) if f.get("ScratchSize", 0)]
    assert not bad, bad[:10]


def test_lds_fits_a_compute_unit(summaries):
    for src, text in summaries.items():
        for name, f in kernels(text):
            assert f.get("LDSByteSize", 0) <= 160 * 1024, (src, name)
