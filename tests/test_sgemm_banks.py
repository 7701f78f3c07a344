"""Bank behaviour of the SGEMM kernel's LDS accesses, on the CPU: a host
program built from the kernel's own geometry (sgemm_lanes.h) lists the LDS
address of every lane in every LDS instruction, and the pages' bank model
(oracle.bankmodel) with gfx950's measured geometry prices each one.

What the pages derive for 32 banks ("Padded Shared Memory: Eliminating Bank
Conflicts", sections "How Shared Memory Is Addressed" and "The Fix Is One
Constant") must come out for the gfx950 kernel too, since gfx950 serves
4-byte accesses 32 lanes at a time over 32 banks: with As's row stride a
multiple of 32 the transposed store is (bk / 4)-way conflicted (2-way at
bk = 8, 4-way at bk = 16; A's tile is read in strips of at most 32 columns,
so 8-way at bk = 32 and 64); the padded stride and the swizzle make it
conflict-free; the product's reads and B's 16-byte copies are conflict-free
in every layout.  The host program also checks that each layout stores every
element of the tile exactly once and that the block order is a bijection."""
import collections
import os
import subprocess
import tempfile

import pytest

from gfx950_banks import degree

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def listing():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "sgemm_lds")
        subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17",
                        "--offload-arch=gfx950", "-o", exe,
                        os.path.join(HERE, "native", "sgemm_lds.cpp")],
                       check=True, capture_output=True, timeout=300)
        return subprocess.run([exe], capture_output=True, text=True,
                              timeout=120, check=True).stdout.splitlines()


@pytest.fixture(scope="module")
def worst(listing):
    res = collections.defaultdict(int)
    for line in listing:
        f = line.split()
        if f[0] != "lds":
            continue
        name, phase, width, wr = f[1], f[2], int(f[3]), int(f[4])
        res[(name, phase)] = max(res[(name, phase)],
                                 degree(width, wr, [int(x) for x in f[5:]]))
    return dict(res)


def test_self_checks_pass(listing):
    checks = [ln.split() for ln in listing if ln.startswith("check ")]
    assert len(checks) > 18 * 4
    bad = [c for c in checks if c[2] != "ok"]
    assert not bad, bad[:5]


@pytest.mark.parametrize("bk, m", [(8, ""), (16, ""), (32, ""), (64, ""),
                                   (16, "/m256"), (32, "/m256"), (16, "/m64")])
def test_transposed_store(worst, bk, m):
    assert worst[(f"sgemm/bk{bk}/unpadded{m}", "a_store")] == min(bk, 32) // 4
    assert worst[(f"sgemm/bk{bk}/padded{m}", "a_store")] == 1
    assert worst[(f"sgemm/bk{bk}/swizzle{m}", "a_store")] == 1


def test_reads_and_b_copies_conflict_free(worst):
    for (name, phase), d in worst.items():
        if phase != "a_store":
            assert d == 1, (name, phase, d)


def test_every_built_kernel_listed(worst):
    names = {n for n, _ in worst}
    layouts = ("unpadded", "padded", "swizzle")
    assert names == ({f"sgemm/bk{bk}/{l}" for bk in (8, 16, 32, 64) for l in layouts} |
                     {f"sgemm/bk{bk}/{l}/m256" for bk in (16, 32) for l in layouts} |
                     {f"sgemm/bk16/{l}/m64" for l in layouts})
