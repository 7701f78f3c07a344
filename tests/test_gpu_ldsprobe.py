"""The LDS microbenchmark against the bank model with the lane groups
measured on gfx950 (GPU).

Measured model (probe timings and SQ_LDS_BANK_CONFLICT): 4-byte words;
32-bit accesses see 32 banks and are resolved per 32-lane half-wave;
64- and 128-bit reads are served 256 bytes per cycle (64 banks, 32 and 16
lanes per group); 64- and 128-bit writes 128 bytes per cycle (32 banks, 16
and 8 lanes per group).  A conflict-free instruction is issue-bound (about
7.5 cycles for a 32-bit read), so only degrees well above 2 show in time;
the checks below use patterns the model calls conflict-free or at least
8-way.  A d-way conflict costs about d cycles for each lane group, so a
pattern the model calls d-way must take at least 3/4 of d * (64 / group)
cycles per instruction.
"""
import pytest

from gfx950_banks import GFX950
from oracle import bankmodel as bm

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
X = pytest.importorskip("lds_tiled_matrix_amd")
from lds_tiled_matrix_amd import ldsprobe  # noqa: E402


def model_degree(width, is_write, lanes):
    banks, group = GFX950[(width, is_write)]
    return bm.conflict_degree(bm.vector_words(lanes, width), banks=banks,
                              group=group)


def test_probe_matches_measured_bank_model():
    assert torch.cuda.is_available()
    buf = torch.zeros(2, dtype=torch.int64, device="cuda")
    base = {}
    for width, name in ((4, "b32 linear"), (8, "b64 linear"), (16, "b128 linear")):
        lanes = dict((n, l) for n, _, l in ldsprobe.PATTERNS)[name]
        for wr in (0, 1):
            base[(width, wr)] = ldsprobe.measure(X, torch, buf, width, lanes, wr, 500)
    checked = 0
    for name, width, lanes in ldsprobe.PATTERNS:
        for wr in (0, 1):
            deg = model_degree(width, wr, lanes)
            cyc = ldsprobe.measure(X, torch, buf, width, lanes, wr, 500)
            ref = base[(width, wr)]
            print(f"{name} {'wr' if wr else 'rd'}: {cyc:.2f} cycles, "
                  f"linear {ref:.2f}, model degree {deg}", flush=True)
            if deg <= 1:
                assert cyc <= 1.3 * ref, name
                checked += 1
            elif deg >= 8:
                group = GFX950[(width, wr)][1]
                assert cyc >= 0.75 * deg * (64 // group), name
                assert cyc > ref, name
                checked += 1
    assert checked >= 20


def test_transpose_gathers_conflict_free_except_unpadded():
    buf = torch.zeros(2, dtype=torch.int64, device="cuda")
    cyc = {lay: ldsprobe.measure(X, torch, buf, 4,
                                 ldsprobe.transpose_gather(lay), 0, 500)
           for lay in ("unpadded", "pad1", "swizzle")}
    for lay in ("pad1", "swizzle"):
        assert model_degree(4, 0, ldsprobe.transpose_gather(lay)) == 1
    assert model_degree(4, 0, ldsprobe.transpose_gather("unpadded")) == 8
    assert abs(cyc["pad1"] - cyc["swizzle"]) <= 0.2 * cyc["swizzle"]
    assert cyc["unpadded"] >= 1.8 * cyc["swizzle"]
