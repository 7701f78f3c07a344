"""Bank conflicts of every built tile kernel, on the CPU: a host program
built from the kernels' own lane maps and LDS layouts
(lds_tiled_matrix_amd/csrc/xpose_lanes.h) lists the LDS address of every
lane in every LDS instruction of every wave, and the bank model of the
pages (oracle.bankmodel), with the bank geometry measured on gfx950,
prices each instruction.

The swizzled layouts must be conflict-free in every built shape (the one
exception, stated with the kernel: direct loads into transpose-read tiles,
2-way); the one-word pad is conflict-free for 4-byte elements; the unpadded
layout shows the column-walk conflict the ablation is there to show."""
import collections
import os
import subprocess
import tempfile

import pytest

from gfx950_banks import degree

X = pytest.importorskip("lds_tiled_matrix_amd")

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def worst():
    """(kernel name, phase) -> worst conflict degree over its instructions."""
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "lds_addresses")
        subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17",
                        "--offload-arch=gfx950", "-o", exe,
                        os.path.join(HERE, "native", "lds_addresses.cpp")],
                       check=True, capture_output=True, timeout=300)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                             check=True).stdout
    res = collections.defaultdict(int)
    for line in out.splitlines():
        f = line.split()
        name, phase, width, wr = f[0], f[1], int(f[2]), int(f[3])
        d = degree(width, wr, [int(a) for a in f[4:]])
        res[(name, phase)] = max(res[(name, phase)], d)
    assert len(res) > 100
    return dict(res)


def kernels(worst):
    return sorted({k for k, _ in worst})


def test_swizzled_layouts_are_conflict_free(worst):
    for (name, phase), d in worst.items():
        if name.endswith("/swizzle"):
            assert d == 1, (name, phase, d)


def test_direct_transpose_read_tiles_are_two_way(worst):
    direct = [(k, p) for k, p in worst if k.startswith("tr/") and k.endswith("/direct")]
    assert direct
    for k, p in direct:
        assert worst[(k, p)] == 2, k


def test_pad_and_unpadded_ablation(worst):
    for (name, phase), d in worst.items():
        if name.startswith("tile/s4/") and name.endswith("/pad1"):
            assert d == 1, (name, phase)
        if name.startswith("tile/s4/") and name.endswith("/unpadded") and phase == "read":
            assert d == 8, name  # the 8 row groups of one column share a bank


def test_line_aligned_tiles_every_pitch(worst):
    shift = [k for k in kernels(worst) if k.startswith("shift/")]
    assert len(shift) == 14
    for k in shift:
        assert worst[(k, "read")] == 1 and worst[(k, "write")] == 1


def _probe(s, tr, tc, nt, layout, flags):
    code = {1: X.XPOSE_U8, 2: X.XPOSE_F16, 4: X.XPOSE_F32, 8: X.XPOSE_F64}[s]
    opts = X.make_opts(layout, (tr, tc), flags, X.CACHE_AUTO, 0, 0, nt)
    rc, info = X.xpose_plan(1 << 40, 1 << 44, 1, 1024, 1024, 1024, 1024, 0, 0,
                            code, opts)
    return rc == 0 and info.threads == nt


def test_enumerated_shapes_are_the_built_ones(worst):
    """The host program covers exactly the kernels the library has."""
    names = set(kernels(worst))
    lay = {"unpadded": X.LAYOUT_UNPADDED, "pad1": X.LAYOUT_PAD1,
           "swizzle": X.LAYOUT_SWIZZLE}
    for n in names:
        kind, s, shape, nt, variant = n.split("/")
        s, nt = int(s[1:]), int(nt)
        tr, tc = map(int, shape.split("x"))
        if kind == "tile":
            assert _probe(s, tr, tc, nt, lay[variant], X.FLAG_NO_ALIGN_OUT), n
        elif kind == "shift":
            assert _probe(s, tr, tc, nt, X.LAYOUT_SWIZZLE, X.FLAG_ALIGN_OUT), n
        else:
            fl = X.FLAG_TR_READ | (X.FLAG_DIRECT_LDS if variant == "direct" else 0)
            assert _probe(s, tr, tc, nt, X.LAYOUT_SWIZZLE, fl), n
    dims = (16, 32, 64, 128, 256)
    for s in (1, 2, 4, 8):
        for tr in dims:
            for tc in dims:
                for nt in (64, 128, 256):
                    for v, l in lay.items():
                        for extra in (0, X.FLAG_DIRECT_LDS):
                            if _probe(s, tr, tc, nt, l, X.FLAG_NO_ALIGN_OUT | extra):
                                assert f"tile/s{s}/{tr}x{tc}/{nt}/{v}" in names
                    if _probe(s, tr, tc, nt, X.LAYOUT_SWIZZLE, X.FLAG_ALIGN_OUT):
                        assert f"shift/s{s}/{tr}x{tc}/{nt}/swizzle" in names
                    for v, fl in (("swizzle", 0), ("direct", X.FLAG_DIRECT_LDS)):
                        if _probe(s, tr, tc, nt, X.LAYOUT_SWIZZLE, X.FLAG_TR_READ | fl):
                            assert f"tr/s{s}/{tr}x{tc}/{nt}/{v}" in names


def _packed_worst(rows, cols, s, pad, block=16384):
    """Worst conflict degree of the packed kernel's gathers: lane l of a wave
    builds output vector v = base + l, whose element x is input element
    g m + i cols + j of the block, held at LDS element g mp + i cs + j
    (cs = cols + pad, mp = rows cs); the reads are s-byte (8-byte units for
    f64, else the 4-byte word holding the element)."""
    v_el = 16 // s
    m = rows * cols
    n = max(1, block // (m * s)) * m
    cs, mp = cols + pad, rows * (cols + pad)
    width = 8 if s == 8 else 4
    worst = 1
    for base in range(0, min(n // v_el, 1024), 64):
        for x in range(v_el):
            addrs = []
            for lane in range(64):
                o = (base + lane) * v_el + x
                if o >= n:
                    addrs.append(-1)
                    continue
                g, t = divmod(o, m)
                j, i = divmod(t, rows)
                addrs.append((g * mp + i * cs + j) * s // width * width)
            worst = max(worst, degree(width, 0, addrs))
    return worst


def test_packed_padding_spreads_column_reads():
    """Rows of 64 bytes or a multiple get one word of padding (8 bytes for
    f64) per row; it takes the worst gather of every such shape down to
    4-way at most, from up to 32-way."""
    before = after = 0
    for s in (1, 2, 4, 8):
        pad = 1 if s == 8 else 4 // s
        for rows, cols in ((16, 16), (32, 32), (128, 32), (64, 64), (32, 128),
                           (64, 16), (16, 64), (128, 128), (16, 128)):
            if (cols * s) % 64 or rows * cols * s > 16384:
                continue
            u, p = _packed_worst(rows, cols, s, 0), _packed_worst(rows, cols, s, pad)
            assert p <= 4 and p <= u, (s, rows, cols, u, p)
            before, after = max(before, u), max(after, p)
    assert before == 32 and after == 4
