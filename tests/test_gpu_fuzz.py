"""Seeded random cases through the C ABI against the oracle (GPU): random
shapes, pitches, batch strides, pointer offsets, element sizes and every
launch option, so that option interactions no targeted test names are
still checked bit for bit."""
import random

import pytest

from xpose_testlib import DTYPE_OF_SIZE, check_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
X = pytest.importorskip("lds_tiled_matrix_amd")

TILES = ((32, 32), (64, 64), (128, 64), (64, 128), (128, 128), (32, 64),
         (64, 32), (16, 16), (256, 128), (256, 256))


def random_opts(rng, s):
    """A random valid option set for element size s (None = defaults)."""
    if rng.random() < 0.25:
        return None
    for _ in range(50):
        layout = rng.choice((0, 1, 2, 3, 3, 3, 4, 5))
        tile = rng.choice(TILES + (None,))
        flags = rng.choice((0, 0, X.FLAG_XCD_REMAP, X.FLAG_NO_XCD_REMAP,
                            X.FLAG_ELEMENTWISE, X.FLAG_DIRECT_LDS))
        cache = rng.choice((0, 1, 2))
        order = rng.choice((0, 1, 2))
        gr, gc = rng.choice(((0, 0), (1, 0), (3, 5), (8, 32), (1000, 2)))
        persistent = rng.choice((0, 0, 0, 1, 2))
        occupancy = 0 if persistent else rng.choice((0, 0, 0, 1, 2, 3, -1))
        opts = X.make_opts(layout, tile, flags, cache, gr, gc, 0, order,
                           persistent, occupancy)
        rc, _ = X.xpose_plan(0x100000, 0x40000000, 1, 64, 64, 64, 64, 0, 0,
                             DTYPE_OF_SIZE[s], opts)
        if rc == 0:
            return opts
    return None


@pytest.mark.parametrize("seed", range(6))
def test_random_cases(seed):
    rng = random.Random(1000 + seed)
    for case in range(25):
        s = rng.choice((1, 2, 4, 8))
        batch = rng.choice((1, 1, 1, 2, 5))
        rows = rng.choice((1, rng.randint(1, 40), rng.randint(1, 700),
                           rng.randint(100, 1500)))
        cols = rng.choice((1, rng.randint(1, 40), rng.randint(1, 700),
                           rng.randint(100, 1500)))
        ld_in = cols + rng.choice((0, 0, 1, 3, 16, 37))
        ld_out = rows + rng.choice((0, 0, 1, 2, 32, 41))
        stride_in = rows * ld_in + rng.choice((0, 0, 5, 64))
        stride_out = cols * ld_out + rng.choice((0, 0, 3, 128))
        opts = random_opts(rng, s)
        check_case(s, batch, rows, cols, ld_in=ld_in, ld_out=ld_out,
                   stride_in=stride_in, stride_out=stride_out,
                   seed=seed * 100 + case, opts=opts,
                   in_shift=rng.choice((0, 0, 1, 3)),
                   out_shift=rng.choice((0, 0, 1, 2)),
                   label=f"fuzz {seed}/{case}")


TR_TILES = {2: ((64, 64), (128, 64), (64, 128), (128, 128), (64, 32), None),
            1: ((128, 128), (64, 128), (128, 64), (128, 256), None)}


@pytest.mark.parametrize("seed", range(4))
def test_random_tr_cases(seed):
    """The same kind of random cases through the LDS transpose-read tiles."""
    rng = random.Random(2000 + seed)
    for case in range(25):
        s = rng.choice((1, 2))
        opts = None
        for _ in range(50):
            flags = X.FLAG_TR_READ | rng.choice(
                (0, 0, X.FLAG_DIRECT_LDS, X.FLAG_ELEMENTWISE, X.FLAG_XCD_REMAP,
                 X.FLAG_NO_XCD_REMAP | X.FLAG_DIRECT_LDS))
            gr, gc = rng.choice(((0, 0), (1, 0), (3, 5), (8, 32)))
            cand = X.make_opts(X.LAYOUT_SWIZZLE, rng.choice(TR_TILES[s]), flags,
                               rng.choice((0, 1, 2)), gr, gc, 0,
                               rng.choice((0, 1, 2)))
            if X.xpose_plan(0x100000, 0x40000000, 1, 64, 64, 64, 64, 0, 0,
                            DTYPE_OF_SIZE[s], cand)[0] == 0:
                opts = cand
                break
        assert opts is not None
        batch = rng.choice((1, 1, 2, 4))
        rows = rng.choice((rng.randint(1, 70), rng.randint(1, 900),
                           rng.randint(200, 1500)))
        cols = rng.choice((rng.randint(1, 70), rng.randint(1, 900),
                           rng.randint(200, 1500)))
        ld_in = cols + rng.choice((0, 0, 1, 4, 16, 37))
        ld_out = rows + rng.choice((0, 0, 2, 4, 32, 41))
        stride_in = rows * ld_in + rng.choice((0, 0, 4, 64))
        stride_out = cols * ld_out + rng.choice((0, 0, 8, 128))
        check_case(s, batch, rows, cols, ld_in=ld_in, ld_out=ld_out,
                   stride_in=stride_in, stride_out=stride_out,
                   seed=seed * 100 + case, opts=opts,
                   in_shift=rng.choice((0, 0, 1, 2, 4)),
                   out_shift=rng.choice((0, 0, 2, 4)),
                   label=f"tr fuzz {seed}/{case}")


SHIFT_TILES = {2: ((64, 64), (128, 64), (256, 64)),
               4: ((64, 64), (128, 64), (256, 64), (128, 32), (64, 32),
                   (64, 128), (128, 128), (256, 128)),
               8: ((32, 32), (64, 32), (64, 64))}


def campaign_opts(rng, s):
    """Any launch option set: the generic random options, transpose-read
    tiles (1- and 2-byte elements) or line-aligned output tiles (2-, 4- and
    8-byte elements), or the defaults."""
    r = rng.random()
    if r < 0.4:
        return random_opts(rng, s)
    cands = []
    if r < 0.6 and s in (1, 2):
        for _ in range(50):
            fl = X.FLAG_TR_READ | rng.choice((0, X.FLAG_DIRECT_LDS, X.FLAG_ELEMENTWISE,
                                              X.FLAG_XCD_REMAP))
            cands.append(X.make_opts(X.LAYOUT_SWIZZLE, rng.choice(TR_TILES[s]), fl,
                                     rng.choice((0, 1, 2)),
                                     *rng.choice(((0, 0), (1, 0), (3, 5), (8, 32))), 0,
                                     rng.choice((0, 1, 2))))
    elif r < 0.85 and s in SHIFT_TILES:
        for _ in range(50):
            # persistent: line-aligned tiles in column strips of that many
            # tile rows (built for 4- and 8-byte elements)
            strip = rng.choice((0, 0, 0, 1, 2, 3, 8))
            cands.append(X.make_opts(X.LAYOUT_SWIZZLE, rng.choice(SHIFT_TILES[s] + (None,)),
                                     X.FLAG_ALIGN_OUT | rng.choice((0, 2, 4)),
                                     rng.choice((0, 1, 2)),
                                     *rng.choice(((0, 0), (1, 0), (3, 5), (16, 16),
                                                  (128, 4))), 0,
                                     rng.choice((0, 1, 2, 3)), strip,
                                     0 if strip else rng.choice((0, 0, 2, 4))))
    for o in cands:
        if X.xpose_plan(0x100000, 0x40000000, 1, 64, 64, 64, 64, 0, 0,
                        DTYPE_OF_SIZE[s], o)[0] == 0:
            return o
    return None


@pytest.mark.parametrize("chunk", range(4))
def test_random_campaign(chunk):
    """25 seeds x 25 cases per chunk over every option family, pitches and
    pointer offsets at every residue (one-off runs of 1,260 seeds of the
    generator before the 128 KiB tiles and column strips joined it, of
    seeds 100-699, 15,000 cases, before the wider line-aligned tiles joined
    it, and of seeds 100-6599 and 10600-30599, 662,500 cases, of this one
    also passed)."""
    for seed in range(chunk * 25, chunk * 25 + 25):
        rng = random.Random(50000 + seed)
        for case in range(25):
            s = rng.choice((1, 2, 4, 8))
            batch = rng.choice((1, 1, 1, 2, 3))
            rows = rng.choice((1, rng.randint(1, 80), rng.randint(1, 900),
                               rng.randint(200, 2000)))
            cols = rng.choice((1, rng.randint(1, 80), rng.randint(1, 900),
                               rng.randint(200, 2000)))
            ld_in = cols + rng.choice((0, 0, 1, 2, 3, 5, 16, 37, 64))
            ld_out = rows + rng.choice((0, 0, 1, 2, 3, 7, 32, 41, 64))
            stride_in = rows * ld_in + rng.choice((0, 0, 5, 64, 3))
            stride_out = cols * ld_out + rng.choice((0, 0, 3, 128, 1))
            check_case(s, batch, rows, cols, ld_in=ld_in, ld_out=ld_out,
                       stride_in=stride_in, stride_out=stride_out,
                       seed=seed * 100 + case, opts=campaign_opts(rng, s),
                       in_shift=rng.choice((0, 0, 1, 2, 3)),
                       out_shift=rng.choice((0, 0, 1, 2, 5)),
                       label=f"campaign {seed}/{case}")
