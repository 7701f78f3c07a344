"""GPU parity of the tiled SGEMM (xpose_sgemm*, include/xpose_sgemm.h)
against the oracle (oracle/sgemm.py), through the C ABI.

* Integer-valued inputs keep every partial sum exact in float32, so there
  the GPU must equal the oracle bit for bit, whatever the summation order.
* Uniform [-1, 1) inputs are compared within the fp32 dot-product bound
  (k + 3) * 2^-24 * (|alpha| |A| |B| + |beta| |C|), elementwise.
* The m x n region is the only thing written: pitch padding and guard
  bands around C keep their sentinels.
* Every As layout, k step and load path sums in the same order (k pairs in
  sequence), so all kernels must agree bit for bit with each other."""
import numpy as np
import pytest

import oracle.sgemm as og
import workloads as wl
from xpose_testlib import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
X = pytest.importorskip("lds_tiled_matrix_amd")

GUARD = 64
SENTINEL = np.float32(-12345.5)
LAYOUTS = (X.AS_UNPADDED, X.AS_PADDED, X.AS_SWIZZLE)
BKS = (8, 16, 32, 64)


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _flat(M, ld, fill):
    rows, cols = M.shape
    buf = np.full(max(rows * ld, 1), fill, dtype=np.float32)
    for i in range(rows):
        buf[i * ld:i * ld + cols] = M[i]
    return buf


def _upload(buf, shift):
    """Device copy of a flat buffer starting `shift` floats into a fresh
    allocation (shift 1: 4-byte but not 16-byte aligned)."""
    d = torch.empty(shift + buf.size, dtype=torch.float32, device=_dev())
    d[shift:].copy_(torch.from_numpy(buf))
    return d, d.data_ptr() + 4 * shift


def run_case(A, B, C, alpha, beta, pads=(0, 0, 0), shifts=(0, 0, 0),
             opts=None, stream=None, entry="ex", ws_bytes=None, ws_shift=0,
             want_splits=None):
    """Run the library; return (C buffer as read back, flat C buffer before,
    ldc).  Both buffers include GUARD sentinels on each side.  entry "ws":
    xpose_sgemm_ws with a workspace of ws_bytes (None: what the plan wants)
    starting ws_shift floats into an allocation, NaN-filled (a partial sum
    the split failed to write would reach C as NaN) and followed by GUARD
    sentinels that must stay unchanged."""
    m, k = A.shape
    n = B.shape[1]
    lda, ldb, ldc = max(k, 1) + pads[0], max(n, 1) + pads[1], max(n, 1) + pads[2]
    a = _flat(A, lda, np.nan)
    b = _flat(B, ldb, np.nan)
    c_body = _flat(C, ldc, SENTINEL)
    c_full = np.concatenate([np.full(GUARD, SENTINEL, np.float32), c_body,
                             np.full(GUARD, SENTINEL, np.float32)])
    da, pa = _upload(a, shifts[0])
    db, pb = _upload(b, shifts[1])
    dc, pc0 = _upload(c_full, shifts[2])
    pc = pc0 + 4 * GUARD
    sh = 0 if stream is None else int(stream.cuda_stream)
    say(f"sgemm m={m} n={n} k={k} pads={pads} shifts={shifts} "
        f"opts={None if opts is None else (opts.layout, opts.bk, opts.flags, opts.tile_m)}")
    if entry == "plain":
        rc = X.xpose_sgemm(m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc, sh)
    elif entry == "ws":
        if ws_bytes is None:
            prc, info = X.xpose_sgemm_plan_ws(m, n, k, pa, lda, pb, ldb, pc,
                                              ldc, opts, 1 << 40, 1 << 50)
            assert prc == 0, X.strerror(prc)
            ws_bytes = info.workspace_wanted
        nws = ws_bytes // 4
        dw = torch.full((ws_shift + nws + GUARD,), float("nan"),
                        dtype=torch.float32, device=_dev())
        dw[ws_shift + nws:] = float(SENTINEL)
        pw = dw.data_ptr() + 4 * ws_shift
        prc, info = X.xpose_sgemm_plan_ws(m, n, k, pa, lda, pb, ldb, pc, ldc,
                                          opts, pw, ws_bytes)
        assert prc == 0, X.strerror(prc)
        if want_splits is not None:
            assert info.splits == want_splits, (info.splits, want_splits)
        assert info.workspace_bytes <= ws_bytes
        say(f"  ws splits={info.splits} split_len={info.split_len} "
            f"bytes={info.workspace_bytes} shift={ws_shift}")
        rc = X.xpose_sgemm_ws(m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc,
                              opts, pw, ws_bytes, sh)
        torch.cuda.synchronize()
        tail = dw[ws_shift + nws:].cpu().numpy()
        assert np.array_equal(tail.view(np.uint32),
                              np.full(GUARD, SENTINEL).view(np.uint32))
    else:
        rc = X.xpose_sgemm_ex(m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc,
                              opts, sh)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    got = dc[shifts[2]:].cpu().numpy()
    return got, c_full, (a, lda, b, ldb, ldc)


def expected(A, B, C, alpha, beta, c_full, bufs):
    """Oracle result written into a copy of the C buffer (float32)."""
    a, lda, b, ldb, ldc = bufs
    m, k = A.shape
    n = B.shape[1]
    out = c_full.copy()
    body = out[GUARD:out.size - GUARD]
    og.sgemm_into(m, n, k, alpha, a, lda, b, ldb, beta, body, ldc)
    return out


def region_mask(m, n, ldc, size):
    mask = np.zeros(size, dtype=bool)
    for i in range(m):
        mask[GUARD + i * ldc:GUARD + i * ldc + n] = True
    return mask


def check_exact(A, B, C, alpha, beta, **kw):
    """Exact equality in the m x n region (an exact zero sum may come out as
    +0 or -0 depending on the order of the terms, so zeros compare by value),
    bit equality everywhere else (pitch padding and guards untouched)."""
    got, c_full, bufs = run_case(A, B, C, alpha, beta, **kw)
    exp = expected(A, B, C, alpha, beta, c_full, bufs)
    m, n = A.shape[0], B.shape[1]
    mask = region_mask(m, n, bufs[4], got.size)
    bad = np.flatnonzero(mask & (got != exp))
    assert bad.size == 0, (bad[:8], got[bad[:8]], exp[bad[:8]])
    outside = np.flatnonzero(~mask & (got.view(np.uint32) != exp.view(np.uint32)))
    assert outside.size == 0, outside[:8]
    return got


def check_bound(A, B, C, alpha, beta, **kw):
    got, c_full, bufs = run_case(A, B, C, alpha, beta, **kw)
    m, k = A.shape
    n = B.shape[1]
    ldc = bufs[4]
    ref = og.sgemm(m, n, k, alpha, bufs[0], bufs[1], bufs[2], bufs[3], beta,
                   c_full[GUARD:c_full.size - GUARD], ldc)
    mag = abs(alpha) * (np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)))
    if beta != 0:
        mag += abs(beta) * np.abs(C.astype(np.float64))
    tol = (k + 3) * 2.0 ** -24 * mag
    mask = region_mask(m, n, ldc, got.size)
    g = got[mask].reshape(m, n).astype(np.float64)
    err = np.abs(g - ref)
    assert (err <= tol).all(), (err.max(), np.unravel_index(np.argmax(err - tol), err.shape))
    # nothing outside the m x n region changed
    assert np.array_equal(got[~mask].view(np.uint32), c_full[~mask].view(np.uint32))
    return got


EXACT_SHAPES = [(128, 128, 16), (256, 384, 512), (130, 67, 45), (1, 1, 1),
                (300, 257, 33), (64, 200, 7), (129, 1, 300)]


FLAG_SETS = {"default": 0, "two_buffers": X.SGEMM_DOUBLE_BUFFER,
             "global_loads": X.SGEMM_NO_BUFFER_LOADS}


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("bk", BKS)
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda v: X.AS_NAMES[v])
def test_exact_on_integer_inputs(layout, bk, flags):
    opts = X.make_sgemm_opts(layout, bk, flags=FLAG_SETS[flags])
    for idx, (m, n, k) in enumerate(EXACT_SHAPES):
        A = wl.small_int_f32((m, k), 100 + idx)
        B = wl.small_int_f32((k, n), 200 + idx)
        C = wl.small_int_f32((m, n), 300 + idx)
        check_exact(A, B, C, 2.0, -1.0, opts=opts, pads=(idx % 3, 2 * (idx % 2), 5))
        # beta == 0: C is not read, NaN there must not leak
        Cn = np.full((m, n), np.nan, np.float32)
        got = check_exact(A, B, Cn, 1.0, 0.0, opts=opts)
        assert np.isfinite(got[region_mask(m, n, max(n, 1), got.size)]).all()


@pytest.mark.parametrize("bk, tile_m", [(16, 256), (32, 256), (16, 64)])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda v: X.AS_NAMES[v])
def test_exact_tall_and_short_blocks(layout, bk, tile_m):
    """256 x 128 blocks (8 waves) and 64 x 128 blocks (2 waves), buffer and
    global loads."""
    for flags in (0, X.SGEMM_NO_BUFFER_LOADS):
        opts = X.make_sgemm_opts(layout, bk, 0, flags, tile_m)
        for idx, (m, n, k) in enumerate(EXACT_SHAPES + [(512, 256, 96), (257, 300, 65)]):
            A = wl.small_int_f32((m, k), 700 + idx)
            B = wl.small_int_f32((k, n), 800 + idx)
            C = wl.small_int_f32((m, n), 900 + idx)
            check_exact(A, B, C, 2.0, -1.0, opts=opts, pads=(idx % 3, 2 * (idx % 2), 5))


@pytest.mark.parametrize("bk, tile_m", [(8, 128), (16, 128), (32, 128), (64, 128),
                                         (16, 256), (32, 256), (16, 64)])
def test_whole_blocks_with_ragged_k(bk, tile_m):
    """Blocks wholly inside C with k not a multiple of the k step: buffer
    loads for every whole k step, checked loads for the last one.  A's
    pitch padding holds NaN, so a read past column k would show."""
    for layout in LAYOUTS:
        opts = X.make_sgemm_opts(layout, bk, 0, 0, tile_m)
        for idx, (m, n, k) in enumerate([(2 * tile_m, 256, 45), (tile_m, 384, 100),
                                         (tile_m, 128, bk + 1), (2 * tile_m, 128, 3)]):
            pad_a = (-k) % 4 + 4        # lda a multiple of 4: 16-byte loads
            rc, info = X.xpose_sgemm_plan(m, n, k, 1 << 40, k + pad_a,
                                          1 << 41, n, 1 << 42, n, opts)
            assert rc == 0 and info.vector_loads == 1 and info.buffer_loads == 1
            A = wl.small_int_f32((m, k), 1000 + idx)
            B = wl.small_int_f32((k, n), 1100 + idx)
            C = wl.small_int_f32((m, n), 1200 + idx)
            check_exact(A, B, C, 2.0, -1.0, opts=opts, pads=(pad_a, 0, 3))


@pytest.mark.parametrize("tile_m", (64, 128, 256))
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda v: X.AS_NAMES[v])
def test_whole_matrix_kernels(layout, tile_m):
    """The kernels without edge code (every block, k step, load and C tail
    whole), with both beta paths, C pitch padding, and A and B pitches
    padded by 4 floats (still 16-byte multiples, so the plan keeps the
    whole-matrix kernel; the descriptors and lane offsets then scale with
    lda and ldb, and NaN in the padding would show)."""
    opts = X.make_sgemm_opts(layout, 16, 0, 0, tile_m)
    for idx, (m, n, k) in enumerate([(2 * tile_m, 384, 512), (tile_m, 128, 16),
                                     (4 * tile_m, 256, 48)]):
        for pad_a, pad_b in ((0, 0), (4, 4), (8, 0), (0, 12)):
            rc, info = X.xpose_sgemm_plan(m, n, k, 1 << 40, k + pad_a, 1 << 41,
                                          n + pad_b, 1 << 42, n + 3, opts)
            assert rc == 0 and info.whole_matrix == 1, (pad_a, pad_b)
            A = wl.small_int_f32((m, k), 1300 + idx)
            B = wl.small_int_f32((k, n), 1400 + idx)
            C = wl.small_int_f32((m, n), 1500 + idx)
            check_exact(A, B, C, 2.0, -1.0, opts=opts, pads=(pad_a, pad_b, 3))
            Cn = np.full((m, n), np.nan, np.float32)
            got = check_exact(A, B, Cn, 1.0, 0.0, opts=opts,
                              pads=(pad_a, pad_b, 3))
            assert np.isfinite(got[region_mask(m, n, n + 3, got.size)]).all()


def test_edge_blocks_with_buffer_loads():
    """Edge blocks (m or n not a multiple of the block) and ragged last k
    steps read with buffer loads whose descriptors are clipped to the
    matrix, where k and n are multiples of 4.  A's and B's pitch padding
    holds NaN, so a column of A past k that was not zeroed, or a read past
    the matrix, would show; guard sentinels around C must stay unchanged."""
    shapes = [(200, 136, 72), (130, 260, 100), (1000, 132, 44), (129, 4, 4),
              (1, 128, 16), (257, 388, 36), (64, 1028, 8), (300, 300, 300)]
    for tile_m in (64, 128, 256):
        for layout in LAYOUTS:
            opts = X.make_sgemm_opts(layout, 16, 0, 0, tile_m)
            for idx, (m, n, k) in enumerate(shapes):
                for pad_a, pad_b in ((0, 0), (4, 8)):
                    rc, info = X.xpose_sgemm_plan(m, n, k, 1 << 40, k + pad_a,
                                                  1 << 41, n + pad_b, 1 << 42,
                                                  n, opts)
                    assert rc == 0 and info.edge_buffer_loads == 1, (m, n, k)
                    A = wl.small_int_f32((m, k), 1600 + idx)
                    B = wl.small_int_f32((k, n), 1700 + idx)
                    C = wl.small_int_f32((m, n), 1800 + idx)
                    check_exact(A, B, C, 2.0, -1.0, opts=opts,
                                pads=(pad_a, pad_b, 1))
    # k or n not a multiple of 4: the bounds-checked loads
    rc, info = X.xpose_sgemm_plan(200, 130, 72, 1 << 40, 72, 1 << 41, 132,
                                  1 << 42, 130)
    assert rc == 0 and info.edge_buffer_loads == 0


def test_scalar_load_path_is_exact():
    """4-byte aligned (not 16-byte) operands and pitches that are not a
    multiple of 4 take the 4-byte loads."""
    m, n, k = 197, 131, 77
    A = wl.small_int_f32((m, k), 11)
    B = wl.small_int_f32((k, n), 12)
    C = wl.small_int_f32((m, n), 13)
    rc, info = X.xpose_sgemm_plan(m, n, k, 0x7f0000000004, k + 1, 0x7f1000000000,
                                  n + 2, 0x7f2000000000, n)
    assert rc == 0 and info.vector_loads == 0
    for shifts, pads in (((1, 0, 0), (0, 0, 0)), ((0, 3, 1), (1, 2, 0)),
                         ((0, 0, 0), (1, 0, 3))):
        check_exact(A, B, C, 1.0, 1.0, shifts=shifts, pads=pads)


def test_uniform_inputs_within_the_fp32_bound():
    for idx, (m, n, k) in enumerate(((512, 512, 512), (1000, 777, 1025),
                                     (33, 4097, 64), (256, 128, 4096))):
        A = wl.uniform_f32((m, k), 400 + idx)
        B = wl.uniform_f32((k, n), 500 + idx)
        C = wl.uniform_f32((m, n), 600 + idx)
        check_bound(A, B, C, 1.0, 1.0, entry="plain")
        check_bound(A, B, C, -0.75, 0.0, pads=(3, 1, 2))


def test_all_kernels_agree_bit_for_bit():
    m, n, k = 384, 320, 544
    A = wl.uniform_f32((m, k), 71)
    B = wl.uniform_f32((k, n), 72)
    C = wl.uniform_f32((m, n), 73)
    ref = None
    for layout in LAYOUTS:
        for bk in BKS:
            for flags in FLAG_SETS.values():
                for tile_m in (64, 128, 256):
                    if tile_m == 256 and (bk not in (16, 32) or flags == X.SGEMM_DOUBLE_BUFFER):
                        continue
                    if tile_m == 64 and (bk != 16 or flags == X.SGEMM_DOUBLE_BUFFER):
                        continue
                    for shifts in ((0, 0, 0), (1, 1, 0)):
                        got, _, _ = run_case(A, B, C, 1.5, 0.5, shifts=shifts,
                                             opts=X.make_sgemm_opts(layout, bk, 0, flags, tile_m))
                        if ref is None:
                            ref = got
                        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
                            (layout, bk, flags, tile_m, shifts)


def test_degenerate_shapes():
    # k == 0: C = beta * C, a and b may be NULL
    C = wl.uniform_f32((70, 50), 81)
    d = torch.from_numpy(C.copy()).to(_dev())
    say("sgemm k=0")
    assert X.xpose_sgemm(70, 50, 0, 3.0, 0, 1, 0, 50, -0.5, d.data_ptr(), 50, 0) == 0
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), (np.float32(-0.5) * C).astype(np.float32))
    # m == 0 or n == 0: nothing happens, NULL pointers allowed
    assert X.xpose_sgemm(0, 50, 10, 1.0, 0, 10, 0, 50, 0.0, 0, 50, 0) == 0
    assert X.xpose_sgemm(70, 0, 10, 1.0, 0, 10, 0, 1, 0.0, 0, 1, 0) == 0
    # one row, one column
    for m, n, k in ((1, 300, 129), (300, 1, 129), (1, 1, 4096)):
        check_exact(wl.small_int_f32((m, k), 91), wl.small_int_f32((k, n), 92),
                    wl.small_int_f32((m, n), 93), 1.0, 1.0)


def test_side_stream():
    s = torch.cuda.Stream()
    A = wl.small_int_f32((160, 96), 1)
    B = wl.small_int_f32((96, 200), 2)
    C = wl.small_int_f32((160, 200), 3)
    check_exact(A, B, C, 1.0, 1.0, stream=s)


def test_page_size_default_launch_sampled():
    """The 4096^3 workload in the launch the benchmark times: 96 sampled rows
    of C against the oracle within the bound, and with B = 1 and integer A
    every element of C against the row sums (a property at any size)."""
    w = wl.GEMM_WORKLOADS["sgemm_4096"]
    A, B, C = wl.make_gemm_inputs(w)
    dev = _dev()
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C).to(dev)
    say("sgemm 4096^3 default")
    X.sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    rows = np.random.default_rng(5).choice(w.m, 96, replace=False)
    a_rows = np.ascontiguousarray(A[rows]).reshape(-1)
    c_rows = np.ascontiguousarray(C[rows]).reshape(-1)
    ref = og.sgemm(len(rows), w.n, w.k, w.alpha, a_rows, w.k, B.reshape(-1),
                   w.n, w.beta, c_rows, w.n)
    mag = abs(w.alpha) * (np.abs(A[rows].astype(np.float64)) @ np.abs(B.astype(np.float64)))
    mag += abs(w.beta) * np.abs(C[rows].astype(np.float64))
    err = np.abs(got[rows].astype(np.float64) - ref)
    assert (err <= (w.k + 3) * 2.0 ** -24 * mag).all(), err.max()
    del dA, dB, dC
    # B = 1: every column of C is alpha times A's row sums, exact on integers
    Ai = wl.small_int_f32((w.m, w.k), 6)
    ones = np.ones((w.k, w.n), np.float32)
    dA = torch.from_numpy(Ai).to(dev)
    dB = torch.from_numpy(ones).to(dev)
    say("sgemm 4096^3 row sums")
    dC = X.sgemm(dA, dB)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    sums = og.sgemm(w.m, 1, w.k, 1.0, Ai.reshape(-1), w.k,
                    np.ones(w.k, np.float32), 1, 0.0, np.zeros(w.m, np.float32), 1)
    assert np.array_equal(got, np.broadcast_to(sums.astype(np.float32), got.shape))


def test_random_campaign():
    """Seeded random cases over shapes (ragged, thin, empty k), pitches,
    pointer offsets, scalars and every option; integer inputs keep the
    result exact, so each case is compared bit for bit."""
    rng = np.random.default_rng(2024)
    dims = [1, 2, 3, 5, 17, 31, 64, 127, 128, 129, 200, 255, 256, 300, 513]
    for case in range(60):
        m, n = int(rng.choice(dims)), int(rng.choice(dims))
        k = int(rng.choice(dims + [0, 0]))
        pads = tuple(int(x) for x in rng.choice([0, 0, 1, 3, 4, 8], 3))
        shifts = tuple(int(x) for x in rng.choice([0, 0, 0, 1, 2, 3], 3))
        alpha = float(rng.choice([1.0, 2.0, -1.0, 0.5, 0.0]))
        beta = float(rng.choice([0.0, 1.0, -2.0, 0.25]))
        flags = int(rng.choice([0, 0, X.SGEMM_DOUBLE_BUFFER, X.SGEMM_NO_BUFFER_LOADS,
                                X.SGEMM_NO_XCD_REMAP]))
        bk = int(rng.choice(BKS))
        tile_m = 128
        if flags != X.SGEMM_DOUBLE_BUFFER and bk in (16, 32):
            tile_m = int(rng.choice([64, 128, 256] if bk == 16 else [128, 256]))
        opts = X.make_sgemm_opts(int(rng.choice(LAYOUTS)), bk,
                                 int(rng.choice([0, 1, 3, 8])), flags, tile_m)
        A = wl.small_int_f32((m, k), 10_000 + case)
        B = wl.small_int_f32((k, n), 20_000 + case)
        C = wl.small_int_f32((m, n), 30_000 + case)
        say(f"campaign case {case}")
        check_exact(A, B, C, alpha, beta, pads=pads, shifts=shifts, opts=opts)


SPLIT_SHAPES = [(128, 128, 512), (130, 67, 450), (300, 257, 1000),
                (256, 384, 768), (1, 129, 333), (64, 200, 48), (257, 4, 36)]


@pytest.mark.parametrize("splits", (2, 3, 4, 7, 64))
def test_split_k_exact_on_integer_inputs(splits):
    """k split into slices whose partial sums land in the workspace and are
    added by the second kernel: exact on integer inputs, with both beta
    paths (NaN in C with beta == 0 must not leak), ragged shapes, slices
    that end inside a k step, every load path and A/B pitch padding."""
    for idx, (m, n, k) in enumerate(SPLIT_SHAPES):
        for layout, bk, tile_m, flags in ((X.AS_PADDED, 16, 128, 0),
                                          (X.AS_SWIZZLE, 16, 256, 0),
                                          (X.AS_UNPADDED, 32, 128,
                                           X.SGEMM_NO_BUFFER_LOADS),
                                          (X.AS_PADDED, 8, 128,
                                           X.SGEMM_DOUBLE_BUFFER),
                                          (X.AS_SWIZZLE, 16, 64, 0)):
            opts = X.make_sgemm_opts(layout, bk, 0, flags, tile_m, splits)
            A = wl.small_int_f32((m, k), 3100 + idx)
            B = wl.small_int_f32((k, n), 3200 + idx)
            C = wl.small_int_f32((m, n), 3300 + idx)
            check_exact(A, B, C, 2.0, -1.0, opts=opts, entry="ws",
                        pads=(idx % 3, 4 * (idx % 2), 5))
            Cn = np.full((m, n), np.nan, np.float32)
            got = check_exact(A, B, Cn, 1.0, 0.0, opts=opts, entry="ws")
            assert np.isfinite(got[region_mask(m, n, max(n, 1), got.size)]).all()


def test_split_k_plans_and_small_workspaces():
    """The library's split at a small grid (1024 x 1024: 64 blocks), with
    the workspace it wants, one that holds only two slices, and one that
    holds none (then it does not split); a 4-byte aligned workspace and an
    odd n take the one-element sum."""
    m, n, k = 1024, 1024, 1024
    A = wl.small_int_f32((m, k), 41)
    B = wl.small_int_f32((k, n), 42)
    C = wl.small_int_f32((m, n), 43)
    rc, info = X.xpose_sgemm_plan_ws(m, n, k, 1 << 40, k, 1 << 41, n, 1 << 42,
                                     n, None, 1 << 43, 1 << 40)
    assert rc == 0 and info.splits > 1
    check_exact(A, B, C, 1.0, 1.0, entry="ws", want_splits=info.splits)
    check_exact(A, B, C, 1.0, 1.0, entry="ws", ws_bytes=2 * m * n * 4 + 100,
                want_splits=2)
    check_exact(A, B, C, 1.0, 1.0, entry="ws", ws_bytes=m * n * 4,
                want_splits=1)
    opts = X.make_sgemm_opts(split_k=3)
    m, n, k = 200, 131, 500
    A = wl.small_int_f32((m, k), 44)
    B = wl.small_int_f32((k, n), 45)
    C = wl.small_int_f32((m, n), 46)
    check_exact(A, B, C, -1.0, 0.5, entry="ws", opts=opts, ws_shift=1,
                want_splits=3)
    check_exact(A, B, C, -1.0, 0.5, entry="ws", opts=opts, ws_shift=3,
                pads=(1, 0, 2), shifts=(1, 1, 1), want_splits=3)


def test_split_k_uniform_bound_and_repeatable():
    """Uniform inputs: within the fp32 bound at the library's split, and
    the same call twice gives the same bits (the partials are added in a
    fixed order, no atomics)."""
    for idx, (m, n, k) in enumerate(((1024, 1024, 1024), (640, 384, 3000),
                                     (100, 1000, 2048))):
        A = wl.uniform_f32((m, k), 4100 + idx)
        B = wl.uniform_f32((k, n), 4200 + idx)
        C = wl.uniform_f32((m, n), 4300 + idx)
        got = check_bound(A, B, C, 1.0, 1.0, entry="ws")
        again, _, _ = run_case(A, B, C, 1.0, 1.0, entry="ws")
        assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_sgemm_convenience_splits_small_grids():
    """X.sgemm takes the library's split where the grid is small, with a
    torch-allocated workspace; integer inputs, exact."""
    dev = _dev()
    m, n, k = 768, 640, 1536
    rc, info = X.xpose_sgemm_plan_ws(m, n, k, 1 << 40, k, 1 << 41, n, 1 << 42,
                                     n, None, 1 << 43, 1 << 40)
    assert rc == 0 and info.splits > 1
    A = wl.small_int_f32((m, k), 51)
    B = wl.small_int_f32((k, n), 52)
    C = wl.small_int_f32((m, n), 53)
    dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C))
    say("sgemm convenience split")
    X.sgemm(dA, dB, dC, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    want = og.sgemm(m, n, k, 2.0, A.reshape(-1), k, B.reshape(-1), n, -1.0,
                    C.reshape(-1), n).astype(np.float32).reshape(m, n)
    assert np.array_equal(dC.cpu().numpy(), want)
    # an explicit split, and no split, through the same convenience
    for split_k in (5, 1):
        dC = torch.from_numpy(C).to(dev)
        X.sgemm(dA, dB, dC, alpha=2.0, beta=-1.0, split_k=split_k)
        torch.cuda.synchronize()
        assert np.array_equal(dC.cpu().numpy(), want), split_k


def test_split_k_random_campaign():
    """Seeded random split calls: shapes (ragged, thin, k from 1 to 3000),
    pitches, pointer and workspace offsets, scalars, kernels and splits (the
    library's choice with the workspace it wants, with a smaller one, or an
    explicit 2 to 64); integer inputs, so each is compared bit for bit."""
    rng = np.random.default_rng(4242)
    dims = [1, 3, 17, 64, 127, 128, 129, 200, 256, 300, 513, 700]
    for case in range(40):
        m, n = int(rng.choice(dims)), int(rng.choice(dims))
        k = int(rng.choice([1, 5, 16, 100, 255, 256, 512, 777, 1500, 3000]))
        pads = tuple(int(x) for x in rng.choice([0, 0, 1, 4, 8], 3))
        shifts = tuple(int(x) for x in rng.choice([0, 0, 1, 3], 3))
        alpha = float(rng.choice([1.0, 2.0, -1.0, 0.5]))
        beta = float(rng.choice([0.0, 1.0, -2.0]))
        flags = int(rng.choice([0, 0, X.SGEMM_NO_BUFFER_LOADS,
                                X.SGEMM_NO_XCD_REMAP, X.SGEMM_DOUBLE_BUFFER]))
        bk = int(rng.choice([8, 16, 16, 32]))
        tile_m = 128
        if flags != X.SGEMM_DOUBLE_BUFFER and bk in (16, 32):
            tile_m = int(rng.choice([64, 128, 256] if bk == 16 else [128, 256]))
        split = int(rng.choice([0, 0, 2, 3, 5, 8, 64]))
        opts = X.make_sgemm_opts(int(rng.choice(LAYOUTS)), bk, 0, flags,
                                 tile_m, split)
        ws_bytes = None
        if split == 0 and rng.random() < 0.3:
            ws_bytes = int(rng.integers(0, 3)) * m * n * 4 + 4
        A = wl.small_int_f32((m, k), 40_000 + case)
        B = wl.small_int_f32((k, n), 41_000 + case)
        C = wl.small_int_f32((m, n), 42_000 + case)
        say(f"split campaign {case}: {m}x{n}x{k} split={split} bk={bk} "
            f"tile_m={tile_m} flags={flags}")
        check_exact(A, B, C, alpha, beta, pads=pads, shifts=shifts, opts=opts,
                    entry="ws", ws_bytes=ws_bytes,
                    ws_shift=int(rng.choice([0, 1, 4])))


def test_hip_graph_capture_and_replay():
    """The SGEMM only enqueues its kernels (no allocation, memset or
    synchronisation), so it can be captured into a HIP graph, a split of k
    (product and sum kernels, workspace given) included.  C is reset eagerly
    between replays, and every replay must match the oracle."""
    dev = _dev()
    cases = [((300, 257, 100), 2.0, -1.0, None),
             ((512, 384, 64), 1.0, 0.0, X.make_sgemm_opts(X.AS_SWIZZLE, 32)),
             ((256, 256, 48), 1.0, 1.0, X.make_sgemm_opts(X.AS_PADDED, 16, 0, 0, 256)),
             ((256, 130, 1000), 1.0, 1.0, X.make_sgemm_opts(split_k=4))]
    bufs = []
    for idx, ((m, n, k), alpha, beta, opts) in enumerate(cases):
        A = wl.small_int_f32((m, k), 60 + idx)
        B = wl.small_int_f32((k, n), 70 + idx)
        C = wl.small_int_f32((m, n), 80 + idx)
        want = og.sgemm(m, n, k, alpha, A.reshape(-1), k, B.reshape(-1), n, beta,
                        C.reshape(-1), n).astype(np.float32)
        ws = None
        if opts is not None and opts.split_k:
            ws = torch.empty(4 * m * n, dtype=torch.float32, device=dev)
        bufs.append((torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                     torch.from_numpy(C).to(dev), torch.from_numpy(C).to(dev),
                     alpha, beta, opts, want, ws))

    def enqueue():
        sh = int(torch.cuda.current_stream().cuda_stream)
        for dA, dB, dC, _, alpha, beta, opts, _, ws in bufs:
            m, k = dA.shape
            n = dB.shape[1]
            if ws is None:
                assert X.xpose_sgemm_ex(m, n, k, alpha, dA.data_ptr(), k,
                                        dB.data_ptr(), n, beta, dC.data_ptr(),
                                        n, opts, sh) == 0
            else:
                assert X.xpose_sgemm_ws(m, n, k, alpha, dA.data_ptr(), k,
                                        dB.data_ptr(), n, beta, dC.data_ptr(),
                                        n, opts, ws.data_ptr(),
                                        4 * ws.numel(), sh) == 0

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # eager warm-up on the capture stream
        say("sgemm graph warm-up")
        enqueue()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue()
    for rep in range(3):
        for _, _, dC, dC0, *_ in bufs:
            dC.copy_(dC0)  # eager work between replays: C back to its input
        torch.cuda.synchronize()
        say(f"sgemm graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for i, (_, _, dC, _, _, _, _, want, _) in enumerate(bufs):
            assert np.array_equal(dC.cpu().numpy(), want), f"replay {rep}, case {i}"
