"""Maximum sizes on the GPU, through the C ABI: matrices with more than 2^31
elements, byte offsets past 4 GiB, batches whose later entries start past
2^31 elements, and SGEMM operands whose row offsets pass 2^31 elements.

Every output element is checked against a pattern that the input's
position decides (the element's own row and column index where the
element is wide enough to hold them, a position hash for 1- and 2-byte
elements, with the batch entry mixed in), computed independently on the
device; sampled blocks around the 2^31-element and 4 GiB boundaries and
the ragged corners are also checked against the oracle.  Output pitch
padding and guard bands must keep their sentinel bytes.

The SGEMM cases use small integers, so every sum is exact in fp32: sampled
rows (the first, the last, those around 2^31 elements) must equal the
oracle exactly, and every row sum of C must equal the one the definition
gives (A's rows against B's row sums, exact in float64)."""
import numpy as np
import pytest

import oracle
import oracle.sgemm as og
from xpose_testlib import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
X = pytest.importorskip("lds_tiled_matrix_amd")

GUARD = 4096            # guard bytes after the output
SENT = 0x5A             # sentinel byte of the output buffer
CHUNK_BYTES = 1 << 29   # int64 temporaries per pattern chunk
TORCH_INT = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
RAW_NP = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def pattern(s, b, i, j):
    """Raw bits of input element (b, i, j) as an int64 tensor (i, j int64
    tensors that broadcast): the row and column index themselves for 4- and
    8-byte elements (rows and columns below 2^16), a position hash for 1-
    and 2-byte ones.  Then reduced to the element's width, as two's
    complement for the signed torch types."""
    if s >= 4:
        v = i * 65536 + j + b * 0x01000193
    else:
        v = (i * 0x9E37 + j * 0x7F4B + (i >> 9) * 0x3C6F + (j >> 9) * 0x2A55 +
             b * 0x5BD1)
    if s == 8:
        return v
    m = 1 << (8 * s)
    v = torch.remainder(v, m)
    if s == 1:
        return v
    return torch.where(v >= m // 2, v - m, v)


def fill_input(x, s):
    """x: (batch, rows, cols) strided view; filled chunk by chunk."""
    batch, rows, cols = x.shape
    dev = x.device
    step = max(1, CHUNK_BYTES // (8 * cols))
    j = torch.arange(cols, device=dev, dtype=torch.int64)[None, :]
    for b in range(batch):
        for r0 in range(0, rows, step):
            i = torch.arange(r0, min(rows, r0 + step), device=dev,
                             dtype=torch.int64)[:, None]
            x[b, r0:r0 + i.shape[0]] = pattern(s, b, i, j).to(x.dtype)


def check_output(y, s):
    """y: (batch, cols, rows) strided view of the output; y[b, j, i] must
    hold input element (b, i, j)."""
    batch, cols, rows = y.shape
    dev = y.device
    step = max(1, CHUNK_BYTES // (8 * rows))
    i = torch.arange(rows, device=dev, dtype=torch.int64)[None, :]
    for b in range(batch):
        for c0 in range(0, cols, step):
            j = torch.arange(c0, min(cols, c0 + step), device=dev,
                             dtype=torch.int64)[:, None]
            exp = pattern(s, b, i, j).to(y.dtype)
            got = y[b, c0:c0 + j.shape[0]]
            if not torch.equal(got, exp):
                bad = (got != exp).nonzero()[:4].tolist()
                raise AssertionError(f"batch {b}: output (col, row) offsets "
                                     f"{[(c0 + p[0], p[1]) for p in bad]} "
                                     f"wrong")


def oracle_blocks(x, y, s, spots, h=9, w=11):
    """Blocks of the input at `spots` (b, i0, j0), transposed by the oracle
    on the host, against the same blocks of the output."""
    batch, rows, cols = x.shape
    for b, i0, j0 in spots:
        i0 = min(max(i0, 0), rows - h)
        j0 = min(max(j0, 0), cols - w)
        blk = x[b, i0:i0 + h, j0:j0 + w].cpu().numpy().view(RAW_NP[s])
        got = y[b, j0:j0 + w, i0:i0 + h].cpu().numpy().view(RAW_NP[s])
        assert np.array_equal(got, oracle.transpose(blk)), (b, i0, j0)


LARGE = [
    # name, element bytes, batch, rows, cols, ld_in pad, ld_out pad, stride pads
    ("f32 odd pitches, 2^31 + 97,115 elements", 4, 1, 46341, 46343, 0, 0, (0, 0)),
    ("f32 whole tiles, padded output pitch", 4, 1, 46336, 46400, 0, 64, (0, 0)),
    ("f16 odd pitches, 2^31 + 97,115 elements", 2, 1, 46341, 46343, 0, 0, (0, 0)),
    ("u8 ragged, 2.5e9 elements", 1, 1, 50021, 50023, 0, 0, (0, 0)),
    ("f64 past 4 GiB", 8, 1, 23201, 23203, 0, 0, (0, 0)),
    ("f32 batch of 6, padded strides", 4, 6, 20000, 20001, 3, 5, (17, 33)),
]


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_large_transpose(case):
    name, s, batch, rows, cols, pin, pout, (spin, spout) = case
    dev = _dev()
    ld_in, ld_out = cols + pin, rows + pout
    stride_in = rows * ld_in + spin
    stride_out = cols * ld_out + spout
    n_in = (batch - 1) * stride_in + rows * ld_in
    n_out = (batch - 1) * stride_out + cols * ld_out
    say(f"large transpose: {name}: s={s} batch={batch} {rows}x{cols} "
        f"ld {ld_in}/{ld_out} stride {stride_in}/{stride_out} "
        f"in {n_in * s / 2**30:.2f} GiB")
    dt = TORCH_INT[s]
    src = torch.empty(n_in, dtype=dt, device=dev)
    x = src.as_strided((batch, rows, cols), (stride_in, ld_in, 1))
    fill_input(x, s)
    dst_bytes = torch.full((n_out * s + GUARD,), SENT, dtype=torch.uint8,
                           device=dev)
    dst = dst_bytes[:n_out * s].view(dt)
    y = dst.as_strided((batch, cols, rows), (stride_out, ld_out, 1))
    rc, info = X.xpose_plan(dst.data_ptr(), src.data_ptr(), batch, rows, cols,
                            ld_in, ld_out, stride_in, stride_out,
                            X.dtype_code(dt))
    assert rc == 0, X.strerror(rc)
    say(f"  plan {info.as_dict()}")
    rc = X.xpose_batched_ex(dst.data_ptr(), src.data_ptr(), batch, rows, cols,
                            ld_in, ld_out, stride_in, stride_out,
                            X.dtype_code(dt), None, 0)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    say("  transposed; checking")
    check_output(y, s)
    # ld padding, stride padding and the guard keep their sentinel bytes
    if pout:
        pad = dst.as_strided((batch, cols, pout), (stride_out, ld_out, 1),
                             rows)
        assert bool((pad.contiguous().view(torch.uint8) == SENT).all())
    if spout:
        for b in range(batch - 1):
            o = (b * stride_out + cols * ld_out) * s
            assert bool((dst_bytes[o:o + spout * s] == SENT).all())
    assert bool((dst_bytes[n_out * s:] == SENT).all())
    # oracle on sampled blocks: corners, the middle, and the rows where the
    # input offset passes 2^31 elements and 2^32 bytes
    spots = [(0, 0, 0), (batch - 1, rows, cols), (batch - 1, 0, cols),
             (batch - 1, rows, 0), (batch // 2, rows // 2, cols // 2)]
    for lim in (1 << 31, (1 << 32) // s):
        b, r = divmod(lim, stride_in)
        if b < batch and r // ld_in < rows:
            spots.append((b, r // ld_in - 4, r % ld_in - 5))
    rng = np.random.default_rng(31)
    spots += [(int(rng.integers(batch)), int(rng.integers(rows)),
               int(rng.integers(cols))) for _ in range(6)]
    oracle_blocks(x, y, s, spots)
    del src, x, dst_bytes, dst, y
    _free()


def _int_matrix(gen, shape, dev):
    return torch.randint(-2, 3, shape, generator=gen, device=dev,
                         dtype=torch.float32)


SGEMM_LARGE = [
    # name, m, n, k, lda, buffer loads expected
    ("A rows past 2^31 elements, buffer loads", 525000, 136, 1024, 4096, 1),
    ("pitch past the buffer-load limit", 515, 72, 300, 4200004, 0),
]


@pytest.mark.parametrize("case", SGEMM_LARGE, ids=[c[0] for c in SGEMM_LARGE])
def test_large_sgemm(case):
    name, m, n, k, lda, buf = case
    dev = _dev()
    alpha, beta = 2.0, -1.0
    say(f"large sgemm: {name}: m={m} n={n} k={k} lda={lda} "
        f"A {((m - 1) * lda + k) * 4 / 2**30:.2f} GiB")
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    # A's storage: NaN everywhere, so pitch padding that is read poisons C.
    a_store = torch.full(((m - 1) * lda + k,), float("nan"),
                         dtype=torch.float32, device=dev)
    A = a_store.as_strided((m, k), (lda, 1))
    for r0 in range(0, m, 65536):
        r1 = min(m, r0 + 65536)
        A[r0:r1] = _int_matrix(gen, (r1 - r0, k), dev)
    B = _int_matrix(gen, (k, n), dev)
    C0 = _int_matrix(gen, (m, n), dev)
    C = C0.clone()
    rc, info = X.xpose_sgemm_plan(m, n, k, A.data_ptr(), lda, B.data_ptr(), n,
                                  C.data_ptr(), n, None)
    assert rc == 0 and info.buffer_loads == buf
    rc = X.xpose_sgemm(m, n, k, alpha, A.data_ptr(), lda, B.data_ptr(), n,
                       beta, C.data_ptr(), n, 0)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    say("  multiplied; checking")
    assert bool(torch.isfinite(C).all())
    # every row sum: alpha * A (B 1) + beta * C0 1, exact in float64
    bsum = B.double().sum(1)
    for r0 in range(0, m, 65536):
        r1 = min(m, r0 + 65536)
        exp = alpha * (A[r0:r1].double() @ bsum) + beta * C0[r0:r1].double().sum(1)
        got = C[r0:r1].double().sum(1)
        assert torch.equal(got, exp), r0
    # sampled rows against the oracle, exactly
    rows = {0, 1, 127, 128, m - 2, m - 1}
    for lim in (1 << 29, 1 << 30, 1 << 31):
        r = lim // lda
        rows |= {r - 1, r, r + 1}
    rng = np.random.default_rng(43)
    rows |= set(int(v) for v in rng.integers(0, m, 40))
    rows = sorted(r for r in rows if 0 <= r < m) if m > 4096 else list(range(m))
    idx = torch.tensor(rows, device=dev)
    a_s = A.index_select(0, idx).cpu().numpy().reshape(-1)
    c0_s = C0.index_select(0, idx).cpu().numpy().reshape(-1)
    b_h = B.cpu().numpy().reshape(-1)
    exp = og.sgemm(len(rows), n, k, alpha, a_s, k, b_h, n, beta, c0_s, n)
    got = C.index_select(0, idx).cpu().numpy()
    bad = np.argwhere(got != exp.astype(np.float32))
    assert bad.size == 0, [(rows[p[0]], p[1]) for p in bad[:4]]
    del a_store, A, B, C0, C
    _free()


@pytest.mark.parametrize("tile_m", (128, 256))
@pytest.mark.parametrize("past", (0, 4), ids=("at_limit", "past_limit"))
def test_sgemm_c_pitch_at_the_epilogue_limit(tile_m, past):
    """Whole blocks write C through one buffer descriptor while the block
    spans at most 2^31 bytes (ldc <= 2^29 / tile_m), and through checked
    global stores past that: both sides of the limit, exact against the
    oracle on every element, pitch padding untouched."""
    dev = _dev()
    m, n, k = 2 * tile_m, 256, 48
    ldc = (1 << 29) // tile_m + past
    say(f"sgemm C pitch: tile_m={tile_m} ldc={ldc} m={m} n={n} k={k}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(47)
    A = _int_matrix(gen, (m, k), dev)
    B = _int_matrix(gen, (k, n), dev)
    c_store = torch.full(((m - 1) * ldc + n,), -7.5, dtype=torch.float32,
                         device=dev)
    C = c_store.as_strided((m, n), (ldc, 1))
    C0 = _int_matrix(gen, (m, n), dev)
    C.copy_(C0)
    opts = X.make_sgemm_opts(tile_m=tile_m)
    rc = X.xpose_sgemm_ex(m, n, k, 2.0, A.data_ptr(), k, B.data_ptr(), n, -1.0,
                          C.data_ptr(), ldc, opts, 0)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    exp = og.sgemm(m, n, k, 2.0, A.cpu().numpy().reshape(-1), k,
                   B.cpu().numpy().reshape(-1), n, -1.0,
                   C0.cpu().numpy().reshape(-1), n)
    got = C.cpu().numpy()
    bad = np.argwhere(got != exp.astype(np.float32))
    assert bad.size == 0, bad[:4].tolist()
    pad = c_store.as_strided((m - 1, 4096), (ldc, 1), n)
    assert bool((pad == -7.5).all())
    del A, B, c_store, C, C0
    _free()
