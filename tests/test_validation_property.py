"""Property test of the C ABI's argument validation (CPU only): for random
arguments, xpose_plan's status must equal the rules include/xpose.h states,
written out here independently of the library."""
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import lds_tiled_matrix_amd as X  # noqa: E402

ELEM = {0: 4, 1: 2, 2: 2, 3: 1, 4: 8}


def expected_status(out, inp, batch, rows, cols, ld_in, ld_out, stride_in,
                    stride_out, dtype):
    """The documented contract of xpose_batched, as a plain function."""
    if dtype not in ELEM:
        return X.XPOSE_EDTYPE
    s = ELEM[dtype]
    if batch < 0 or rows < 0 or cols < 0:
        return X.XPOSE_EINVAL
    if batch == 0 or rows == 0 or cols == 0:
        return X.XPOSE_OK
    if out == 0 or inp == 0:
        return X.XPOSE_EINVAL
    if ld_in < cols or ld_out < rows:
        return X.XPOSE_EINVAL
    if batch > 1 and stride_in < 0:
        return X.XPOSE_EINVAL
    if batch == 1:
        stride_in = stride_out = 0
    out_one = (cols - 1) * ld_out + rows
    if batch > 1 and stride_out < out_one:
        return X.XPOSE_EINVAL
    ext_in = (batch - 1) * stride_in + (rows - 1) * ld_in + cols
    ext_out = (batch - 1) * stride_out + out_one
    if max(ext_in, ext_out) * s >= 2 ** 63:
        return X.XPOSE_EINVAL
    if inp % s or out % s:
        return X.XPOSE_EALIGN
    if inp < out + ext_out * s and out < inp + ext_in * s:
        return X.XPOSE_EALIAS
    return X.XPOSE_OK


dims = st.integers(min_value=-2, max_value=300)
pads = st.integers(min_value=-3, max_value=40)
ptrs = st.sampled_from([0, 1 << 32, (1 << 32) + 2, (1 << 32) + 4,
                        (1 << 32) + 8, (1 << 32) + 1000, (1 << 33), 4096])


@settings(max_examples=3000, deadline=None, derandomize=True)
@given(out=ptrs, inp=ptrs, batch=st.integers(-1, 4), rows=dims, cols=dims,
       pad_in=pads, pad_out=pads, gap_in=st.integers(-500, 500),
       gap_out=st.integers(-500, 500), dtype=st.integers(-1, 5))
def test_plan_status_matches_contract(out, inp, batch, rows, cols, pad_in,
                                      pad_out, gap_in, gap_out, dtype):
    ld_in, ld_out = cols + pad_in, rows + pad_out
    stride_in = rows * ld_in + gap_in
    stride_out = cols * ld_out + gap_out
    want = expected_status(out, inp, batch, rows, cols, ld_in, ld_out,
                           stride_in, stride_out, dtype)
    rc, info = X.xpose_plan(out, inp, batch, rows, cols, ld_in, ld_out,
                            stride_in, stride_out, dtype, None)
    assert rc == want
    if rc == 0 and batch > 0 and rows > 0 and cols > 0:
        assert info.tiles >= batch * -(-rows // info.tile_rows) * -(-cols // info.tile_cols)
        assert info.tile_rows > 0 and info.tile_cols > 0


@settings(max_examples=500, deadline=None, derandomize=True)
@given(rows=st.integers(1, 5000), cols=st.integers(1, 5000),
       batch=st.integers(1, 70), dtype=st.sampled_from([0, 1, 3, 4]))
def test_every_default_plan_has_a_kernel(rows, cols, batch, dtype):
    """Whatever the shape, the default launch resolves to a built kernel and
    covers the matrix with whole tiles (line-aligned output tiles shift
    segments back by up to one line less one element, hence up to one more
    tile row)."""
    rc, info = X.xpose_plan(1 << 40, 1 << 44, batch, rows, cols, cols, rows,
                            rows * cols, rows * cols, dtype, None)
    assert rc == 0
    if info.packed:
        # packed batch of small matrices: whole matrices per workgroup
        edge = 128 if ELEM[dtype] == 1 else 64
        ragged = rows % edge or cols % edge
        assert batch > 1 and rows * cols * ELEM[dtype] <= (32768 if ragged else 16384)
        assert (info.tile_rows, info.tile_cols) == (rows, cols)
        assert info.packed * rows * cols * ELEM[dtype] <= info.lds_bytes
        assert info.tiles == -(-batch // info.packed)
        return
    extra = 128 // ELEM[dtype] - 1 if info.aligned_out else 0
    assert info.aligned_out in (0, 1) and (not extra or dtype in (0, 1, 2, 4))
    per = -(-(rows + extra) // info.tile_rows) * -(-cols // info.tile_cols)
    assert info.tiles == batch * per
    assert info.lds_bytes > 0 and info.threads in (64, 128, 256)


SG_A, SG_B, SG_C, SG_W = 0x7f0000000000, 0x7f1000000000, 0x7f2000000000, 0x7f3000000000


@settings(max_examples=400, deadline=None)
@given(m=st.integers(1, 5000), n=st.integers(1, 5000), k=st.integers(0, 70000),
       bk=st.sampled_from([0, 8, 16, 32, 64]), tile_m=st.sampled_from([0, 64, 128, 256]),
       split=st.integers(0, 64), ws_planes=st.integers(0, 80),
       ws_extra=st.integers(0, 4096))
def test_sgemm_split_plan_invariants(m, n, k, bk, tile_m, split, ws_planes,
                                     ws_extra):
    """Any xpose_sgemm_plan_ws result: slices of whole k steps covering k
    exactly once, a workspace use that fits what was given, the grid the
    slices imply; the library's choice never shorter than 64 per slice and
    an explicit split never more slices than asked."""
    X = pytest.importorskip("lds_tiled_matrix_amd")
    opts = X.make_sgemm_opts(0, bk, 0, 0, tile_m, split)
    ws_bytes = ws_planes * m * n * 4 + ws_extra
    rc, info = X.xpose_sgemm_plan_ws(m, n, k, SG_A, max(k, 1), SG_B, n, SG_C,
                                     n, opts, SG_W, ws_bytes)
    if rc == X.XPOSE_ENOTILE:      # e.g. bk 64 with 256-row blocks
        return
    if rc == X.XPOSE_EWORKSPACE:
        assert split >= 2 and info.workspace_wanted > ws_bytes
        return
    assert rc == 0
    S, L = info.splits, info.split_len
    base = -(-m // info.tile_m) * -(-n // 128)
    assert info.tiles == base * S
    if S == 1:
        assert L == k and info.workspace_bytes == 0
        return
    assert L % info.bk == 0 and (S - 1) * L < k <= S * L
    assert info.workspace_bytes == S * m * n * 4 <= ws_bytes
    if split == 0:
        assert L >= 64
    else:
        assert S <= split
