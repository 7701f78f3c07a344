"""Host-side checks of the SGEMM entry points (include/xpose_sgemm.h): plan
defaults, option handling and argument validation.  No GPU: bogus pointer
values are fine, invalid calls return before anything is launched and
xpose_sgemm_plan never dereferences."""
import pytest

import lds_tiled_matrix_amd as X

A, B, C = 0x7f0000000000, 0x7f1000000000, 0x7f2000000000


def plan(m=4096, n=4096, k=4096, a=A, lda=None, b=B, ldb=None, c=C, ldc=None,
         opts=None):
    lda = max(k, 1) if lda is None else lda
    ldb = max(n, 1) if ldb is None else ldb
    ldc = max(n, 1) if ldc is None else ldc
    return X.xpose_sgemm_plan(m, n, k, a, lda, b, ldb, c, ldc, opts)


def test_default_plan():
    """The pages' padded store in 128 x 128 blocks; large round shapes
    (4096^3: 512 blocks of 256 x 128, one full round) take the swizzled
    layout in 256-row blocks."""
    rc, info = plan(m=3072)
    assert rc == 0
    assert (info.layout, info.bk, info.as_stride) == (X.AS_PADDED, 16, 130)
    assert (info.tile_m, info.tile_n, info.threads) == (128, 128, 256)
    assert info.tiles == 24 * 32 and info.vector_loads == 1
    assert info.lds_bytes == 4 * (16 * 130 + 16 * 128)
    assert info.group_m == 8 and info.xcd_remap == 1 and info.stages == 1
    assert info.buffer_loads == 1
    rc, info = plan()
    assert rc == 0
    assert (info.layout, info.bk, info.as_stride) == (X.AS_SWIZZLE, 16, 256)
    assert (info.tile_m, info.tile_n, info.threads) == (256, 128, 512)
    assert info.tiles == 16 * 32 and info.lds_bytes == 4 * (16 * 256 + 16 * 128)
    rc, info = plan(opts=X.make_sgemm_opts(flags=X.SGEMM_DOUBLE_BUFFER))
    assert rc == 0 and info.stages == 2 and info.layout == X.AS_PADDED
    assert info.lds_bytes == 2 * 4 * (16 * 130 + 16 * 128)


@pytest.mark.parametrize("m, n, k, tall", [
    (4096, 4096, 4096, True), (8192, 4096, 4096, True), (2048, 16384, 4096, True),
    (16384, 16384, 2048, True), (4096, 4096, 1024, True),
    (4096, 4096, 1023, False),       # k below the rule
    (3072, 4096, 4096, False),       # 384 blocks: a partial round
    (4096, 4100, 4096, False),       # n not a multiple of 128
    (4224, 4096, 4096, False),       # m not a multiple of 256
    (6144, 6144, 6144, False),       # 1152 blocks: 2.25 rounds
    (0, 4096, 4096, False)])
def test_default_tall_rule(m, n, k, tall):
    rc, info = plan(m=m, n=n, k=k)
    assert rc == 0
    if m == 0:
        return
    assert (info.layout, info.tile_m) == ((X.AS_SWIZZLE, 256) if tall else (X.AS_PADDED, 128))


def test_any_choice_turns_the_tall_rule_off():
    for opts in (X.make_sgemm_opts(layout=X.AS_PADDED), X.make_sgemm_opts(bk=16),
                 X.make_sgemm_opts(tile_m=128), X.make_sgemm_opts(flags=X.SGEMM_DOUBLE_BUFFER)):
        rc, info = plan(opts=opts)
        assert rc == 0 and info.tile_m == 128
    # block order and load options keep it
    for opts in (X.make_sgemm_opts(group_m=3), X.make_sgemm_opts(flags=X.SGEMM_NO_BUFFER_LOADS),
                 X.make_sgemm_opts(flags=X.SGEMM_NO_XCD_REMAP)):
        rc, info = plan(opts=opts)
        assert rc == 0 and (info.layout, info.tile_m) == (X.AS_SWIZZLE, 256)


@pytest.mark.parametrize("bk", (8, 16, 32, 64))
def test_layout_strides(bk):
    """Padded stride 128 + 32 / min(bk, 32): the pad that spreads one
    half-wave's transposed stores over the 32 banks; the others keep 128."""
    for layout, stride in ((X.AS_UNPADDED, 128), (X.AS_PADDED, 128 + 32 // min(bk, 32)),
                           (X.AS_SWIZZLE, 128)):
        rc, info = plan(opts=X.make_sgemm_opts(layout, bk))
        assert rc == 0 and info.as_stride == stride and info.bk == bk
        assert info.lds_bytes == 4 * bk * (stride + 128)


def test_tall_blocks():
    """256 x 128 blocks (8 waves) for k steps 16 and 32, one LDS buffer."""
    for bk in (16, 32):
        rc, info = plan(opts=X.make_sgemm_opts(bk=bk, tile_m=256))
        assert rc == 0 and (info.tile_m, info.tile_n, info.threads) == (256, 128, 512)
        assert info.tiles == 16 * 32
        assert info.lds_bytes == 4 * bk * ((256 + 32 // bk) + 128)
    rc, info = plan(m=300, n=129, opts=X.make_sgemm_opts(tile_m=256))
    assert rc == 0 and info.tiles == 2 * 2
    assert plan(opts=X.make_sgemm_opts(bk=8, tile_m=256))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.make_sgemm_opts(tile_m=256, flags=X.SGEMM_DOUBLE_BUFFER))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.make_sgemm_opts(tile_m=96))[0] == X.XPOSE_EINVAL
    # 64-row blocks: 2 waves, k step 16, one LDS buffer
    rc, info = plan(opts=X.make_sgemm_opts(tile_m=64))
    assert rc == 0 and (info.tile_m, info.threads) == (64, 128)
    assert plan(opts=X.make_sgemm_opts(bk=32, tile_m=64))[0] == X.XPOSE_ENOTILE
    # buffer loads: half the lda limit of 128-row blocks
    big = (1 << 31) // (4 * 257)
    assert plan(m=512, lda=big - big % 4, opts=X.make_sgemm_opts(tile_m=256))[1].buffer_loads == 1
    assert plan(m=512, lda=big + 4 - big % 4, opts=X.make_sgemm_opts(tile_m=256))[1].buffer_loads == 0


def test_ragged_tiles_and_group_clamp():
    rc, info = plan(m=130, n=67, k=45)
    assert rc == 0 and info.tiles == 2 * 1 and info.group_m == 2
    rc, info = plan(m=1, n=1, k=1)
    assert rc == 0 and info.tiles == 1 and info.group_m == 1
    rc, info = plan(opts=X.make_sgemm_opts(group_m=3, flags=X.SGEMM_NO_XCD_REMAP))
    assert rc == 0 and info.group_m == 3 and info.xcd_remap == 0


def test_vector_load_rules():
    assert plan()[1].vector_loads == 1
    assert plan(a=A + 4)[1].vector_loads == 0          # 4-byte aligned only
    assert plan(b=B + 8)[1].vector_loads == 0
    assert plan(lda=4097)[1].vector_loads == 0         # pitch not a multiple of 4
    assert plan(ldb=4098)[1].vector_loads == 0
    assert plan(c=C + 4, ldc=4099)[1].vector_loads == 1  # C is never vector-loaded


def test_buffer_load_rules():
    """Whole tiles are read with buffer loads where 128 rows of A and 32 of B
    fit in 31-bit byte offsets, 16-byte loads are allowed and no flag turns
    them off."""
    assert plan()[1].buffer_loads == 1
    assert plan(a=A + 4)[1].buffer_loads == 0            # 4-byte loads
    big = (1 << 31) // (4 * 129)                        # 4161790
    rc, info = plan(lda=big - 2, m=256)
    assert rc == 0 and info.buffer_loads == 1
    rc, info = plan(lda=big + 2, m=256)
    assert rc == 0 and info.vector_loads == 1 and info.buffer_loads == 0
    rc, info = plan(ldb=big * 2, k=32)
    assert rc == 0 and info.buffer_loads == 1
    rc, info = plan(ldb=big * 2 + 4, k=32)
    assert rc == 0 and info.vector_loads == 1 and info.buffer_loads == 0
    rc, info = plan(opts=X.make_sgemm_opts(flags=X.SGEMM_NO_BUFFER_LOADS))
    assert rc == 0 and info.buffer_loads == 0 and info.vector_loads == 1
    assert plan(k=0, a=0, b=0, lda=1)[1].buffer_loads == 0


@pytest.mark.parametrize("kw, code", [
    (dict(m=-1), X.XPOSE_EINVAL),
    (dict(k=-1), X.XPOSE_EINVAL),
    (dict(lda=4095), X.XPOSE_EINVAL),
    (dict(ldb=4095), X.XPOSE_EINVAL),
    (dict(ldc=4095), X.XPOSE_EINVAL),
    (dict(a=0), X.XPOSE_EINVAL),
    (dict(b=0), X.XPOSE_EINVAL),
    (dict(c=0), X.XPOSE_EINVAL),
    (dict(a=A + 2), X.XPOSE_EALIGN),
    (dict(c=C + 1), X.XPOSE_EALIGN),
    (dict(c=A), X.XPOSE_EALIAS),
    (dict(c=B + 4 * 4096 * 4095), X.XPOSE_EALIAS),   # C starts on B's last row
    (dict(lda=1 << 62), X.XPOSE_EINVAL),               # extent overflows
    (dict(opts=X.make_sgemm_opts(layout=4)), X.XPOSE_EINVAL),
    (dict(opts=X.make_sgemm_opts(bk=12)), X.XPOSE_EINVAL),
    (dict(opts=X.make_sgemm_opts(bk=128)), X.XPOSE_EINVAL),
    (dict(opts=X.make_sgemm_opts(group_m=-1)), X.XPOSE_EINVAL),
    (dict(opts=X.make_sgemm_opts(flags=8)), X.XPOSE_EINVAL),
])
def test_invalid_calls(kw, code):
    assert plan(**kw)[0] == code
    # the entry points validate the same way, before launching anything
    args = dict(m=4096, n=4096, k=4096, a=A, lda=4096, b=B, ldb=4096, c=C,
                ldc=4096, opts=None)
    args.update(kw)
    rc = X.xpose_sgemm_ex(args["m"], args["n"], args["k"], 1.0, args["a"],
                          args["lda"], args["b"], args["ldb"], 0.0, args["c"],
                          args["ldc"], args["opts"], 0)
    assert rc == code


def test_a_and_b_may_overlap():
    assert plan(b=A)[0] == 0


def test_empty_shapes_are_noops_even_with_null_pointers():
    for m, n in ((0, 5), (5, 0), (0, 0)):
        rc, info = plan(m=m, n=n, k=7, a=0, b=0, c=0)
        assert rc == 0 and info.tiles == 0
        assert X.xpose_sgemm(m, n, 7, 1.0, 0, 7, 0, max(n, 1), 0.0, 0,
                             max(n, 1), 0) == 0


def test_k_zero_needs_only_c():
    rc, info = plan(k=0, a=0, b=0, lda=1)
    assert rc == 0 and info.tiles == 1024
    assert plan(k=0, a=0, b=0, lda=1, c=0)[0] == X.XPOSE_EINVAL


@pytest.mark.parametrize("kw, whole", [
    (dict(), 1),                                   # 4096^3: tall swizzled blocks
    (dict(m=3072), 1),                             # padded 128-row blocks
    (dict(k=4100, lda=4100), 0),                   # k not a multiple of the k step
    (dict(m=4100), 0),                             # ragged block rows
    (dict(n=4100, ldb=4100, ldc=4100), 0),         # ragged block columns
    (dict(lda=4097), 0),                           # 4-byte loads
    (dict(a=A + 4), 0),                            # A not 16-byte aligned
    (dict(m=256, ldc=(1 << 29) // 128 + 4), 0),    # C pitch past the tail's limit
    (dict(opts=X.make_sgemm_opts(bk=32)), 0),      # built for k step 16 only
    (dict(opts=X.make_sgemm_opts(flags=X.SGEMM_DOUBLE_BUFFER)), 0),
    (dict(opts=X.make_sgemm_opts(flags=X.SGEMM_NO_BUFFER_LOADS)), 0),
    (dict(opts=X.make_sgemm_opts(layout=X.AS_UNPADDED)), 1),
    (dict(opts=X.make_sgemm_opts(layout=X.AS_PADDED, tile_m=256)), 1)])
def test_whole_matrix_kernel_choice(kw, whole):
    """The kernel without edge code serves a call only when every block, k
    step, load and C tail is whole."""
    rc, info = plan(**kw)
    assert rc == 0 and info.whole_matrix == whole


WS = 0x7f3000000000


def plan_ws(m=1024, n=1024, k=1024, ws=WS, ws_bytes=1 << 40, opts=None,
            a=A, b=B, c=C, ldc=None):
    ldc = max(n, 1) if ldc is None else ldc
    return X.xpose_sgemm_plan_ws(m, n, k, a, max(k, 1), b, max(n, 1), c, ldc,
                                 opts, ws, ws_bytes)


def test_no_split_without_a_workspace():
    """xpose_sgemm and xpose_sgemm_ex never split; the plan still reports
    what the workspace entry point would want."""
    rc, info = plan(m=1024, n=1024, k=1024)
    assert rc == 0 and info.splits == 1 and info.split_len == 1024
    assert info.workspace_bytes == 0 and info.tiles == 64
    assert info.workspace_wanted == 4 * 1024 * 1024 * 4
    rc, info = plan(opts=X.make_sgemm_opts(split_k=4), m=1024, n=1024, k=1024)
    assert rc == X.XPOSE_EWORKSPACE
    # the call returns the same before launching anything
    assert X.xpose_sgemm_ex(1024, 1024, 1024, 1.0, A, 1024, B, 1024, 0.0, C,
                            1024, X.make_sgemm_opts(split_k=4)) == X.XPOSE_EWORKSPACE
    assert X.strerror(X.XPOSE_EWORKSPACE).startswith("workspace")


@pytest.mark.parametrize("m, n, k, splits, split_len", [
    # each within 0.96 of the fastest split measured on MI355X (1 to 32
    # slices), most of them the fastest
    (1024, 1024, 1024, 4, 256),     # 64 blocks: one per compute unit
    (1024, 1024, 4096, 8, 512),
    (2048, 2048, 2048, 4, 512),     # 256 blocks
    (1536, 1536, 1536, 5, 320),     # 144 blocks: 4 slices unbalance
    (768, 768, 768, 7, 112),        # 36 blocks: short slices still pay
    (512, 512, 512, 8, 64),
    (2560, 2560, 2560, 5, 512),
    (3072, 3072, 3072, 3, 1024),    # 576 blocks
    (4100, 4100, 4100, 3, 1376),    # 1089 blocks: 65 in a second round
    (4096, 4096, 4096, 1, 4096),    # 512 blocks of 256 rows: full rounds
    (3072, 4096, 4096, 1, 4096),    # 768 blocks
    (6144, 6144, 6144, 1, 6144),
    (8192, 8192, 2048, 1, 2048),
    (100, 100, 100000, 64, 1568)])  # one block: at most 64 slices
def test_library_split_rule(m, n, k, splits, split_len):
    rc, info = plan_ws(m, n, k)
    assert rc == 0
    assert (info.splits, info.split_len) == (splits, split_len)
    tiles = -(-m // info.tile_m) * -(-n // 128)
    assert info.tiles == tiles * splits
    assert info.workspace_bytes == (4 * splits * m * n if splits > 1 else 0)
    assert info.workspace_wanted == info.workspace_bytes
    assert (splits - 1) * split_len < k <= splits * split_len


def test_library_split_shrinks_to_the_workspace():
    plane = 1024 * 1024 * 4
    for ws_bytes, splits in ((4 * plane, 4), (4 * plane - 4, 3),
                             (2 * plane + 7, 2), (2 * plane - 1, 1), (0, 1)):
        rc, info = plan_ws(ws_bytes=ws_bytes)
        assert rc == 0 and info.splits == splits, ws_bytes
        assert info.workspace_bytes <= ws_bytes
        assert info.workspace_wanted == 4 * plane
    # no split: the workspace is not used and may be NULL
    rc, info = plan_ws(ws=0, ws_bytes=0)
    assert rc == 0 and info.splits == 1


@pytest.mark.parametrize("k, split_k, splits, split_len", [
    (1000, 3, 3, 336), (1000, 4, 4, 256), (450, 64, 57, 8 * 1),
    (16, 4, 1, 16), (17, 2, 2, 16), (0, 8, 1, 0), (4096, 1, 1, 4096),
    (4096, 2, 2, 2048)])
def test_explicit_split(k, split_k, splits, split_len):
    """split_k slices of ceil(k / split_k) rounded up to whole k steps."""
    bk = 8 if split_k == 64 else 16
    opts = X.make_sgemm_opts(bk=bk, split_k=split_k)
    rc, info = plan_ws(m=300, n=200, k=k, opts=opts)
    assert rc == 0
    assert (info.splits, info.split_len) == (splits, split_len)
    assert info.split_len % info.bk == 0 or splits == 1


def test_split_validation():
    plane = 1024 * 1024 * 4
    four = X.make_sgemm_opts(split_k=4)
    rc, info = plan_ws(opts=four, ws_bytes=4 * plane - 1)
    assert rc == X.XPOSE_EWORKSPACE
    assert info.workspace_wanted == 4 * plane and info.splits == 0
    rc, info = plan_ws(opts=four, ws=0, ws_bytes=0)     # the size query
    assert rc == X.XPOSE_EWORKSPACE and info.workspace_wanted == 4 * plane
    assert plan_ws(opts=four, ws_bytes=4 * plane)[0] == 0
    assert plan_ws(opts=X.make_sgemm_opts(split_k=65))[0] == X.XPOSE_EINVAL
    assert plan_ws(opts=X.make_sgemm_opts(split_k=-1))[0] == X.XPOSE_EINVAL
    assert plan_ws(ws_bytes=-1)[0] == X.XPOSE_EINVAL
    assert plan_ws(ws=0)[0] == X.XPOSE_EINVAL          # a split needs it
    assert plan_ws(ws=WS + 2)[0] == X.XPOSE_EALIGN
    assert plan_ws(ws=WS + 4)[0] == 0
    # the workspace may not overlap A, B or C (over the bytes it uses)
    assert plan_ws(ws=C + 4 * 1024 * 1024 - 4)[0] == X.XPOSE_EALIAS
    assert plan_ws(ws=A - 4 * plane + 4)[0] == X.XPOSE_EALIAS
    assert plan_ws(ws=A - 4 * plane)[0] == 0
    assert plan_ws(ws=B)[0] == X.XPOSE_EALIAS
    # a workspace larger than the split uses may overlap C beyond those bytes
    assert plan_ws(ws=C - 4 * plane, ws_bytes=1 << 40)[0] == 0
    # split_k 1: never, whatever the workspace
    rc, info = plan_ws(opts=X.make_sgemm_opts(split_k=1))
    assert rc == 0 and info.splits == 1 and info.workspace_wanted == 0
    # the xpose_sgemm_ws call validates the same way before launching
    assert X.xpose_sgemm_ws(1024, 1024, 1024, 1.0, A, 1024, B, 1024, 0.0, C,
                            1024, four, WS, 4 * plane - 1) == X.XPOSE_EWORKSPACE
    assert X.xpose_sgemm_ws(1024, 1024, 1024, 1.0, A, 1024, B, 1024, 0.0, C,
                            1024, None, B, 1 << 40) == X.XPOSE_EALIAS


def test_noalloc_validates_before_touching_the_gpu():
    """xpose_sgemm_noalloc checks its arguments, and an explicit split
    against its 64 MiB scratch, before it looks the scratch up or launches
    anything."""
    assert X.SGEMM_SCRATCH_BYTES == 64 << 20
    assert X.xpose_sgemm_noalloc(1024, 1024, 1024, 1.0, A, 1000, B, 1024,
                                 0.0, C, 1024) == X.XPOSE_EINVAL
    assert X.xpose_sgemm_noalloc(1024, 1024, 1024, 1.0, A, 1024, B, 1024,
                                 0.0, A, 1024) == X.XPOSE_EALIAS
    # 1024 x 1024 planes are 4 MiB: 16 fit, 17 (k = 17 * 256) do not
    assert X.xpose_sgemm_noalloc(1024, 1024, 4352, 1.0, A, 4352, B, 1024,
                                 0.0, C, 1024,
                                 X.make_sgemm_opts(split_k=17)) == X.XPOSE_EWORKSPACE
    assert X.xpose_sgemm_noalloc(0, 1024, 4096, 1.0, 0, 4096, 0, 1024, 0.0,
                                 0, 1024) == X.XPOSE_OK
