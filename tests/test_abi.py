"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/xpose.h declares, and validates arguments on the host
(bogus pointer values are fine here: invalid calls return before anything
is launched, and xpose_plan never dereferences)."""
import ctypes
import glob
import os
import re

import pytest

import lds_tiled_matrix_amd as X

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("xpose.h", "xpose_sgemm.h")]

IN = 0x7f0000000000       # pretend device addresses, 256-byte aligned
OUT = 0x7f1000000000


def declared_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(xpose_\w+)\s*\(", text))
    return sorted(names)


def test_every_header_is_known():
    assert sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))) == sorted(HEADERS)


def test_header_and_binding_agree():
    assert declared_functions() == sorted(X.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(X.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_codes():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = X.strerror(code)
        assert s and s != X.strerror(-99)
    assert X.strerror(-99) == "unknown status code"


def plan(out=OUT, inp=IN, batch=1, rows=64, cols=64, ld_in=None, ld_out=None,
         stride_in=0, stride_out=0, dtype=X.XPOSE_F32, opts=None):
    ld_in = cols if ld_in is None else ld_in
    ld_out = rows if ld_out is None else ld_out
    return X.xpose_plan(out, inp, batch, rows, cols, ld_in, ld_out, stride_in,
                        stride_out, dtype, opts)


def test_valid_plan_defaults():
    # 8192^2 fp32 (512 MiB read + write): 128 x 128 tiles in diagonal order,
    # one workgroup per compute unit
    rc, info = plan(rows=8192, cols=8192)
    assert rc == X.XPOSE_OK
    assert (info.tile_rows, info.tile_cols) == (128, 128)
    assert info.layout == X.LAYOUT_SWIZZLE and info.order == X.ORDER_DIAGONAL
    assert info.cache == X.CACHE_NT_STORE and info.xcd_remap == 0
    assert info.occupancy == 1
    assert info.vector_path == 1 and info.tiles == 64 * 64
    assert info.launches == 1 and info.threads == 256
    assert info.lds_bytes == 128 * 128 * 4
    # 4096^2 fp32: 32 x 32 tiles in 8 x 32 super-tiles, per-XCD ranges
    rc, info = plan(rows=4096, cols=4096)
    assert rc == X.XPOSE_OK
    assert (info.tile_rows, info.tile_cols) == (32, 32)
    assert info.cache == X.CACHE_NT_STORE and info.xcd_remap == 1
    assert (info.group_rows, info.group_cols) == (8, 32)
    assert info.tiles == 128 * 128 and info.occupancy == 0
    assert info.lds_bytes == 32 * 32 * 4


def test_occupancy_option():
    rc, info = plan(rows=4096, cols=4096, opts=X.make_opts(occupancy=3))
    assert rc == 0 and info.occupancy == 3
    # -1: no cap, even where the default has one
    rc, info = plan(rows=8192, cols=8192, opts=X.make_opts(occupancy=-1))
    assert rc == 0 and info.occupancy == 0 and info.tile_rows == 128
    # the default cap belongs to the default tile
    rc, info = plan(rows=8192, cols=8192, opts=X.make_opts(tile=(64, 64)))
    assert rc == 0 and info.occupancy == 0
    for bad in (-2, 65):
        assert plan(opts=X.make_opts(occupancy=bad))[0] == X.XPOSE_EINVAL
    assert plan(opts=X.make_opts(occupancy=2, persistent=2))[0] == X.XPOSE_EINVAL
    # naive kernels have no LDS to reserve: the cap is not reported
    rc, info = plan(opts=X.make_opts(layout=X.LAYOUT_NAIVE_READ, occupancy=2))
    assert rc == 0 and info.occupancy == 0


def test_ragged_and_batched_tile_counts():
    # Odd pitches: output rows are not line-aligned, so line-aligned output
    # tiles are chosen, with one extra tile row for the shifted segments.
    # From 512 MiB moved on, 64 x 128 tiles; below, 64 x 64.
    rc, info = plan(rows=12345, cols=6789)
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (64, 128)
    assert info.aligned_out == 1 and info.cache == X.CACHE_NT_STORE
    assert info.tiles == 194 * 54 and info.vector_path == 1
    assert (info.group_rows, info.group_cols) == (1, 54)
    rc, info = plan(rows=8193, cols=8191)   # 4 bytes short of 512 MiB moved
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (64, 64)
    assert info.aligned_out == 1 and info.tiles == 129 * 128
    assert (info.group_rows, info.group_cols) == (1, 64)
    # 12288 rows fill 192 tile rows; shifted segments need a 193rd.
    rc, info = plan(rows=12288, cols=6789, ld_out=12289)
    assert rc == 0 and info.aligned_out == 1 and info.tiles == 193 * 54
    rc, info = plan(rows=12288, cols=6789)
    assert rc == 0 and info.aligned_out == 0 and info.tiles == 384 * 213
    # A batch of small matrices: taller tiles, small super-tiles.
    rc, info = plan(batch=64, rows=2048, cols=1024, stride_in=2048 * 1024,
                    stride_out=1024 * 2048)
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (128, 64)
    assert info.tiles == 64 * 16 * 16 and info.xcd_remap == 0


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), X.XPOSE_EINVAL),
    (dict(cols=-5), X.XPOSE_EINVAL),
    (dict(batch=-1), X.XPOSE_EINVAL),
    (dict(ld_in=63), X.XPOSE_EINVAL),
    (dict(ld_out=63), X.XPOSE_EINVAL),
    (dict(inp=0), X.XPOSE_EINVAL),
    (dict(out=0), X.XPOSE_EINVAL),
    (dict(dtype=7), X.XPOSE_EDTYPE),
    (dict(dtype=-1), X.XPOSE_EDTYPE),
    (dict(inp=IN + 2), X.XPOSE_EALIGN),
    (dict(out=OUT + 1, dtype=X.XPOSE_F16), X.XPOSE_EALIGN),
    # output starts inside the input
    (dict(out=IN + 64 * 4), X.XPOSE_EALIAS),
    # input starts inside the output
    (dict(inp=OUT + 4 * 63 * 64), X.XPOSE_EALIAS),
    # batch outputs would overlap each other
    (dict(batch=2, stride_in=4096, stride_out=100), X.XPOSE_EINVAL),
    (dict(batch=2, stride_in=-1, stride_out=4096), X.XPOSE_EINVAL),
    # extents that overflow int64
    (dict(rows=1 << 40, cols=1 << 40), X.XPOSE_EINVAL),
])
def test_invalid_calls_rejected(kw, code):
    rc, info = plan(**kw)
    assert rc == code
    assert info.tiles == 0


def test_invalid_calls_rejected_by_entry_points_too():
    # The real entry points validate first and return without launching.
    assert X.xpose_2d(OUT, IN, 64, 64, 63, 64, X.XPOSE_F32, 0) == X.XPOSE_EINVAL
    assert X.xpose_2d(IN, IN, 64, 64, 64, 64, X.XPOSE_F32, 0) == X.XPOSE_EALIAS
    assert X.xpose_batched(OUT, IN, 2, 8, 8, 8, 8, 64, 1, 9, 0) == X.XPOSE_EDTYPE
    assert X.xpose_copy(OUT, IN, -1, 0) == X.XPOSE_EINVAL
    assert X.xpose_copy(IN + 8, IN, 64, 0) == X.XPOSE_EALIAS
    assert X.xpose_copy(0, IN, 64, 0) == X.XPOSE_EINVAL
    assert X.xpose_lds_probe(OUT, [0] * 64, 12, 0, 10) == X.XPOSE_EINVAL
    assert X.xpose_lds_probe(OUT, [16384] * 64, 4, 0, 10) == X.XPOSE_EINVAL
    assert X.xpose_lds_probe(OUT, [2] * 64, 4, 0, 10) == X.XPOSE_EINVAL
    assert X.xpose_lds_probe(OUT, [0] * 64, 4, 0, 0) == X.XPOSE_EINVAL


def test_2d_ex_validates_like_the_batched_call():
    # xpose_2d_ex is xpose_batched_ex with batch 1: same host validation,
    # including every opts field, before anything is launched.
    assert X.xpose_2d_ex(OUT, IN, 64, 64, 63, 64, X.XPOSE_F32) == X.XPOSE_EINVAL
    assert X.xpose_2d_ex(IN, IN, 64, 64, 64, 64, X.XPOSE_F32) == X.XPOSE_EALIAS
    assert X.xpose_2d_ex(OUT, IN + 2, 64, 64, 64, 64, X.XPOSE_F32) == X.XPOSE_EALIGN
    assert X.xpose_2d_ex(OUT, IN, 64, 64, 64, 64, 11) == X.XPOSE_EDTYPE
    for bad in (X.make_opts(layout=9), X.make_opts(cache=7),
                X.make_opts(flags=1 << 20), X.make_opts(order=5),
                X.make_opts(flags=X.FLAG_ALIGN_OUT | X.FLAG_TR_READ)):
        assert X.xpose_2d_ex(OUT, IN, 64, 64, 64, 64, X.XPOSE_F32,
                             bad) == X.XPOSE_EINVAL
        assert X.xpose_batched_ex(OUT, IN, 1, 64, 64, 64, 64, 0, 0,
                                  X.XPOSE_F32, bad) == X.XPOSE_EINVAL
    # An unbuilt tile shape is reported, not launched.
    assert X.xpose_2d_ex(OUT, IN, 64, 64, 64, 64, X.XPOSE_F32,
                         X.make_opts(tile=(48, 48))) == X.XPOSE_ENOTILE
    assert X.xpose_2d_ex(0, 0, 0, 7, 7, 0, X.XPOSE_U8,
                         X.make_opts(layout=X.LAYOUT_PAD1)) == X.XPOSE_OK


def test_binding_rejects_host_tensors():
    # The torch conveniences check where the tensors live before calling the
    # library, so a host tensor never reaches a kernel.
    torch = pytest.importorskip("torch")
    a = torch.zeros(8, 8)
    with pytest.raises(ValueError, match="CUDA tensor"):
        X.transpose(a)
    with pytest.raises(ValueError, match="CUDA tensor"):
        X.copy(torch.zeros(8, 8), a)
    with pytest.raises(ValueError, match="CUDA tensor"):
        X.sgemm(a, a)
    with pytest.raises(ValueError, match="CUDA tensor"):
        X.sgemm(a, a, torch.zeros(8, 8))


def test_zero_sizes_are_noops_even_with_null_pointers():
    for b, r, c in ((0, 5, 5), (1, 0, 5), (1, 5, 0)):
        assert X.xpose_batched(0, 0, b, r, c, 5, 5, 25, 25, X.XPOSE_F32, 0) == 0
        rc, info = X.xpose_plan(0, 0, b, r, c, 5, 5, 25, 25, X.XPOSE_F32, None)
        assert rc == 0 and info.tiles == 0
    assert X.xpose_2d(0, 0, 0, 0, 0, 0, X.XPOSE_F16, 0) == 0
    assert X.xpose_copy(0, 0, 0, 0) == 0


def test_vector_path_rules():
    # 128-bit accesses at any alignment: odd pitches and shifted pointers of
    # 1- and 2-byte elements keep the vector path ...
    assert plan(dtype=X.XPOSE_F16, rows=64, cols=64)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_F16, rows=64, cols=63, ld_in=63)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_F16, rows=63, cols=64, ld_out=63)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_F16, inp=IN + 2)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_U8, rows=128, cols=128)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_U8, rows=128, cols=130, ld_in=130)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_U8, inp=IN + 1, out=OUT + 3)[1].vector_path == 1
    assert plan(rows=12345, cols=6789)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_F64, rows=33, cols=31)[1].vector_path == 1
    # ... except into direct global->LDS loads, which need 4-byte aligned
    # input rows (output rows may be anything)
    direct = X.make_opts(tile=(128, 64), flags=X.FLAG_TR_READ | X.FLAG_DIRECT_LDS)
    assert plan(dtype=X.XPOSE_F16, rows=256, cols=128, opts=direct)[1].vector_path == 1
    assert plan(dtype=X.XPOSE_F16, rows=256, cols=128, ld_in=129, opts=direct)[1].vector_path == 0
    assert plan(dtype=X.XPOSE_F16, rows=256, cols=128, inp=IN + 2, opts=direct)[1].vector_path == 0
    assert plan(dtype=X.XPOSE_F16, rows=256, cols=128, ld_out=257, opts=direct)[1].vector_path == 1
    forced = X.XposeOpts(0, 0, 0, X.FLAG_ELEMENTWISE)
    assert plan(opts=forced)[1].vector_path == 0


def test_opts_select_layout_and_tile():
    for layout in (X.LAYOUT_UNPADDED, X.LAYOUT_PAD1, X.LAYOUT_SWIZZLE):
        rc, info = plan(opts=X.XposeOpts(layout, 32, 32, 0))
        assert rc == 0 and info.layout == layout
        assert (info.tile_rows, info.tile_cols) == (32, 32)
    # The one-word pad on the default 32 x 32 fp32 tile is the pages'
    # 4,224-byte tile[32][33].
    assert plan(opts=X.XposeOpts(X.LAYOUT_PAD1, 0, 0, 0))[1].lds_bytes == 4224
    assert plan(opts=X.XposeOpts(X.LAYOUT_UNPADDED, 0, 0, 0))[1].lds_bytes == 4096
    rc, info = plan(opts=X.make_opts(tile=(32, 32), threads=64))
    assert rc == 0 and info.threads == 64
    assert plan(opts=X.make_opts(tile=(32, 32), threads=96))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.XposeOpts(0, 48, 48, 0))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.XposeOpts(9, 0, 0, 0))[0] == X.XPOSE_EINVAL
    assert plan(opts=X.XposeOpts(0, 0, 0, 512))[0] == X.XPOSE_EINVAL


def test_large_batch_splits_launches():
    # 2**31 workgroups is over the grid limit: the plan splits the batch.
    rc, info = plan(batch=1 << 20, rows=4096, cols=4096,
                    stride_in=4096 * 4096, stride_out=4096 * 4096,
                    out=0x100000000000000, inp=0x10000)
    assert rc == 0
    per = (4096 // info.tile_rows) * (4096 // info.tile_cols)
    assert info.tiles == (1 << 20) * per
    assert info.launches == -(-info.tiles // (0x7fffffff // per * per))


def test_one_hip_runtime_per_process():
    """Importing the binding (before or after torch) must leave exactly one
    HIP runtime mapped: two runtimes in one process give each its own device
    context, and launches on the other runtime's memory fail or crash."""
    import subprocess
    import sys
    probe = ("import lds_tiled_matrix_amd, torch; "
             "print(len({l.split()[-1] for l in open('/proc/self/maps') "
             "if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", probe], capture_output=True,
                         text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr[-500:]
    assert out.stdout.strip() == "1"


def test_footprint_rules():
    # One large fp16 matrix (>= 256 MiB moved, both sides >= 1024): 256 x 256
    # tiles of 128 KiB (one workgroup per compute unit) in the diagonal order.
    rc, info = plan(rows=16384, cols=16384, dtype=X.XPOSE_F16)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert (info.tile_rows, info.tile_cols, info.threads) == (256, 256, 256)
    assert info.xcd_remap == 0 and info.occupancy == 0
    assert info.lds_bytes == 128 * 1024
    rc, info = plan(rows=8192, cols=8192, dtype=X.XPOSE_F16)  # 256 MiB
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert (info.tile_rows, info.tile_cols) == (256, 256)
    rc, info = plan(rows=6144, cols=6144, dtype=X.XPOSE_F16)  # 144 MiB
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES
    assert (info.tile_rows, info.tile_cols) == (128, 64)
    rc, info = plan(rows=65536, cols=512, dtype=X.XPOSE_F16)  # narrow
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (128, 64)
    # A batch moving at least 512 MiB: the diagonal order, 128 x 64 tiles,
    # at most 3 workgroups per compute unit.
    rc, info = plan(batch=4, rows=8192, cols=8192, stride_in=8192 * 8192,
                    stride_out=8192 * 8192, dtype=X.XPOSE_F16)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert (info.tile_rows, info.tile_cols) == (128, 64) and info.occupancy == 3
    # 4-byte elements from 1 GiB on (in the diagonal order's pitches):
    # 256 x 128 tiles of 128 KiB.
    rc, info = plan(rows=16384, cols=8192)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL and info.occupancy == 0
    assert (info.tile_rows, info.tile_cols) == (256, 128)
    # 8-byte elements from 256 MiB on, output rows a multiple of 32 KiB
    # apart: 128 x 128 tiles of 128 KiB.
    rc, info = plan(rows=8192, cols=8192, dtype=X.XPOSE_F64)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert (info.tile_rows, info.tile_cols) == (128, 128) and info.occupancy == 0
    rc, info = plan(rows=4096, cols=4096, dtype=X.XPOSE_F64)  # 256 MiB
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert (info.tile_rows, info.tile_cols) == (128, 128)
    rc, info = plan(rows=4096, cols=2048, dtype=X.XPOSE_F64)  # 128 MiB
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES
    assert (info.tile_rows, info.tile_cols) == (32, 32)
    # 8192^2 fp32 moves exactly 512 MiB: big.
    rc, info = plan(rows=8192, cols=8192)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert (info.tile_rows, info.tile_cols) == (128, 128)
    # 1-byte elements: 128 x 64 tiles of 128 threads, at most 4 per CU.
    rc, info = plan(rows=32768, cols=16384, dtype=X.XPOSE_U8)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL and info.occupancy == 4
    assert (info.tile_rows, info.tile_cols, info.threads) == (128, 64, 128)
    # Just under 512 MiB, output rows 48 KiB apart: compact super-tiles, no
    # cap.
    rc, info = plan(rows=12288, cols=5461)
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES and info.occupancy == 0
    # 4-byte elements: the diagonal order only where output rows lie (nearly)
    # a multiple of 32 KiB apart
    rc, info = plan(rows=12288, cols=12288)
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES
    assert (info.tile_rows, info.tile_cols) == (32, 32) and info.occupancy == 0
    rc, info = plan(rows=8192, cols=8192, ld_in=8224, ld_out=8224)
    assert rc == 0 and info.order == X.ORDER_DIAGONAL and info.occupancy == 1
    rc, info = plan(rows=12288, cols=8192, ld_out=16384 + 32)  # 128 B off 64 KiB
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    rc, info = plan(rows=12288, cols=8192, ld_out=16384 + 256)  # 1 KiB off
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES
    # ... also under 512 MiB for one matrix of at least 1024 x 1024: 256 x
    # 128 tiles, except where output rows lie 128 KiB apart with more than
    # 2048 columns, and at 8192^2 (128 x 128 tiles, one workgroup per
    # compute unit)
    for rows, cols in ((8192, 1024), (8192, 4096), (16384, 2048),
                       (32768, 1024), (32768, 2048), (65536, 4096),
                       (16384, 4096), (8192, 16384)):
        rc, info = plan(rows=rows, cols=cols)
        assert rc == 0 and info.order == X.ORDER_DIAGONAL
        assert (info.tile_rows, info.tile_cols) == (256, 128)
    for rows, cols in ((32768, 4096), (32768, 8192), (32768, 16384),
                       (8192, 8192)):
        rc, info = plan(rows=rows, cols=cols)
        assert rc == 0 and info.order == X.ORDER_DIAGONAL
        assert (info.tile_rows, info.tile_cols) == (128, 128)
        assert info.occupancy == 1
    for rows, cols in ((4096, 4096), (1024, 8192), (8192, 512)):
        rc, info = plan(rows=rows, cols=cols)
        assert rc == 0 and info.order == X.ORDER_SUPER_TILES
        assert (info.tile_rows, info.tile_cols) == (32, 32)
    # a batch under 512 MiB keeps super-tiles
    rc, info = plan(batch=2, rows=8192, cols=2048, stride_in=8192 * 2048,
                    stride_out=8192 * 2048)
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES
    # an explicit order drops the default cap
    rc, info = plan(batch=4, rows=8192, cols=8192, stride_in=8192 * 8192,
                    stride_out=8192 * 8192, dtype=X.XPOSE_F16,
                    opts=X.make_opts(order=X.ORDER_SUPER_TILES))
    assert rc == 0 and info.occupancy == 0 and info.tile_rows == 128
    # A batch of small matrices keeps super-tiles even when the call is big.
    rc, info = plan(batch=64, rows=2048, cols=1024, stride_in=2048 * 1024,
                    stride_out=1024 * 2048)
    assert rc == 0 and info.order == X.ORDER_SUPER_TILES
    # Explicit order wins.
    rc, info = plan(opts=X.make_opts(order=X.ORDER_DIAGONAL))
    assert rc == 0 and info.order == X.ORDER_DIAGONAL
    assert plan(opts=X.make_opts(order=4))[0] == X.XPOSE_EINVAL
    rc, info = plan(rows=1024, cols=1024,
                    opts=X.make_opts(order=X.ORDER_COLUMN_BANDS, group_cols=16))
    assert rc == 0 and info.order == X.ORDER_COLUMN_BANDS and info.group_cols == 16


def test_naive_plans():
    rc, info = plan(rows=100, cols=700, opts=X.XposeOpts(X.LAYOUT_NAIVE_READ, 0, 0, 0))
    assert rc == 0 and info.layout == X.LAYOUT_NAIVE_READ and info.lds_bytes == 0
    assert info.tiles == 3 * 100
    rc, info = plan(rows=100, cols=700, opts=X.XposeOpts(X.LAYOUT_NAIVE_WRITE, 0, 0, 0))
    assert rc == 0 and info.tiles == 1 * 700
    assert plan(opts=X.XposeOpts(6, 0, 0, 0))[0] == X.XPOSE_EINVAL


def test_persistent_option():
    rc, info = plan(opts=X.make_opts(persistent=4))
    assert rc == 0 and info.persistent == 4
    # only the swizzled layout is built persistent
    assert plan(opts=X.make_opts(layout=X.LAYOUT_PAD1, persistent=2))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.make_opts(persistent=-1))[0] == X.XPOSE_EINVAL
    assert plan(opts=X.make_opts(persistent=65))[0] == X.XPOSE_EINVAL


def test_direct_lds_option():
    rc, info = plan(opts=X.make_opts(tile=(32, 32), flags=X.FLAG_DIRECT_LDS))
    assert rc == 0 and info.direct_lds == 1
    rc, info = plan(opts=X.make_opts(tile=(32, 32)))
    assert rc == 0 and info.direct_lds == 0
    # not built for packed sub-word elements or the padded layout
    assert plan(dtype=X.XPOSE_F16, opts=X.make_opts(flags=X.FLAG_DIRECT_LDS))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.make_opts(layout=X.LAYOUT_PAD1, flags=X.FLAG_DIRECT_LDS))[0] == X.XPOSE_ENOTILE


def test_align_out_option():
    # fp32 with line-aligned output rows: the ordinary tiles
    assert plan(rows=8192, cols=8192)[1].aligned_out == 0
    # output pitch off the line: aligned-out tiles by default, either way
    # selectable explicitly
    assert plan(rows=1000, cols=512)[1].aligned_out == 1
    assert plan(rows=1000, cols=512, opts=X.make_opts(flags=X.FLAG_NO_ALIGN_OUT))[1].aligned_out == 0
    rc, info = plan(rows=1024, cols=512, opts=X.make_opts(tile=(64, 64), flags=X.FLAG_ALIGN_OUT))
    assert rc == 0 and info.aligned_out == 1 and info.tiles == 17 * 8
    # 2- and 8-byte elements on request; not 1-byte elements, other layouts
    # or contradicting flags
    for dt, s in ((X.XPOSE_F16, 2), (X.XPOSE_BF16, 2), (X.XPOSE_F64, 8)):
        rc, info = plan(rows=1000, cols=512, ld_out=1001, dtype=dt,
                        opts=X.make_opts(flags=X.FLAG_ALIGN_OUT))
        assert rc == 0 and info.aligned_out == 1
        assert info.tiles == -(-(1000 + 128 // s - 1) // info.tile_rows) * -(-512 // info.tile_cols)
    assert plan(dtype=X.XPOSE_U8, opts=X.make_opts(flags=X.FLAG_ALIGN_OUT))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.make_opts(layout=X.LAYOUT_PAD1, flags=X.FLAG_ALIGN_OUT))[0] == X.XPOSE_ENOTILE
    assert plan(opts=X.make_opts(flags=X.FLAG_ALIGN_OUT | X.FLAG_ELEMENTWISE))[0] == X.XPOSE_EINVAL
    # an explicit knob with no aligned-out kernel falls back to the ordinary
    # tiles, with their defaults (write-back stores for unaligned rows)
    rc, info = plan(rows=1000, cols=512, opts=X.make_opts(tile=(32, 32)))
    assert rc == 0 and info.aligned_out == 0 and info.cache == X.CACHE_DEFAULT
    rc, info = plan(rows=1000, cols=512, opts=X.make_opts(tile=(32, 32), cache=X.CACHE_NT_STORE))
    assert rc == 0 and info.aligned_out == 0 and info.cache == X.CACHE_NT_STORE
    rc, info = plan(rows=1000, cols=512, opts=X.make_opts(layout=X.LAYOUT_PAD1))
    assert rc == 0 and info.aligned_out == 0 and info.layout == X.LAYOUT_PAD1
    rc, info = plan(rows=1000, cols=512, opts=X.make_opts(tile=(64, 64), cache=X.CACHE_NT_ALL))
    assert rc == 0 and info.aligned_out == 0 and info.cache == X.CACHE_NT_ALL
    # ... but not when aligned-out tiles were asked for
    assert plan(rows=1000, cols=512, opts=X.make_opts(tile=(32, 32), flags=X.FLAG_ALIGN_OUT))[0] == X.XPOSE_ENOTILE
    # 2-byte elements: by default only from 256 rows on (a short matrix pays
    # more for the halo tile row than whole lines gain); on request always
    kw = dict(dtype=X.XPOSE_F16, batch=40, cols=600, stride_in=600 * 1000,
              stride_out=600 * 1000)
    assert plan(rows=255, ld_out=255, **kw)[1].aligned_out == 0
    assert plan(rows=256, ld_out=257, **kw)[1].aligned_out == 1
    assert plan(rows=150, ld_out=150, opts=X.make_opts(flags=X.FLAG_ALIGN_OUT), **kw)[1].aligned_out == 1
    assert plan(rows=150, ld_out=150, dtype=X.XPOSE_F32, batch=40, cols=600,
                stride_in=600 * 150, stride_out=600 * 150)[1].aligned_out == 1
    # 2-byte calls of 128 MiB (read + write) or more take 128 x 64
    # line-aligned tiles in column bands, smaller ones 64 x 64 super-tiles
    for r, c in ((16383, 16383), (9999, 9999), (5793, 5793)):
        rc, info = plan(rows=r, cols=c, ld_out=r, dtype=X.XPOSE_F16)
        assert rc == 0 and info.aligned_out == 1
        assert (info.tile_rows, info.tile_cols) == (128, 64), (r, c)
        assert info.order == X.ORDER_COLUMN_BANDS
    for r, c in ((5791, 5791), (4097, 4097)):
        rc, info = plan(rows=r, cols=c, ld_out=r, dtype=X.XPOSE_F16)
        assert rc == 0 and info.aligned_out == 1
        assert (info.tile_rows, info.tile_cols) == (64, 64), (r, c)
        assert info.order == X.ORDER_SUPER_TILES
    # asked for on line-aligned rows: the aligned-out default tile
    rc, info = plan(rows=8192, cols=8192, opts=X.make_opts(flags=X.FLAG_ALIGN_OUT))
    assert rc == 0 and info.aligned_out == 1 and info.tiles == -(-(8192 + 31) // info.tile_rows) * (8192 // info.tile_cols)


def test_tr_read_option():
    """LDS transpose-read tiles: 1- and 2-byte elements, swizzled layout."""
    f16, u8 = X.XPOSE_F16, X.XPOSE_U8
    rc, info = plan(rows=8192, cols=8192, dtype=f16, opts=X.make_opts(flags=X.FLAG_TR_READ))
    assert rc == 0 and info.tr_read == 1 and info.layout == X.LAYOUT_SWIZZLE
    assert info.lds_bytes == info.tile_rows * info.tile_cols * 2
    rc, info = plan(rows=4096, cols=4096, dtype=u8, opts=X.make_opts(flags=X.FLAG_TR_READ))
    assert rc == 0 and info.tr_read == 1
    assert info.lds_bytes == info.tile_rows * info.tile_cols
    # bf16 moves by size like fp16
    assert plan(dtype=X.XPOSE_BF16, opts=X.make_opts(flags=X.FLAG_TR_READ))[1].tr_read == 1
    # combined with direct loads
    rc, info = plan(rows=8192, cols=8192, dtype=f16,
                    opts=X.make_opts(tile=(128, 64), flags=X.FLAG_TR_READ | X.FLAG_DIRECT_LDS))
    assert rc == 0 and info.tr_read == 1 and info.direct_lds == 1
    # without the flag: the packed-register tiles
    assert plan(dtype=f16)[1].tr_read == 0
    # not for 4- or 8-byte elements, other layouts, persistent workgroups
    assert plan(opts=X.make_opts(flags=X.FLAG_TR_READ))[0] == X.XPOSE_ENOTILE
    assert plan(dtype=X.XPOSE_F64, opts=X.make_opts(flags=X.FLAG_TR_READ))[0] == X.XPOSE_ENOTILE
    assert plan(dtype=f16, opts=X.make_opts(layout=X.LAYOUT_PAD1, flags=X.FLAG_TR_READ))[0] == X.XPOSE_ENOTILE
    assert plan(dtype=f16, opts=X.make_opts(flags=X.FLAG_TR_READ, persistent=1))[0] == X.XPOSE_ENOTILE
    assert plan(dtype=f16, opts=X.make_opts(tile=(32, 32), flags=X.FLAG_TR_READ))[0] == X.XPOSE_ENOTILE
    # contradicts line-aligned output tiles
    assert plan(opts=X.make_opts(flags=X.FLAG_TR_READ | X.FLAG_ALIGN_OUT))[0] == X.XPOSE_EINVAL
    # unaligned fp32 output rows with the flag: no line-aligned default either
    assert plan(rows=1000, cols=512, opts=X.make_opts(flags=X.FLAG_TR_READ))[0] == X.XPOSE_ENOTILE


def test_auto_cache_takes_a_built_policy():
    # fp16 64 x 32 transpose-read tiles are built with non-temporal stores
    # only; unaligned rows default to write-back, so AUTO takes the other.
    opts = X.make_opts(tile=(64, 32), flags=X.FLAG_TR_READ)
    rc, info = plan(rows=100, cols=100, ld_in=101 * 2, ld_out=103 * 2,
                    dtype=X.XPOSE_F16, opts=opts)
    assert rc == 0 and info.cache == X.CACHE_NT_STORE
    explicit = X.make_opts(tile=(64, 32), flags=X.FLAG_TR_READ, cache=X.CACHE_DEFAULT)
    assert plan(rows=100, cols=100, ld_in=202, ld_out=206, dtype=X.XPOSE_F16,
                opts=explicit)[0] == X.XPOSE_ENOTILE


def test_big_f64_default_follows_the_pitch():
    # One large matrix: 128 x 128 tiles (128 KiB, one workgroup per compute
    # unit) in the diagonal order where output rows lie a multiple of 32 KiB
    # apart but not of 128 KiB; 32 x 32 tiles in 16 x 16 super-tiles
    # elsewhere from 512 MiB on
    rc, info = plan(rows=12288, cols=12288, dtype=X.XPOSE_F64)
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (128, 128)
    assert info.order == X.ORDER_DIAGONAL and info.cache == X.CACHE_NT_STORE
    assert info.occupancy == 0
    for rows, cols in ((16384, 16384), (16384, 4096), (16384, 3000), (6000, 6000),
                       (10000, 8000)):
        rc, info = plan(rows=rows, cols=cols, dtype=X.XPOSE_F64)
        assert rc == 0 and (info.tile_rows, info.tile_cols) == (32, 32)
        assert info.order == X.ORDER_SUPER_TILES and info.xcd_remap == 1
        assert (info.group_rows, info.group_cols) == (16, 16)
    # 128 KiB apart with 2048 columns, and 384 KiB apart: 128 x 128 tiles
    for rows, cols in ((16384, 2048), (49152, 4096)):
        rc, info = plan(rows=rows, cols=cols, dtype=X.XPOSE_F64)
        assert rc == 0 and (info.tile_rows, info.tile_cols) == (128, 128)
        assert info.order == X.ORDER_DIAGONAL
    # a batch: 32 x 32 tiles at most 4 workgroups per compute unit
    rc, info = plan(batch=2, rows=8192, cols=8192, stride_in=8192 * 8192,
                    stride_out=8192 * 8192, dtype=X.XPOSE_F64)
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (32, 32)
    assert info.order == X.ORDER_DIAGONAL and info.occupancy == 4
    # under 512 MiB off the period: 8 x 32 super-tiles
    rc, info = plan(rows=2048, cols=8192, dtype=X.XPOSE_F64)
    assert rc == 0 and (info.tile_rows, info.tile_cols) == (32, 32)
    assert info.order == X.ORDER_SUPER_TILES
    assert (info.group_rows, info.group_cols) == (8, 32)


def test_store_policy_follows_output_alignment():
    # misaligned input rows with line-aligned output rows: non-temporal stores
    rc, info = plan(rows=1024, cols=1000, ld_in=1001)
    assert rc == 0 and info.cache == X.CACHE_NT_STORE and info.aligned_out == 0
    rc, info = plan(rows=1024, cols=1000, dtype=X.XPOSE_U8, inp=IN + 1)
    assert rc == 0 and info.cache == X.CACHE_NT_STORE
    # output rows off the line: line-aligned output tiles (u8: write-back)
    assert plan(rows=1000, cols=1024)[1].aligned_out == 1
    rc, info = plan(rows=1000, cols=1024, dtype=X.XPOSE_U8)
    assert rc == 0 and info.aligned_out == 0 and info.cache == X.CACHE_DEFAULT


def test_default_tile_falls_back_to_a_built_shape():
    # fp32 with unaligned output rows: the default 128 x 64 tile has no
    # direct-load unpadded kernel; the first built shape that has one is used
    opts = X.make_opts(layout=X.LAYOUT_UNPADDED, flags=X.FLAG_DIRECT_LDS)
    rc, info = plan(rows=1211, cols=1713, ld_out=1213, opts=opts)
    assert rc == 0 and info.direct_lds == 1 and info.layout == X.LAYOUT_UNPADDED
    # an explicit shape without such a kernel is still an error
    opts = X.make_opts(layout=X.LAYOUT_UNPADDED, tile=(128, 64), flags=X.FLAG_DIRECT_LDS)
    assert plan(rows=1211, cols=1713, ld_out=1213, opts=opts)[0] == X.XPOSE_ENOTILE


def test_packed_batches_of_small_matrices():
    dense = dict(batch=1000, rows=16, cols=16, stride_in=256, stride_out=256)
    rc, info = plan(**dense)
    assert rc == 0 and info.packed == 16 and info.tiles == -(-1000 // 16)
    assert (info.tile_rows, info.tile_cols) == (16, 16)
    assert info.cache == X.CACHE_NT_STORE and info.vector_path == 1
    # 3 x 5 fp32 = 60 bytes: 32 matrices make whole lines, 256 fit a block
    rc, info = plan(batch=10000, rows=3, cols=5, stride_in=15, stride_out=15)
    assert rc == 0 and info.packed == 256
    # the XCD flags leave it on; any other knob, a pitch or gap, a single
    # matrix or a larger one selects the tiles
    assert plan(**dense, opts=X.make_opts(flags=X.FLAG_XCD_REMAP))[1].packed == 16
    assert plan(**dense, opts=X.make_opts(tile=(32, 32)))[1].packed == 0
    assert plan(**dense, opts=X.make_opts(flags=X.FLAG_NO_PACKED))[1].packed == 0
    assert plan(batch=1000, rows=16, cols=16, ld_in=17, stride_in=16 * 17,
                stride_out=256)[1].packed == 0
    assert plan(batch=1000, rows=16, cols=16, stride_in=260, stride_out=256)[1].packed == 0
    assert plan(rows=16, cols=16)[1].packed == 0
    assert plan(batch=8, rows=64, cols=64, stride_in=4096, stride_out=4096)[1].packed == 1
    assert plan(batch=8, rows=128, cols=64, stride_in=8192, stride_out=8192)[1].packed == 0
    # 16-32 KiB: packed only when the matrix is not a whole number of tiles
    assert plan(batch=8, rows=64, cols=96, stride_in=6144, stride_out=6144)[1].packed == 1
    assert plan(batch=8, rows=96, cols=96, stride_in=9216, stride_out=9216)[1].packed == 0
    # asked for: also a single matrix
    want = X.make_opts(flags=X.FLAG_PACKED)
    assert plan(rows=16, cols=16, opts=want)[1].packed >= 1
    rc, info = plan(batch=8, rows=128, cols=64, stride_in=8192, stride_out=8192, opts=want)
    assert rc == 0 and info.packed >= 1
    assert plan(batch=8, rows=128, cols=128, stride_in=16384, stride_out=16384,
                opts=want)[0] == X.XPOSE_ENOTILE
    assert plan(batch=8, rows=16, cols=16, ld_in=20, stride_in=320, stride_out=256,
                opts=want)[0] == X.XPOSE_ENOTILE
    assert plan(**dense, opts=X.make_opts(flags=X.FLAG_PACKED | X.FLAG_TR_READ))[0] == X.XPOSE_EINVAL
    assert plan(**dense, opts=X.make_opts(flags=X.FLAG_PACKED | X.FLAG_NO_PACKED))[0] == X.XPOSE_EINVAL
    # an output base off the line: write-back stores
    assert plan(**dense, out=OUT + 4)[1].cache == X.CACHE_DEFAULT
