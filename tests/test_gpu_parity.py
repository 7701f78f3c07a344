"""GPU parity: the HIP path, called through the C ABI, against the oracle,
bit for bit.  Needs an MI355X and the built library."""
import numpy as np
import pytest

import oracle
import workloads as wl
from xpose_testlib import DTYPE_OF_SIZE, check_case, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
X = pytest.importorskip("lds_tiled_matrix_amd")

SIZES = (4, 2, 1, 8)
EDGE_DIMS = (1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129)


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


SIGNED = {1: np.int8, 2: np.int16, 4: np.int32, 8: np.int64}


def _to_dev(a):
    """Host array -> device tensor through a signed view of the same width
    (torch's unsigned 16/32/64-bit support is limited)."""
    if a.dtype.kind == "u" and a.dtype.itemsize > 1:
        a = a.view(SIGNED[a.dtype.itemsize])
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


def _run_workload_tensor(w, host_in):
    """Default launch (the one the benchmark times) on a workload's input."""
    d_in = _to_dev(host_in)
    out_shape = (w.cols, w.rows) if w.batch == 1 else (w.batch, w.cols, w.rows)
    d_out = torch.empty(out_shape, dtype=d_in.dtype, device=_dev())
    code = DTYPE_OF_SIZE[w.elem_bytes]
    if w.batch == 1:
        rc = X.xpose_2d(d_out.data_ptr(), d_in.data_ptr(), w.rows, w.cols,
                        w.cols, w.rows, code, 0)
    else:
        rc = X.xpose_batched(d_out.data_ptr(), d_in.data_ptr(), w.batch,
                             w.rows, w.cols, w.cols, w.rows, w.rows * w.cols,
                             w.cols * w.rows, code, 0)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    return d_out.cpu().numpy()


def _as_raw(a, s):
    return a.view(wl.RAW_UINT[s])


@pytest.mark.parametrize("key", sorted(wl.WORKLOADS))
def test_workload_full_size_bit_exact(key):
    """Each workload at its full size, every element, against the oracle."""
    w = wl.WORKLOADS[key]
    s = w.elem_bytes
    say(f"workload {key}")
    host = wl.make_input(w)
    got = _run_workload_tensor(w, host)
    want = oracle.transpose(host)
    assert got.shape == want.shape
    assert np.array_equal(_as_raw(got, s), _as_raw(want, s))
    if w.recipe == "index":
        # out[r][c] == float(c * cols + r) exactly
        r = np.arange(w.cols)[:, None]
        c = np.arange(w.rows)[None, :]
        assert np.array_equal(got, (c * w.cols + r).astype(np.float32))


@pytest.mark.parametrize("key", sorted(wl.WORKLOADS))
def test_workload_coordinate_planes(key):
    """Raw-bit coordinate planes at each workload's shape: with in = row
    index the output must hold its column index, and vice versa.  Both
    planes together fix every element's destination."""
    w = wl.WORKLOADS[key]
    s = w.elem_bytes
    shape = w.in_shape
    for axis, want_axis in ((-2, -1), (-1, -2)):
        say(f"workload {key} plane axis={axis}")
        plane = wl.index_plane(shape, axis, s)
        got = _as_raw(_run_workload_tensor(w, plane), s)
        out_shape = got.shape
        want = wl.index_plane(out_shape, want_axis, s)
        assert np.array_equal(got, want)
        del plane, got, want


@pytest.mark.parametrize("s", SIZES)
def test_edge_sweep(s):
    """Every shape in {1,2,3,31,32,33,63,64,65,127,128,129}^2: tiles that are
    full, one short, one over, single rows and columns."""
    for r in EDGE_DIMS:
        for c in EDGE_DIMS:
            check_case(s, 1, r, c, seed=r * 1000 + c, label="edge")


@pytest.mark.parametrize("s", SIZES)
def test_primes_and_multi_tile_ragged(s):
    for r, c in ((257, 509), (1021, 131), (131, 1021), (997, 1009)):
        check_case(s, 1, r, c, seed=r + c, label="prime")


def _tiles_for(s):
    """Every built (tile rows, tile cols, workgroup size) for element size s."""
    out = set()
    for tr, tc in ((32, 32), (32, 64), (64, 32), (64, 64), (64, 128),
                   (128, 64), (128, 128), (32, 128), (128, 32), (256, 128),
                   (256, 256)):
        for nt in (64, 128, 256, 512):
            opts = X.XposeOpts(1, tr, tc, 0)
            opts.threads = nt
            rc, info = X.xpose_plan(0x10000000, 0x20000000, 1, 8, 8, 8, 8, 0,
                                    0, DTYPE_OF_SIZE[s], opts)
            if rc == 0:
                out.add((tr, tc, nt))
    return sorted(out)


@pytest.mark.parametrize("s", SIZES)
@pytest.mark.parametrize("layout", (X.LAYOUT_UNPADDED, X.LAYOUT_PAD1,
                                    X.LAYOUT_SWIZZLE))
def test_every_built_kernel(s, layout):
    """Every compiled (element size, tile, layout) kernel on a ragged
    multi-tile shape, on the vector path and forced element-wise."""
    for tr, tc, nt in _tiles_for(s):
        for flags in (0, X.FLAG_ELEMENTWISE):
            opts = X.XposeOpts(layout, tr, tc, flags)
            opts.threads = nt
            tag = f"{tr}x{tc}/{nt} L{layout} f{flags}"
            check_case(s, 1, 3 * tr + 5, 2 * tc + 3, seed=tr * tc + flags,
                       opts=opts, label=f"kernel {tag}")
            check_case(s, 1, 2 * tr, 3 * tc, seed=tr + tc + flags, opts=opts,
                       label=f"kernel-full {tag}")


@pytest.mark.parametrize("s", SIZES)
def test_pitches_and_padding_untouched(s):
    """ld_in > cols and ld_out > rows: padding of the output keeps its
    sentinel, guard bands before and after the output stay intact."""
    for r, c, ldi, ldo in ((100, 70, 77, 108), (64, 64, 72, 68),
                           (129, 255, 256, 136), (33, 65, 65, 33)):
        check_case(s, 1, r, c, ld_in=ldi, ld_out=ldo, seed=r * c, label="ld")


@pytest.mark.parametrize("s", SIZES)
def test_unaligned_pointers(s):
    """Base pointers shifted by one element: every element size keeps the
    128-bit path (unaligned dwordx4 for 1- and 2-byte types)."""
    for shift_in, shift_out in ((1, 0), (0, 1), (3, 5)):
        check_case(s, 1, 150, 90, seed=shift_in * 7 + shift_out,
                   in_shift=shift_in, out_shift=shift_out, label="shift")


@pytest.mark.parametrize("s", SIZES)
def test_batched_strides(s):
    # minimal strides, gaps between matrices, and a broadcast input
    check_case(s, 5, 70, 45, seed=1, label="batch-min")
    check_case(s, 4, 70, 45, ld_in=50, ld_out=80, stride_in=70 * 50 + 13,
               stride_out=45 * 80 + 29, seed=2, label="batch-gaps")
    check_case(s, 3, 40, 66, stride_in=0, seed=3, label="batch-broadcast")


def test_2d_entry_matches():
    check_case(4, 1, 300, 200, seed=5, entry="2d", label="2d")
    check_case(2, 1, 300, 200, seed=6, entry="2d", label="2d")


@pytest.mark.parametrize("layout", (X.LAYOUT_UNPADDED, X.LAYOUT_PAD1,
                                    X.LAYOUT_SWIZZLE, X.LAYOUT_NAIVE_READ,
                                    X.LAYOUT_NAIVE_WRITE))
def test_2d_ex_entry_per_layout(layout):
    """xpose_2d_ex: every layout of the pages' record (the 32-word row, the
    one-word pad, the swizzle, the naive kernels), on a ragged shape with
    padded pitches and on the pages' 32 x 32 tile, bit-exact."""
    for s, seed in ((4, 21), (2, 22), (1, 23), (8, 24)):
        check_case(s, 1, 300, 200, ld_in=203, ld_out=301, seed=seed + layout,
                   entry="2d_ex", opts=X.make_opts(layout),
                   label=f"2d_ex layout={layout}")
    if layout <= X.LAYOUT_SWIZZLE:
        check_case(4, 1, 256, 192, seed=25, entry="2d_ex",
                   opts=X.make_opts(layout, (32, 32)),
                   label=f"2d_ex 32x32 layout={layout}")


@pytest.mark.parametrize("s", (1, 2, 4, 8))
def test_occupancy_caps(s):
    """Reserved LDS caps the workgroups per compute unit; results are the
    same for every cap, on the ordinary, line-aligned and transpose-read
    tiles, with diagonal and super-tile orders."""
    fam = [(None, 0), (None, X.FLAG_NO_ALIGN_OUT)]
    if s in (2, 4, 8):
        fam.append((None, X.FLAG_ALIGN_OUT))
    if s in (1, 2):
        fam.append((None, X.FLAG_TR_READ))
    for occ in (1, 2, 3, -1):
        for tile, fl in fam:
            for order in (X.ORDER_DIAGONAL, X.ORDER_SUPER_TILES):
                o = X.make_opts(X.LAYOUT_SWIZZLE, tile, fl, X.CACHE_AUTO, 0, 0,
                                0, order, 0, occ)
                check_case(s, 1, 515, 333, ld_out=517, seed=40 + occ,
                           opts=o, label=f"occupancy {occ} flags {fl}")
                check_case(s, 2, 256, 384, seed=50 + occ, opts=o,
                           label=f"occupancy {occ} flags {fl} batch")


@pytest.mark.parametrize("s", (2, 4))
def test_special_float_bits(s):
    """NaN payloads, infinities, -0, subnormals move unchanged."""
    special = wl.special_f16_bits() if s == 2 else wl.special_f32_bits()
    src = np.resize(special, 96 * 80).astype(wl.RAW_UINT[s])
    check_case(s, 1, 96, 80, src=src, label="special")


def test_double_transpose_is_identity():
    for s in SIZES:
        a = wl.random_bits((777, 333), s, seed=s)
        t = _to_dev(a)
        say(f"double transpose s={s}")
        back = X.transpose(X.transpose(t))
        torch.cuda.synchronize()
        assert np.array_equal(back.cpu().numpy().view(a.dtype), a)


def test_repeated_index_check_no_races():
    """The exact index check many times over: a read of the tile before the
    barrier would show up as a misplaced index ("Shared memory and the bank
    conflict", section "The barrier")."""
    w = wl.WORKLOADS["c1_index_1024_f32"]
    a = torch.from_numpy(wl.make_input(w)).to(_dev())
    want = torch.from_numpy(oracle.transpose(wl.make_input(w))).to(_dev())
    out = torch.empty_like(a)
    for layout in (X.LAYOUT_SWIZZLE, X.LAYOUT_PAD1, X.LAYOUT_UNPADDED):
        say(f"repeat index layout={layout}")
        for _ in range(100):
            out.fill_(-1.0)
            X.transpose(a, out, layout=layout)
            assert torch.equal(out.view(torch.int32), want.view(torch.int32))


def test_torch_views_and_streams():
    x = _to_dev(wl.random_bits((300, 500), 4, 11))
    view = x[10:250, 20:470]             # ld_in = 500
    out = torch.empty((600, 400), dtype=x.dtype, device=_dev())
    dst = out[:450, :240]                # ld_out = 400
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        X.transpose(view, dst, stream=s)
    s.synchronize()
    want = oracle.transpose(view.cpu().numpy())
    assert np.array_equal(dst.cpu().numpy(), want)


def test_threads_on_their_own_streams():
    """Calls are reentrant: four host threads, each with its own stream,
    enqueue transposes of every element size and SGEMMs at the same time
    (ctypes releases the interpreter lock during each call).  Every result
    must equal the oracle's."""
    import threading

    import oracle.sgemm as og
    dev = _dev()
    results, errors = {}, []

    def worker(tid):
        try:
            torch.cuda.set_device(dev)
            s = torch.cuda.Stream()
            rng = np.random.default_rng(500 + tid)
            jobs = []
            with torch.cuda.stream(s):
                for it in range(12):
                    size = (1, 2, 4, 8)[(tid + it) % 4]
                    r, c = int(rng.integers(1, 400)), int(rng.integers(1, 400))
                    h = wl.random_bits((r, c), size, 1000 * tid + it)
                    if size > 1:
                        h = h.view(SIGNED[size])
                    y = X.transpose(torch.from_numpy(h).to(dev), stream=s)
                    jobs.append(("t", h, y))
                    if it % 4 == 0:
                        m, n, k = (int(v) for v in rng.integers(1, 300, 3))
                        A = wl.small_int_f32((m, k), 2000 + 10 * tid + it)
                        B = wl.small_int_f32((k, n), 3000 + 10 * tid + it)
                        C = wl.small_int_f32((m, n), 4000 + 10 * tid + it)
                        dC = torch.from_numpy(C.copy()).to(dev)
                        X.sgemm(torch.from_numpy(A).to(dev),
                                torch.from_numpy(B).to(dev), dC,
                                alpha=2.0, beta=-1.0, stream=s)
                        jobs.append(("g", (A, B, C), dC))
            s.synchronize()
            results[tid] = [(kind, src, out.cpu().numpy()) for kind, src, out in jobs]
        except Exception as e:  # reported by the main thread
            errors.append((tid, repr(e)))

    say("4 threads, own streams, transposes and SGEMMs")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for tid, jobs in results.items():
        for kind, src, got in jobs:
            if kind == "t":
                assert np.array_equal(got, oracle.transpose(src)), (tid, src.shape)
            else:
                A, B, C = src
                m, k = A.shape
                n = B.shape[1]
                want = og.sgemm(m, n, k, 2.0, A.reshape(-1), k, B.reshape(-1), n,
                                -1.0, C.reshape(-1), n)
                assert np.array_equal(got, want.astype(np.float32)), (tid, m, n, k)
    assert len(results) == 4


def test_hip_graph_capture_and_replay():
    """Calls only enqueue kernels (no allocation, memset or synchronisation),
    so they can be captured into a HIP graph.  Every replay, with eager work
    on the same buffers in between, must match the oracle."""
    cases = [(wl.random_bits((777, 1031), 2, 21), None),              # fp16 packed
             (wl.random_bits((3, 300, 517), 4, 22), None),            # line-aligned out
             (wl.random_bits((512, 640), 1, 23), X.FLAG_TR_READ),     # transpose reads
             (wl.random_bits((256, 384), 8, 24), None)]               # f64
    devs, outs, wants = [], [], []
    for host, _ in cases:
        x = _to_dev(host)
        devs.append(x)
        shape = host.shape[:-2] + (host.shape[-1], host.shape[-2])
        outs.append(torch.empty(shape, dtype=x.dtype, device=_dev()))
        wants.append(oracle.transpose(host))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # eager warm-up on the capture stream
        for (host, fl), x, y in zip(cases, devs, outs):
            X.transpose(x, y, flags=fl or 0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (host, fl), x, y in zip(cases, devs, outs):
            X.transpose(x, y, flags=fl or 0)
    for rep in range(3):
        for y in outs:
            y.fill_(rep + 1)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, want) in enumerate(zip(outs, wants)):
            got = y.cpu().numpy().view(want.dtype)
            assert np.array_equal(got, want), f"replay {rep}, case {i}"


def test_copy_kernel():
    for nbytes, src_off, dst_off in ((1 << 20, 0, 0), (12345, 0, 0),
                                     (100003, 3, 1), (16, 0, 0), (1, 0, 0)):
        say(f"copy {nbytes} {src_off} {dst_off}")
        host = wl.random_bits((nbytes + 64,), 1, nbytes)
        src = torch.from_numpy(host).to(_dev())
        dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=_dev())
        rc = X.xpose_copy(dst.data_ptr() + dst_off, src.data_ptr() + src_off,
                          nbytes, 0)
        assert rc == 0
        torch.cuda.synchronize()
        got = dst.cpu().numpy()
        assert np.array_equal(got[dst_off:dst_off + nbytes],
                              host[src_off:src_off + nbytes])
        assert not got[:dst_off].any() and not got[dst_off + nbytes:].any()


@pytest.mark.parametrize("s", SIZES)
def test_tile_orders_and_cache_policies(s):
    """Tile enumeration order, XCD remap and non-temporal accesses change
    only the schedule: results stay bit-exact, batches included."""
    for cache in (X.CACHE_DEFAULT, X.CACHE_NT_STORE):
        for gr, gc in ((1, 0), (3, 0), (1000, 0), (2, 3), (4, 1), (5, 1000)):
            for flags in (X.FLAG_XCD_REMAP, X.FLAG_NO_XCD_REMAP):
                opts = X.make_opts(X.LAYOUT_SWIZZLE, None, flags, cache, gr, gc)
                tag = f"c{cache} g{gr}x{gc} f{flags}"
                check_case(s, 1, 777, 555, seed=cache * 100 + gr + gc + flags,
                           opts=opts, label=f"order {tag}")
                check_case(s, 3, 301, 257, seed=gr + gc + flags, opts=opts,
                           label=f"order-batch {tag}")
        for flags in (X.FLAG_XCD_REMAP, X.FLAG_NO_XCD_REMAP):
            opts = X.make_opts(X.LAYOUT_SWIZZLE, None, flags, cache,
                               order=X.ORDER_DIAGONAL)
            check_case(s, 1, 777, 555, seed=cache + flags, opts=opts,
                       label=f"diagonal c{cache} f{flags}")
            check_case(s, 3, 301, 257, seed=cache + flags + 1, opts=opts,
                       label=f"diagonal-batch c{cache} f{flags}")


@pytest.mark.parametrize("s", SIZES)
def test_naive_kernels(s):
    """The two no-LDS ablation kernels give the same bits as the oracle."""
    for layout in (X.LAYOUT_NAIVE_READ, X.LAYOUT_NAIVE_WRITE):
        opts = X.XposeOpts(layout, 0, 0, 0)
        for r, c in ((1, 1), (33, 257), (300, 70), (1, 600), (600, 1)):
            check_case(s, 1, r, c, seed=r + c + layout, opts=opts,
                       label=f"naive{layout}")
        check_case(s, 3, 70, 45, ld_in=50, ld_out=80, stride_in=70 * 50 + 7,
                   stride_out=45 * 80 + 3, seed=layout, opts=opts,
                   label=f"naive{layout}-batch")


@pytest.mark.parametrize("s", SIZES)
def test_persistent_kernels(s):
    """Persistent double-buffered workgroups: each walks many tiles, interior
    and edge, cycling both LDS buffers; every tile order, both cache
    policies, batches."""
    tiles = {4: ((32, 32), (128, 64)), 2: ((128, 64), (64, 64)),
             1: ((128, 128),), 8: ((32, 32),)}[s]
    for tile in tiles:
        for per_cu in (1, 3):
            for cache in (X.CACHE_DEFAULT, X.CACHE_NT_STORE):
                for order, flags in ((X.ORDER_SUPER_TILES, X.FLAG_XCD_REMAP),
                                     (X.ORDER_DIAGONAL, X.FLAG_NO_XCD_REMAP)):
                    opts = X.make_opts(X.LAYOUT_SWIZZLE, tile, flags, cache,
                                       order=order, persistent=per_cu)
                    tag = f"persistent {tile} x{per_cu} c{cache} o{order}"
                    check_case(s, 1, 2000, 1777, seed=per_cu + cache + order,
                               opts=opts, label=tag)
                    check_case(s, 3, 301, 513, seed=7 + per_cu, opts=opts,
                               label=tag + " batch")


def test_persistent_repeated_index_check():
    w = wl.WORKLOADS["c1_index_1024_f32"]
    a = torch.from_numpy(wl.make_input(w)).to(_dev())
    want = torch.from_numpy(oracle.transpose(wl.make_input(w))).to(_dev())
    out = torch.empty_like(a)
    say("persistent repeat index")
    for per_cu in (1, 2):
        for _ in range(50):
            out.fill_(-1.0)
            X.transpose(a, out, tile=(32, 32), persistent=per_cu)
            assert torch.equal(out.view(torch.int32), want.view(torch.int32))


@pytest.mark.parametrize("s", (4, 8))
def test_direct_lds_kernels(s):
    """Interior tiles loaded straight into LDS with the swizzle applied on the
    global side: bit-exact for every built shape, layout and cache policy."""
    built = []
    for tile in ((32, 32), (64, 64), (128, 64)):
        for layout in (X.LAYOUT_SWIZZLE, X.LAYOUT_UNPADDED):
            for cache in (X.CACHE_DEFAULT, X.CACHE_NT_STORE):
                opts = X.make_opts(layout, tile, X.FLAG_DIRECT_LDS, cache)
                rc, info = X.xpose_plan(0x10000000, 0x20000000, 1, 8, 8, 8, 8,
                                        0, 0, DTYPE_OF_SIZE[s], opts)
                if rc == 0:
                    assert info.direct_lds == 1
                    built.append((tile, layout, cache, opts))
    assert built
    for tile, layout, cache, opts in built:
        tag = f"direct {tile} L{layout} c{cache}"
        check_case(s, 1, 5 * tile[0] + 3, 3 * tile[1] + 7, seed=layout + cache,
                   opts=opts, label=tag)
        check_case(s, 1, 4 * tile[0], 4 * tile[1], seed=11, opts=opts, label=tag)
        check_case(s, 3, 2 * tile[0] + 1, 2 * tile[1], seed=12, opts=opts,
                   label=tag + " batch")


SHIFT_TILES = {4: ((64, 64), (128, 64), (256, 64), (128, 32), (64, 32),
                   (64, 128), (128, 128), (256, 128)),
               2: ((64, 64), (128, 64), (256, 64)),
               8: ((32, 32), (64, 32), (64, 64))}


def test_aligned_out_defaults_by_call_size():
    """The default line-aligned tile changes with the call size: fp16 from
    128 MiB on takes 128 x 64 tiles in column bands, below it 64 x 64
    super-tiles; fp32 from 512 MiB on 64 x 128 tiles, below it 64 x 64;
    fp64 keeps one tile.  Each default at an odd pitch, every element against
    the oracle."""
    for s, r, c, want in ((2, 5793, 5793, (128, 64)), (2, 5791, 5791, (64, 64)),
                          (2, 12345, 3001, (128, 64)), (4, 4001, 3333, (64, 64)),
                          (4, 8193, 8193, (64, 128)), (4, 8193, 8191, (64, 64)),
                          (8, 3001, 2999, (32, 32))):
        rc, info = X.xpose_plan(0x100000000000, 0x200000000000, 1, r, c, c,
                                r, 0, 0, DTYPE_OF_SIZE[s], None)
        assert rc == 0 and info.aligned_out == 1
        assert (info.tile_rows, info.tile_cols) == want, (s, r, c)
        check_case(s, 1, r, c, seed=r + c + s, label=f"align-out default s{s}")


@pytest.mark.parametrize("s", sorted(SHIFT_TILES))
def test_aligned_out_kernels(s):
    """Line-aligned output tiles: every built shape and cache policy, output
    pitches and pointers at many element offsets within a line (odd ones for
    2-byte elements, where segments start mid-unit), edge tiles in both
    dimensions, batches with odd strides."""
    built = []
    for tile in SHIFT_TILES[s]:
        for cache in (X.CACHE_DEFAULT, X.CACHE_NT_STORE):
            opts = X.make_opts(X.LAYOUT_SWIZZLE, tile, X.FLAG_ALIGN_OUT, cache)
            rc, info = X.xpose_plan(0x10000000, 0x20000000, 1, 8, 8, 8, 8, 0,
                                    0, DTYPE_OF_SIZE[s], opts)
            if rc == 0:
                assert info.aligned_out == 1
                built.append((tile, cache, opts))
    assert len(built) >= len(SHIFT_TILES[s])
    line = 128 // s
    for tile, cache, opts in built:
        tag = f"align-out s{s} {tile} c{cache}"
        for r, c, pad, shift in ((777, 555, 3, 0), (2 * tile[0] + line - 1, 130, 0, 5),
                                 (1000, 3 * tile[1], 13, line - 1), (33, 7, 1, 2),
                                 (tile[0], tile[1], line, 0), (301, 99, 1, 1)):
            check_case(s, 1, r, c, ld_out=r + pad, out_shift=shift,
                       seed=r + c + cache, opts=opts, label=tag)
        check_case(s, 3, 301, 257, ld_out=305, stride_out=257 * 305 + 9,
                   seed=3, opts=opts, label=tag + " batch")
        # input rows off alignment as well
        check_case(s, 1, 2 * tile[0] + 3, tile[1] + 5, ld_in=tile[1] + 6,
                   ld_out=2 * tile[0] + 7, in_shift=1, out_shift=3, seed=4,
                   opts=opts, label=tag + " in-shift")


STRIP_TILES = {4: ((64, 64), (128, 64), (128, 32)), 8: ((32, 32), (64, 32))}


@pytest.mark.parametrize("s", sorted(STRIP_TILES))
def test_aligned_out_column_strips(s):
    """Line-aligned output tiles in column strips (persistent = tile rows
    per workgroup, the halo kept in an LDS ring): segments of 1, 2, 3 and 8
    tile rows and one segment per strip, ragged in both dimensions, output
    rows at many offsets within a line, input rows off alignment, batches
    with odd strides, with and without the per-XCD remap."""
    line = 128 // s
    for tile in STRIP_TILES[s]:
        for seg in (1, 2, 3, 8, 64):
            for flags in (X.FLAG_XCD_REMAP, X.FLAG_NO_XCD_REMAP):
                opts = X.make_opts(X.LAYOUT_SWIZZLE, tile,
                                   X.FLAG_ALIGN_OUT | flags,
                                   X.CACHE_NT_STORE, persistent=seg)
                rc, info = X.xpose_plan(0x10000000, 0x20000000, 1, 8, 8, 8,
                                        8, 0, 0, DTYPE_OF_SIZE[s], opts)
                assert rc == 0 and info.aligned_out == 1
                assert info.persistent == seg
                tag = f"strip s{s} {tile} seg{seg} f{flags}"
                for r, c, pad, shift in ((777, 555, 3, 0),
                                         (5 * tile[0] + line - 1, 130, 0, 5),
                                         (1000, 3 * tile[1], 13, line - 1),
                                         (33, 7, 1, 2), (tile[0], tile[1], line, 0)):
                    check_case(s, 1, r, c, ld_out=r + pad, out_shift=shift,
                               seed=r + c + seg, opts=opts, label=tag)
                check_case(s, 3, 301, 257, ld_out=305,
                           stride_out=257 * 305 + 9, seed=3, opts=opts,
                           label=tag + " batch")
                check_case(s, 1, 4 * tile[0] + 3, tile[1] + 5,
                           ld_in=tile[1] + 6, ld_out=4 * tile[0] + 7,
                           in_shift=1, out_shift=3, seed=4, opts=opts,
                           label=tag + " in-shift")


TR_TILES = {2: ((64, 64), (128, 64), (64, 128), (128, 128), (64, 32)),
            1: ((128, 128), (64, 128), (128, 64), (128, 256))}


def test_tr_read_kernels():
    """LDS transpose-read tiles (1- and 2-byte elements): every built shape,
    both cache policies and direct loads, interior and edge tiles, pitches,
    pointers off 16-byte alignment, elementwise (unaligned rows) and
    batches."""
    built = 0
    for s, tiles in TR_TILES.items():
        for tile in tiles:
            for flags in (X.FLAG_TR_READ, X.FLAG_TR_READ | X.FLAG_DIRECT_LDS):
                for cache in (X.CACHE_DEFAULT, X.CACHE_NT_STORE):
                    opts = X.make_opts(X.LAYOUT_SWIZZLE, tile, flags, cache)
                    rc, info = X.xpose_plan(0x10000000, 0x20000000, 1, 512, 512,
                                            512, 512, 0, 0, DTYPE_OF_SIZE[s], opts)
                    if rc != 0:
                        continue
                    assert info.tr_read == 1
                    built += 1
                    tag = f"tr s{s} {tile} f{flags} c{cache}"
                    tr, tc = tile
                    for r, c, pi, po in ((2 * tr, 3 * tc, 0, 0), (777, 555, 0, 0),
                                         (tr + 1, tc - 1, 4, 8), (33, 17, 0, 0),
                                         (3 * tr + 5, 2 * tc + 7, 16, 2)):
                        check_case(s, 1, r, c, ld_in=c + pi, ld_out=r + po,
                                   seed=r * 7 + c + cache, opts=opts, label=tag)
                    # rows 4-byte aligned but not 16: still the vector path
                    check_case(s, 1, 2 * tr, 2 * tc, ld_in=2 * tc + 4 // s * 3,
                               ld_out=2 * tr + 4 // s, in_shift=4 // s,
                               out_shift=4 // s, seed=5, opts=opts, label=tag + " off16")
                    # odd pitches (rows not 4-byte aligned): unaligned vectors
                    check_case(s, 1, 2 * tr + 3, tc + 9, ld_in=tc + 9 + 1,
                               ld_out=2 * tr + 3 + 1, in_shift=1, seed=6,
                               opts=opts, label=tag + " odd")
                    check_case(s, 3, tr + 17, tc + 33, ld_in=tc + 40,
                               ld_out=tr + 20, stride_in=(tr + 17) * (tc + 40) + 8,
                               stride_out=(tc + 33) * (tr + 20) + 16, seed=7,
                               opts=opts, label=tag + " batch")
    assert built >= 20


def test_tr_read_forced_elementwise():
    for s, tile in ((2, (128, 64)), (1, (128, 128))):
        opts = X.make_opts(X.LAYOUT_SWIZZLE, tile, X.FLAG_TR_READ | X.FLAG_ELEMENTWISE)
        check_case(s, 2, 300, 259, seed=11, opts=opts, label=f"tr elementwise s{s}")


PACKED_SHAPES = ((1, 1), (1, 7), (7, 1), (3, 5), (8, 8), (16, 16), (7, 100),
                 (100, 7), (32, 32), (17, 33), (64, 16), (16, 64), (128, 32),
                 (64, 64), (48, 48), (45, 91))


@pytest.mark.parametrize("s", SIZES)
def test_packed_small_matrices(s):
    """Packed batches of dense small matrices: batches that end with a
    partial workgroup, shifted pointers (write-back blocks), rows of 64 bytes
    or more (padded LDS rows), the forced kernel, and a single matrix."""
    for r, c in PACKED_SHAPES:
        if r * c * s > 16384:
            continue
        for batch, shift in ((1000, 0), (37, 1), (2, 0), (513, 3)):
            rc, info = X.xpose_plan(1 << 40, 1 << 44, batch, r, c, c, r, r * c,
                                    r * c, DTYPE_OF_SIZE[s], None)
            assert rc == 0 and info.packed >= 1, (r, c, batch)
            check_case(s, batch, r, c, seed=r * 131 + c + batch,
                       in_shift=shift, out_shift=shift,
                       label=f"packed s{s} {batch}x{r}x{c}")
    want = X.make_opts(flags=X.FLAG_PACKED)
    for r, c in ((64, 64), (45, 91), (1, 2048 // s), (2048 // s, 2)):
        if r * c * s <= 16384:
            check_case(s, 19, r, c, seed=7, opts=want, label=f"packed forced s{s} {r}x{c}")
    check_case(s, 1, 13, 29, seed=8, opts=want, label=f"packed single s{s}")
    check_case(s, 300, 8, 8, seed=9, opts=X.make_opts(flags=X.FLAG_PACKED, cache=X.CACHE_DEFAULT),
               label=f"packed write-back s{s}")


# Dense matrices of 16-32 KiB that are not a whole number of tiles: packed
# by default into 32 KiB blocks.
RAGGED_32K = {4: ((64, 96), (90, 90), (70, 117)), 2: ((100, 100), (127, 127), (90, 150)),
              1: ((150, 150), (181, 181), (100, 300)), 8: ((45, 60), (63, 63))}


@pytest.mark.parametrize("s", SIZES)
def test_packed_ragged_up_to_32k(s):
    for r, c in RAGGED_32K[s]:
        assert 16384 < r * c * s <= 32768
        for batch, shift in ((300, 0), (29, 1)):
            rc, info = X.xpose_plan(1 << 40, 1 << 44, batch, r, c, c, r, r * c,
                                    r * c, DTYPE_OF_SIZE[s], None)
            assert rc == 0 and info.packed >= 1, (r, c, batch)
            check_case(s, batch, r, c, seed=r * 7 + c + batch, in_shift=shift,
                       out_shift=shift, label=f"packed 32k s{s} {batch}x{r}x{c}")
    # forced: a whole-tile matrix of 32 KiB, a single matrix
    r, c = (128, 64) if s == 4 else (128, 128) if s == 2 else (128, 256) if s == 1 else (64, 64)
    want = X.make_opts(flags=X.FLAG_PACKED)
    check_case(s, 9, r, c, seed=3, opts=want, label=f"packed forced 32k s{s} {r}x{c}")
    check_case(s, 1, r, c, seed=4, opts=want, label=f"packed forced single 32k s{s}")


def test_nontemporal_loads_variant():
    """Non-temporal loads and stores are built for two fp32 tiles only."""
    for tile in ((32, 32), (64, 64)):
        opts = X.make_opts(X.LAYOUT_SWIZZLE, tile, 0, X.CACHE_NT_ALL)
        check_case(4, 1, 777, 555, seed=9, opts=opts, label=f"nt-all {tile}")
        check_case(4, 2, 256, 512, seed=10, opts=opts, label=f"nt-all {tile}")


def test_copy_variants():
    nbytes = (3 << 20) + 44
    host = wl.random_bits((nbytes,), 1, 123)
    src = torch.from_numpy(host).to(_dev())
    n_ok = 0
    for thr in (256, 512, 1024):
        for unroll in (4, 8, 16):
            for cache in (X.CACHE_DEFAULT, X.CACHE_NT_STORE, X.CACHE_NT_ALL):
                opts = X.XposeCopyOpts(thr, unroll, cache, 0)
                dst = torch.zeros(nbytes, dtype=torch.uint8, device=_dev())
                rc = X.xpose_copy_ex(dst.data_ptr(), src.data_ptr(), nbytes, opts, 0)
                if rc == X.XPOSE_ENOTILE:
                    continue
                say(f"copy variant {thr} {unroll} {cache}")
                assert rc == 0
                torch.cuda.synchronize()
                assert np.array_equal(dst.cpu().numpy(), host)
                n_ok += 1
    assert n_ok >= 5
