"""The no-allocation SGEMM entry point (xpose_sgemm_noalloc,
include/xpose_sgemm.h) through the C ABI, against the workspace entry point
whose kernels it shares (xpose_sgemm_ws) and against the oracle: two calls
in a row on the library's one scratch array, the second with a smaller
input, each bit-identical to xpose_sgemm_ws given a workspace of the
scratch's size (the same split, so the same kernels and summation order)
and exact against the oracle on integer inputs."""
import numpy as np
import pytest

import oracle.sgemm as og
import workloads as wl
from xpose_testlib import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
X = pytest.importorskip("lds_tiled_matrix_amd")


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _one_call(m, n, k, alpha, beta, opts, seed, want_splits):
    dev = _dev()
    A = wl.small_int_f32((m, k), seed)
    B = wl.small_int_f32((k, n), seed + 1)
    C = wl.small_int_f32((m, n), seed + 2)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC_ws, dC_na = torch.from_numpy(C).to(dev), torch.from_numpy(C).to(dev)
    args = (m, n, k, dA.data_ptr(), k, dB.data_ptr(), n)
    rc, info = X.xpose_sgemm_plan_ws(*args, dC_na.data_ptr(), n, opts,
                                     1 << 44, X.SGEMM_SCRATCH_BYTES)
    assert rc == 0, X.strerror(rc)
    assert info.splits == want_splits, (info.splits, want_splits)
    ws = torch.empty(X.SGEMM_SCRATCH_BYTES // 4, dtype=torch.float32,
                     device=dev)
    say(f"noalloc m={m} n={n} k={k} splits={info.splits} (workspace entry)")
    rc = X.xpose_sgemm_ws(m, n, k, alpha, dA.data_ptr(), k, dB.data_ptr(), n,
                          beta, dC_ws.data_ptr(), n, opts, ws.data_ptr(),
                          X.SGEMM_SCRATCH_BYTES, 0)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    say(f"noalloc m={m} n={n} k={k} (no-allocation entry)")
    rc = X.xpose_sgemm_noalloc(m, n, k, alpha, dA.data_ptr(), k,
                               dB.data_ptr(), n, beta, dC_na.data_ptr(), n,
                               opts, 0)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    got_ws, got_na = dC_ws.cpu().numpy(), dC_na.cpu().numpy()
    assert np.array_equal(got_na.view(np.uint32), got_ws.view(np.uint32))
    want = og.sgemm(m, n, k, alpha, A.reshape(-1), k, B.reshape(-1), n, beta,
                    C.reshape(-1), n).astype(np.float32).reshape(m, n)
    assert np.array_equal(got_na, want)


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: the library's split (1024^3: 4 slices, 16 MiB of the
    # scratch); second, smaller: an explicit split of 3, whose partials
    # overwrite only the start of what the first call left there
    _one_call(1024, 1024, 1024, 1.0, 1.0, None, 500, 4)
    _one_call(300, 257, 700, 2.0, -1.0, X.make_sgemm_opts(split_k=3), 510, 3)


def test_noalloc_limits():
    """The library's choice shrinks to the scratch (2048^2: 16 MiB planes,
    so 4 fit); an explicit split past 64 MiB is refused before anything
    runs; a call that does not split leaves the scratch alone."""
    rc, info = X.xpose_sgemm_plan_ws(2048, 2048, 2048, 1 << 40, 2048, 1 << 41,
                                     2048, 1 << 42, 2048, None, 1 << 44,
                                     X.SGEMM_SCRATCH_BYTES)
    assert rc == 0 and info.splits == 4
    rc = X.xpose_sgemm_noalloc(2048, 2048, 2048, 1.0, 1 << 40, 2048, 1 << 41,
                               2048, 0.0, 1 << 42, 2048,
                               X.make_sgemm_opts(split_k=5))
    assert rc == X.XPOSE_EWORKSPACE
    assert "scratch" in X.strerror(rc)
    _one_call(256, 256, 32, 1.0, 0.5, None, 520, 1)


def test_noalloc_under_graph_capture():
    """The callers it is for: captured into a HIP graph (after one eager
    call, which looks the scratch address up), two split calls in a row
    share the scratch; C is reset eagerly between replays and every replay
    must match the oracle exactly."""
    dev = _dev()
    cases = [((1024, 1024, 1024), 1.0, 1.0, None),
             ((256, 130, 1000), 2.0, 0.0, X.make_sgemm_opts(split_k=4))]
    bufs = []
    for idx, ((m, n, k), alpha, beta, opts) in enumerate(cases):
        A = wl.small_int_f32((m, k), 530 + 3 * idx)
        B = wl.small_int_f32((k, n), 531 + 3 * idx)
        C = wl.small_int_f32((m, n), 532 + 3 * idx)
        want = og.sgemm(m, n, k, alpha, A.reshape(-1), k, B.reshape(-1), n,
                        beta, C.reshape(-1), n).astype(np.float32)
        bufs.append((torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                     torch.from_numpy(C).to(dev), torch.from_numpy(C).to(dev),
                     alpha, beta, opts, want.reshape(m, n)))

    def enqueue():
        sh = int(torch.cuda.current_stream().cuda_stream)
        for dA, dB, dC, _, alpha, beta, opts, _ in bufs:
            m, k = dA.shape
            n = dB.shape[1]
            rc = X.xpose_sgemm_noalloc(m, n, k, alpha, dA.data_ptr(), k,
                                       dB.data_ptr(), n, beta, dC.data_ptr(),
                                       n, opts, sh)
            assert rc == 0, X.strerror(rc)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        say("noalloc graph warm-up")
        enqueue()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue()
    for rep in range(3):
        for _, _, dC, dC0, *_ in bufs:
            dC.copy_(dC0)
        torch.cuda.synchronize()
        say(f"noalloc graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for i, (_, _, dC, _, _, _, _, want) in enumerate(bufs):
            assert np.array_equal(dC.cpu().numpy(), want), (rep, i)
