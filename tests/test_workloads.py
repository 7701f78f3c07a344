"""Seeded input generators (CPU only): deterministic, right shape, right
value ranges."""
import numpy as np

import workloads as wl


def test_workload_table():
    assert set(wl.WORKLOADS) == {
        "c1_index_1024_f32", "c2_8192_f32", "c3_ragged_12345x6789_f32",
        "c4_16384_f16", "c5_batched_64x2048x1024_f32",
        "shard_1024x8192_f32", "shard_batched_8x2048x1024_f32"}
    assert wl.WORKLOADS["shard_1024x8192_f32"].rw_bytes * 8 == 536_870_912
    assert wl.WORKLOADS["shard_batched_8x2048x1024_f32"].rw_bytes * 8 == 1_073_741_824
    c2 = wl.WORKLOADS[wl.HEADLINE]
    assert (c2.rows, c2.cols, c2.dtype) == (8192, 8192, "f32")
    assert c2.rw_bytes == 536_870_912
    assert wl.WORKLOADS["c3_ragged_12345x6789_f32"].rw_bytes == 670_481_640
    assert wl.WORKLOADS["c4_16384_f16"].rw_bytes == 1_073_741_824
    assert wl.WORKLOADS["c5_batched_64x2048x1024_f32"].rw_bytes == 1_073_741_824
    assert wl.WORKLOADS["c1_index_1024_f32"].rw_bytes == 8_388_608


def test_index_workload_exact():
    a = wl.make_input(wl.WORKLOADS["c1_index_1024_f32"])
    assert a.dtype == np.float32 and a.shape == (1024, 1024)
    assert a[3, 5] == np.float32(3 * 1024 + 5) and a[-1, -1] == 1024 * 1024 - 1


def test_uniform_range_and_determinism():
    small = wl.Workload("t", 1, 300, 200, "f32", "uniform", 2, "")
    a, b = wl.make_input(small), wl.make_input(small)
    assert np.array_equal(a, b)
    assert a.min() >= -1.0 and a.max() < 1.0
    other = wl.Workload("t", 1, 300, 200, "f32", "uniform", 3, "")
    assert not np.array_equal(a, wl.make_input(other))


def test_f16_raw_bits():
    w = wl.Workload("t", 1, 64, 64, "f16", "normal_f16", 4, "")
    a = wl.make_input(w)
    assert a.dtype == np.uint16
    v = a.view(np.float16).astype(np.float32)
    assert np.all(np.isfinite(v)) and 0.5 < v.std() < 1.5


def test_planes():
    p = wl.index_plane((3, 5), 0, 4)
    assert p.tolist() == [[0] * 5, [1] * 5, [2] * 5]
    q = wl.index_plane((3, 5), 1, 2)
    assert q.dtype == np.uint16 and q[2].tolist() == [0, 1, 2, 3, 4]
    wrap = wl.index_plane((1, 300), 1, 1)
    assert wrap[0, 257] == 1
    lin = wl.linear_index_plane((2, 3, 4), 8)
    assert lin.dtype == np.uint64 and lin[1, 2, 3] == 23
    assert wl.random_bits((4, 4), 8, 1).dtype == np.uint64
