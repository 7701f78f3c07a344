"""Seeded synthetic inputs for the out-of-place transpose, shared by the oracle
side and the HIP side.

This module only *makes input bytes*. It performs no transpose, holds no
index permutation and no bank arithmetic, so neither side of a parity
comparison can borrow the other's logic through it.

The pages' only workload is a square fp32 matrix whose side is a multiple of
the tile ("Shared memory and the bank conflict", section "Turn the tile around
on chip"), and their correctness check fills every element with its own index
(same page, section "The barrier"). The five workloads below widen that to
the shapes a transpose library must handle: a cache-resident index-valued
square, a large square, a ragged non-square, a 2-byte element type and a
batch of independent matrices. Values never affect timing, because the path
moves raw bits; they matter only for parity.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Element types the library moves, by their size in bytes.  Names follow the
# C ABI's dtype enumeration; "u8" is any one-byte type.
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "u8": 1, "f64": 8}
# numpy unsigned type with the same width, used to hold and compare raw bits.
RAW_UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


@dataclass(frozen=True)
class Workload:
    """One transpose job: ``batch`` matrices of ``rows x cols`` elements."""

    key: str
    batch: int
    rows: int
    cols: int
    dtype: str
    recipe: str
    seed: int | None
    description: str

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def rw_bytes(self) -> int:
        """Algorithmic traffic: every element is read once and written once."""
        return 2 * self.batch * self.rows * self.cols * self.elem_bytes

    @property
    def in_shape(self) -> tuple:
        if self.batch == 1:
            return (self.rows, self.cols)
        return (self.batch, self.rows, self.cols)


WORKLOADS = {
    "c1_index_1024_f32": Workload(
        "c1_index_1024_f32", 1, 1024, 1024, "f32", "index", None,
        "2-D transpose 1024x1024 fp32, element (i,j) = float(i*1024+j)"),
    "c2_8192_f32": Workload(
        "c2_8192_f32", 1, 8192, 8192, "f32", "uniform", 2,
        "2-D transpose 8192x8192 fp32, uniform [-1,1), ld = cols"),
    "c3_ragged_12345x6789_f32": Workload(
        "c3_ragged_12345x6789_f32", 1, 12345, 6789, "f32", "uniform", 3,
        "2-D transpose 12345x6789 fp32 (ragged edge tiles), uniform [-1,1)"),
    "c4_16384_f16": Workload(
        "c4_16384_f16", 1, 16384, 16384, "f16", "normal_f16", 4,
        "2-D transpose 16384x16384 fp16, normal(0,1) as raw bits"),
    "c5_batched_64x2048x1024_f32": Workload(
        "c5_batched_64x2048x1024_f32", 64, 2048, 1024, "f32", "uniform", 5,
        "batched transpose, 64 matrices of 2048x1024 fp32, uniform [-1,1)"),
    # One GPU's share of the two workloads above when they are spread over 8
    # GPUs (rows of the input and of the output in contiguous blocks, or the
    # batch split 8 ways): the local kernel each GPU would run, measured at
    # its real shape.
    "shard_1024x8192_f32": Workload(
        "shard_1024x8192_f32", 1, 1024, 8192, "f32", "uniform", 6,
        "2-D transpose 1024x8192 fp32 (one GPU's row block of 8192x8192 "
        "on 8 GPUs), uniform [-1,1)"),
    "shard_batched_8x2048x1024_f32": Workload(
        "shard_batched_8x2048x1024_f32", 8, 2048, 1024, "f32", "uniform", 7,
        "batched transpose, 8 matrices of 2048x1024 fp32 (one GPU's share "
        "of the 64-matrix batch on 8 GPUs), uniform [-1,1)"),
}

# The workload the headline throughput is quoted on.
HEADLINE = "c2_8192_f32"


def make_input(w: Workload) -> np.ndarray:
    """Return the workload's input as a C-contiguous array of ``w.in_shape``.

    fp32 workloads come back as float32, fp16 as the raw uint16 bit patterns
    of a float16 array (compared as bits, never as values).
    """
    if w.recipe == "index":
        n = w.batch * w.rows * w.cols
        # Every value is below 2**24, so each index is exact in float32.
        assert n <= 1 << 24
        return np.arange(n, dtype=np.float32).reshape(w.in_shape)
    rng = np.random.default_rng(w.seed)
    if w.recipe == "uniform":
        u = rng.random(w.in_shape, dtype=np.float32)
        # 2u is exact in float32; 2u - 1 stays inside [-1, 1).
        return u * np.float32(2) - np.float32(1)
    if w.recipe == "normal_f16":
        x = rng.standard_normal(w.in_shape, dtype=np.float32)
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown recipe {w.recipe!r}")


@dataclass(frozen=True)
class GemmWorkload:
    """One SGEMM job, C = alpha * A @ B + beta * C with A m x k, B k x n."""

    key: str
    m: int
    n: int
    k: int
    alpha: float
    beta: float
    seed: int
    description: str

    @property
    def flops(self) -> int:
        """Algorithmic work: one multiply and one add per term of each sum."""
        return 2 * self.m * self.n * self.k


# The SGEMM of "Padded Shared Memory: Eliminating Bank Conflicts" is measured
# at M = N = K = 4096 (section "Mechanics"); the pages give no values, alpha
# or beta, so the inputs are uniform [-1, 1) and C += A @ B.
GEMM_WORKLOADS = {
    "sgemm_4096": GemmWorkload(
        "sgemm_4096", 4096, 4096, 4096, 1.0, 1.0, 11,
        "SGEMM 4096x4096x4096 fp32, C += A @ B, uniform [-1,1)"),
}


def uniform_f32(shape: tuple, seed: int) -> np.ndarray:
    """float32 values uniform on [-1, 1), from a seeded generator."""
    rng = np.random.default_rng(seed)
    u = rng.random(shape, dtype=np.float32)
    return u * np.float32(2) - np.float32(1)


def small_int_f32(shape: tuple, seed: int, bound: int = 4) -> np.ndarray:
    """float32 holding integers in [-bound, bound], from a seeded generator:
    products and sums of such values stay exact in float32 while they stay
    below 2**24 in magnitude."""
    rng = np.random.default_rng(seed)
    return rng.integers(-bound, bound + 1, size=shape).astype(np.float32)


def make_gemm_inputs(w: GemmWorkload) -> tuple:
    """(A, B, C) of a GEMM workload as C-contiguous float32 arrays."""
    return (uniform_f32((w.m, w.k), w.seed), uniform_f32((w.k, w.n), w.seed + 1),
            uniform_f32((w.m, w.n), w.seed + 2))


def index_plane(shape: tuple, axis: int, elem_bytes: int) -> np.ndarray:
    """Raw-bit plane whose every element holds its own coordinate on ``axis``.

    ``shape`` is (rows, cols) or (batch, rows, cols).  The value is stored in
    an unsigned integer of ``elem_bytes`` bytes, so for 1- and 2-byte types it
    wraps modulo 2**(8*elem_bytes); callers keep extents small enough when
    they need the plane to be unique.
    """
    t = RAW_UINT[elem_bytes]
    axis = axis % len(shape)
    coord = np.arange(shape[axis], dtype=np.uint64)
    if elem_bytes < 8:
        coord &= np.uint64((1 << (8 * elem_bytes)) - 1)
    view = [1] * len(shape)
    view[axis] = shape[axis]
    return np.ascontiguousarray(
        np.broadcast_to(coord.astype(t).reshape(view), shape))


def linear_index_plane(shape: tuple, elem_bytes: int) -> np.ndarray:
    """Raw-bit plane holding each element's flat (row-major) index, wrapped to
    the element width."""
    t = RAW_UINT[elem_bytes]
    n = int(np.prod(shape))
    idx = np.arange(n, dtype=np.uint64)
    if elem_bytes < 8:
        idx &= np.uint64((1 << (8 * elem_bytes)) - 1)
    return idx.astype(t).reshape(shape)


def random_bits(shape: tuple, elem_bytes: int, seed: int) -> np.ndarray:
    """Uniformly random raw bit patterns.  For float types these include NaN
    payloads, infinities, -0 and subnormals, which catch any path that
    converts values instead of moving bits."""
    rng = np.random.default_rng(seed)
    t = RAW_UINT[elem_bytes]
    n = int(np.prod(shape)) * elem_bytes
    return np.frombuffer(rng.bytes(n), dtype=t).reshape(shape).copy()


def special_f16_bits() -> np.ndarray:
    """Every fp16 class at least once: +-0, subnormals, normals, +-inf, quiet
    and signalling NaNs with payloads."""
    vals = [0x0000, 0x8000, 0x0001, 0x03FF, 0x8001, 0x83FF, 0x0400, 0x3C00,
            0xBC00, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00, 0x7C01, 0x7DFF, 0x7E00,
            0x7FFF, 0xFE01, 0xFFFF]
    return np.array(vals, dtype=np.uint16)


def special_f32_bits() -> np.ndarray:
    """fp32 counterpart of :func:`special_f16_bits`."""
    vals = [0x00000000, 0x80000000, 0x00000001, 0x007FFFFF, 0x80000001,
            0x00800000, 0x3F800000, 0xBF800000, 0x7F7FFFFF, 0x7F800000,
            0xFF800000, 0x7F800001, 0x7FBFFFFF, 0x7FC00000, 0x7FFFFFFF,
            0xFFC00001, 0xFFFFFFFF]
    return np.array(vals, dtype=np.uint32)
