"""Oracle for the out-of-place transpose -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library under test never imports, links or runs
anything here, and this package imports nothing from the library.

Contents
--------
``transpose`` / ``transpose_into``
    The plain definition of a transpose, out[b][j][i] = in[b][i][j], run by
    the single-threaded C loop in ``xpose_ref.c`` (built with gcc into
    ``liboracle.so``).  Source: "Shared memory and the bank conflict",
    section "Turn the tile around on chip" (a thread loads in[y][x] and the
    transposed tile is stored at out[x][y]), and "Shared-memory tiling and
    bank conflicts", section "Reference summary" (non-square form
    out[col * height + row] = in[row * width + col]).

``transpose_lists``
    The same definition on Python lists, for tiny brute-force cases.

``bankmodel``
    The pages' LDS bank-conflict model (a separate module).

Pins (``tests/test_oracle.py``): brute force on every shape up to 9x9 against
the list definition, index-valued inputs (every element holds its own index),
raw-bit coordinate planes, transpose of a transpose is the identity, numpy's
own transpose on medium shapes, untouched leading-dimension padding and
batch gaps, and planted mistakes that each pin must catch.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import bankmodel  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64 = ctypes.c_int64
        lib.oracle_xpose.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64,
                                     i64, i64, i64, i64, i64, i64]
        lib.oracle_xpose.restype = ctypes.c_int
        _lib = lib
    return _lib


def transpose_into(out: np.ndarray, inp: np.ndarray, batch: int, rows: int,
                   cols: int, ld_in: int, ld_out: int, stride_in: int = 0,
                   stride_out: int = 0) -> None:
    """Strided transpose between two flat host buffers of the same itemsize.

    ``out`` and ``inp`` are C-contiguous numpy arrays; their itemsize is the
    element size.  Leading dimensions and batch strides are in elements, as
    in the C ABI.  Elements of ``out`` outside each output matrix's
    ``cols x rows`` region are left as they were.
    """
    if out.dtype.itemsize != inp.dtype.itemsize:
        raise ValueError("element sizes differ")
    if not (out.flags.c_contiguous and inp.flags.c_contiguous):
        raise ValueError("buffers must be C-contiguous")
    if not out.flags.writeable:
        raise ValueError("output buffer is read-only")
    # Bounds of the furthest element touched, checked here so the C loop can
    # stay a plain loop.
    if batch > 0 and rows > 0 and cols > 0:
        last_in = (batch - 1) * stride_in + (rows - 1) * ld_in + cols - 1
        last_out = (batch - 1) * stride_out + (cols - 1) * ld_out + rows - 1
        if last_in >= inp.size or last_out >= out.size:
            raise ValueError("strided extent exceeds the buffer")
    rc = _load().oracle_xpose(out.ctypes.data, inp.ctypes.data, batch, rows,
                              cols, ld_in, ld_out, stride_in, stride_out,
                              out.dtype.itemsize)
    if rc != 0:
        raise ValueError(f"oracle_xpose rejected the arguments (rc={rc})")


def transpose(a: np.ndarray) -> np.ndarray:
    """Transpose of a (rows, cols) or (batch, rows, cols) array.

    Returns a new C-contiguous array of shape (cols, rows) or
    (batch, cols, rows) with the same dtype; values are moved as raw bits.
    """
    a = np.ascontiguousarray(a)
    if a.ndim == 2:
        batch, (rows, cols) = 1, a.shape
        out = np.empty((cols, rows), dtype=a.dtype)
    elif a.ndim == 3:
        batch, rows, cols = a.shape
        out = np.empty((batch, cols, rows), dtype=a.dtype)
    else:
        raise ValueError("expected a 2-D or 3-D array")
    transpose_into(out.reshape(-1), a.reshape(-1), batch, rows, cols,
                   ld_in=cols, ld_out=rows, stride_in=rows * cols,
                   stride_out=rows * cols)
    return out


def transpose_lists(m: list) -> list:
    """out[j][i] = m[i][j] on a list of equal-length lists, by brute force."""
    rows = len(m)
    cols = len(m[0]) if rows else 0
    out = [[None] * rows for _ in range(cols)]
    for i in range(rows):
        for j in range(cols):
            out[j][i] = m[i][j]
    return out
