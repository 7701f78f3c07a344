"""Oracle for the tiled SGEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this module; the library under test never uses it, and it imports
nothing from the library.

What it computes: C' = alpha * A @ B + beta * C for row-major float32
matrices given as flat buffers with row pitches, the operation of the SGEMM
in "Padded Shared Memory: Eliminating Bank Conflicts" (the kernel under "The
Fix Is One Constant"; its epilogue scales the accumulated products by alpha
and adds beta times the old C).  The oracle takes the plain definition,
evaluated in float64 with numpy's matmul as the one library step; nothing is
tiled, blocked or reordered beyond what that matmul does.

Readings (the pages leave these open):
* beta == 0 makes C write-only (the BLAS convention): the old C is not read,
  so NaN there does not reach the result.  The pages' kernel always reads C;
  for finite C the two agree.
* k == 0 gives C' = beta * C (an empty sum is zero).
* Elements of C outside the m x n region (pitch padding) are not part of the
  result and are left alone.

Pins (``tests/test_oracle_sgemm.py``): exact rational brute force on every
shape up to 4 x 4 x 4, closed forms (constant, index-product and ramp
matrices), the identity matrix, (A B)^T = B^T A^T, pitch padding holding NaN
that must not leak, beta == 0 over a NaN-filled C, k == 0, and planted
mistakes (a transposed operand, a dropped beta term, a wrong sign, a wrong
pitch) that the pins must catch.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _view(buf: np.ndarray, rows: int, cols: int, ld: int) -> np.ndarray:
    """rows x cols row-major matrix with row pitch ``ld`` inside a flat
    buffer, as a float64 copy."""
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=np.float64)
    if ld < cols:
        raise ValueError("row pitch smaller than the row")
    last = (rows - 1) * ld + cols
    if last > buf.size:
        raise ValueError("matrix extent exceeds the buffer")
    rows_view = np.lib.stride_tricks.as_strided(
        buf, shape=(rows, cols), strides=(ld * buf.itemsize, buf.itemsize),
        writeable=False)
    return np.array(rows_view, dtype=np.float64)


def sgemm(m: int, n: int, k: int, alpha: float, a: np.ndarray, lda: int,
          b: np.ndarray, ldb: int, beta: float, c: np.ndarray,
          ldc: int) -> np.ndarray:
    """alpha * A @ B + beta * C as an (m, n) float64 array.

    ``a``, ``b`` and ``c`` are flat float32 buffers; A is m x k with pitch
    lda, B is k x n with pitch ldb, C is m x n with pitch ldc (all in
    elements).  alpha and beta are taken as float32 values, as the kernel
    receives them.
    """
    for buf in (a, b, c):
        if buf.dtype != np.float32 or buf.ndim != 1:
            raise ValueError("buffers must be flat float32 arrays")
    alpha64 = float(np.float32(alpha))
    beta64 = float(np.float32(beta))
    A = _view(a, m, k, lda)
    B = _view(b, k, n, ldb)
    out = alpha64 * (A @ B)
    if beta64 != 0.0:
        out = out + beta64 * _view(c, m, n, ldc)
    return out


def sgemm_into(m: int, n: int, k: int, alpha: float, a: np.ndarray, lda: int,
               b: np.ndarray, ldb: int, beta: float, c: np.ndarray,
               ldc: int) -> None:
    """As ``sgemm``, writing the result rounded to float32 into the m x n
    region of ``c`` (pitch padding untouched)."""
    res = sgemm(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc)
    for i in range(m):
        c[i * ldc:i * ldc + n] = res[i].astype(np.float32)


def sgemm_exact(A: list, B: list, C: list, alpha, beta) -> list:
    """The definition on lists of lists, in exact rational arithmetic: for
    tiny brute-force cases (values must be finite floats or ints)."""
    m = len(C)
    n = len(C[0]) if m else 0
    k = len(B)
    al, be = Fraction(alpha), Fraction(beta)
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            s = Fraction(0)
            for l in range(k):
                s += Fraction(A[i][l]) * Fraction(B[l][j])
            v = al * s
            if be != 0:
                v += be * Fraction(C[i][j])
            row.append(v)
        out.append(row)
    return out
