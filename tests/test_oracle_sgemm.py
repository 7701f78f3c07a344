"""Pins of the SGEMM oracle (oracle/sgemm.py) against what the mathematics
fixes, independently of the oracle's own formula: exact rational brute force
on tiny shapes, closed forms, the identity matrix, the transpose identity
(A B)^T = B^T A^T, and the readings it takes (pitch padding ignored, beta == 0
makes C write-only, k == 0).  Each pin is also run against planted mistakes
in a copy of the oracle (a dropped term, a wrong sign, a transposed operand,
a wrong pitch, a short sum), each of which at least one pin must catch."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle.sgemm as og
import workloads as wl


def flat(M: np.ndarray, ld: int, fill=np.nan) -> np.ndarray:
    """Row-major matrix M in a flat float32 buffer of pitch ld, the padding
    (and one spare element) filled with ``fill``."""
    rows, cols = M.shape
    buf = np.full(rows * ld + 1, fill, dtype=np.float32)
    for i in range(rows):
        buf[i * ld:i * ld + cols] = M[i]
    return buf


def call(fn, A, B, C, alpha, beta, pad=(0, 0, 0), fill=np.nan):
    m, k = A.shape
    n = B.shape[1]
    lda, ldb, ldc = max(k, 1) + pad[0], max(n, 1) + pad[1], max(n, 1) + pad[2]
    return fn(m, n, k, alpha, flat(A, lda, fill), lda, flat(B, ldb, fill), ldb,
              beta, flat(C, ldc, fill), ldc)


# ----- pins, each taking the function under test -----------------------------

def pin_brute_force(fn):
    """Every shape up to 4 x 4 x 4 (k = 0 included) against exact rational
    arithmetic; float64 evaluation may differ from the exact value by at
    most (k + 2) * 2^-53 of the absolute sum."""
    rng = np.random.default_rng(101)
    for m, n, k in itertools.product(range(1, 5), range(1, 5), range(0, 5)):
        A = wl.uniform_f32((m, k), int(rng.integers(1 << 30)))
        B = wl.uniform_f32((k, n), int(rng.integers(1 << 30)))
        C = wl.uniform_f32((m, n), int(rng.integers(1 << 30)))
        for alpha, beta in ((1.0, 0.0), (1.5, -0.75), (-2.0, 1.0)):
            got = call(fn, A, B, C, alpha, beta, pad=(1, 2, 3))
            exact = og.sgemm_exact(A.tolist(), B.tolist(), C.tolist(),
                                   float(np.float32(alpha)),
                                   float(np.float32(beta)))
            for i in range(m):
                for j in range(n):
                    mag = abs(alpha) * sum(abs(Fraction(float(A[i][l])) *
                                               Fraction(float(B[l][j])))
                                           for l in range(k))
                    mag += abs(Fraction(beta) * Fraction(float(C[i][j])))
                    err = abs(Fraction(float(got[i][j])) - exact[i][j])
                    assert err <= (k + 2) * Fraction(1, 1 << 53) * mag, \
                        (m, n, k, i, j)


def pin_closed_forms(fn):
    """Matrices whose product has a closed form, at several shapes, some
    square so that a transposed operand cannot pass by shape alone.
    Integer values keep every float64 step exact."""
    for m, n, k in ((5, 7, 9), (6, 6, 6), (33, 17, 65), (16, 16, 16)):
        i = np.arange(m, dtype=np.float32)[:, None]
        j = np.arange(n, dtype=np.float32)[None, :]
        l_row = np.arange(k, dtype=np.float32)[None, :]
        l_col = np.arange(k, dtype=np.float32)[:, None]
        C = (i - 2 * j).astype(np.float32)
        # A[i][l] = i + 1, B[l][j] = j + 1  ->  (A B)[i][j] = k (i + 1)(j + 1)
        A = np.broadcast_to(i + 1, (m, k)).astype(np.float32)
        B = np.broadcast_to(j + 1, (k, n)).astype(np.float32)
        got = call(fn, A, B, C, 2.0, -1.0)
        assert np.array_equal(got, 2.0 * k * (i + 1) * (j + 1) - C)
        # A[i][l] = l, B = 1  ->  k (k - 1) / 2 everywhere
        A = np.broadcast_to(l_row, (m, k)).astype(np.float32)
        B = np.ones((k, n), dtype=np.float32)
        got = call(fn, A, B, C, 1.0, 0.0)
        assert np.array_equal(got, np.full((m, n), k * (k - 1) / 2))
        # A[i][l] = (i + 1) l, B[l][j] = (j + 2) - l: the sum over l of
        # (i + 1) l (j + 2 - l) = (i + 1) ((j + 2) S1 - S2)
        A = ((i + 1) * l_row).astype(np.float32)
        B = ((j + 2) - l_col).astype(np.float32)
        s1, s2 = k * (k - 1) / 2, (k - 1) * k * (2 * k - 1) / 6
        got = call(fn, A, B, C, 1.0, 3.0)
        assert np.array_equal(got, (i + 1) * ((j + 2) * s1 - s2) + 3.0 * C)


def pin_identity(fn):
    """A = I: C' = alpha B + beta C, exactly for power-of-two scalars."""
    for m, n in ((1, 1), (7, 3), (32, 45)):
        B = wl.uniform_f32((m, n), 7)
        C = wl.uniform_f32((m, n), 8)
        got = call(fn, np.eye(m, dtype=np.float32), B, C, 2.0, 0.5)
        assert np.array_equal(got, 2.0 * B.astype(np.float64) + 0.5 * C)


def pin_transpose_identity(fn):
    """(A B)^T = B^T A^T, exactly on small integers."""
    for m, n, k in ((3, 5, 7), (20, 9, 31)):
        A = wl.small_int_f32((m, k), 21)
        B = wl.small_int_f32((k, n), 22)
        Z = np.zeros((m, n), np.float32)
        got = call(fn, A, B, Z, 1.0, 0.0)
        got_t = call(fn, np.ascontiguousarray(B.T), np.ascontiguousarray(A.T),
                     np.zeros((n, m), np.float32), 1.0, 0.0)
        assert np.array_equal(got, got_t.T)
        assert np.isfinite(got).all() and np.abs(got).max() > 0


def pin_padding_ignored(fn):
    """NaN in every pitch gap must not reach the result, which must equal
    the dense computation."""
    A = wl.small_int_f32((9, 13), 31)
    B = wl.small_int_f32((13, 11), 32)
    C = wl.small_int_f32((9, 11), 33)
    dense = call(fn, A, B, C, 1.0, 2.0, pad=(0, 0, 0), fill=0.0)
    padded = call(fn, A, B, C, 1.0, 2.0, pad=(3, 5, 7), fill=np.nan)
    assert np.isfinite(padded).all()
    assert np.array_equal(dense, padded)


def pin_beta_zero(fn):
    """beta == 0 leaves the old C unread: NaN there does not leak."""
    A = wl.small_int_f32((6, 5), 41)
    B = wl.small_int_f32((5, 4), 42)
    C = np.full((6, 4), np.nan, np.float32)
    got = call(fn, A, B, C, 1.0, 0.0)
    assert np.isfinite(got).all()
    ones = call(fn, A, B, np.ones((6, 4), np.float32), 1.0, 1.0)
    assert np.array_equal(got + 1.0, ones)


def pin_k_zero(fn):
    """An empty sum is zero: C' = beta C."""
    C = wl.uniform_f32((4, 6), 51)
    got = call(fn, np.zeros((4, 0), np.float32), np.zeros((0, 6), np.float32),
               C, 3.0, -0.5)
    assert np.array_equal(got, -0.5 * C.astype(np.float64))


PINS = [pin_brute_force, pin_closed_forms, pin_identity,
        pin_transpose_identity, pin_padding_ignored, pin_beta_zero,
        pin_k_zero]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(og.sgemm)


# ----- planted mistakes (CPU only): each must fail at least one pin ----------

def _mutant(kind):
    def fn(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc):
        al, be = float(np.float32(alpha)), float(np.float32(beta))
        A = og._view(a, m, k, lda)
        B = og._view(b, k, n, ldb)
        Cold = og._view(c, m, n, ldc)
        if kind == "dropped_beta":
            return al * (A @ B)
        if kind == "wrong_sign":
            return -al * (A @ B) + (be * Cold if be else 0.0)
        if kind == "transposed_b":
            # only where the shapes allow it, so the square pins must see it
            Bt = B.T if k == n else B
            return al * (A @ Bt) + (be * Cold if be else 0.0)
        if kind == "pitch_of_a":
            A = og._view(a, m, k, k) if k else A
            return al * (A @ B) + (be * Cold if be else 0.0)
        if kind == "short_sum":
            return al * (A[:, :-1] @ B[:-1, :] if k else A @ B) + \
                (be * Cold if be else 0.0)
        if kind == "beta_always_reads_c":
            return al * (A @ B) + be * Cold
        raise AssertionError(kind)
    return fn


@pytest.mark.parametrize("kind", ["dropped_beta", "wrong_sign", "transposed_b",
                                  "pitch_of_a", "short_sum",
                                  "beta_always_reads_c"])
def test_planted_mistakes_are_caught(kind):
    fn = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, kind


def test_sgemm_into_leaves_pitch_padding():
    A = wl.small_int_f32((5, 3), 61)
    B = wl.small_int_f32((3, 4), 62)
    ldc = 7
    c = np.full(5 * ldc, -7.0, np.float32)
    og.sgemm_into(5, 4, 3, 1.0, flat(A, 3), 3, flat(B, 4), 4, 0.0, c, ldc)
    got = c.reshape(5, ldc)
    assert (got[:, 4:] == -7.0).all()
    assert np.array_equal(got[:, :4], A.astype(np.float64) @ B)


def test_gemm_workload():
    w = wl.GEMM_WORKLOADS["sgemm_4096"]
    assert (w.m, w.n, w.k) == (4096, 4096, 4096)
    assert w.flops == 2 * 4096 ** 3
    a = wl.uniform_f32((3, 5), 9)
    assert a.dtype == np.float32 and (a >= -1).all() and (a < 1).all()
    s = wl.small_int_f32((100,), 9, bound=4)
    assert set(np.unique(s)) <= set(range(-4, 5))
