"""Pins for the transpose oracle (CPU only).

Each check below ties the oracle to something other than itself: the
pages' exact index check, brute force against a list definition, numpy's own
transpose, and invariants every transpose must satisfy.  The planted-mistake
test at the end shows that each plausible slip (no permutation, a transposed
shape without moving data, an off-by-one, wrong axes in a batch, a dropped
edge) fails at least one of these checks.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SIZES = (1, 2, 4, 8)


# --------------------------------------------------------------------------
# Check functions: each takes a dense transpose function fn(a) -> out and
# raises AssertionError when fn disagrees with what the pages or mathematics
# fix.  They run against the real oracle below and against planted mistakes
# at the end of the file.
# --------------------------------------------------------------------------

def check_bruteforce(fn, max_dim=9):
    """Every shape up to max_dim x max_dim, every element size, against the
    list-of-lists definition out[j][i] = in[i][j]."""
    for s in SIZES:
        for r in range(1, max_dim + 1):
            for c in range(1, max_dim + 1):
                a = wl.random_bits((r, c), s, seed=1000 * s + 10 * r + c)
                want = oracle.transpose_lists(a.tolist())
                got = fn(a)
                assert got.shape == (c, r), (s, r, c)
                assert got.tolist() == want, (s, r, c)


def check_golden_index(fn):
    """The hand-written 3x4 index fixture."""
    with open(os.path.join(GOLDEN, "index_3x4.txt")) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert lines[0][0] == "input"
    r, c = int(lines[0][1]), int(lines[0][2])
    a = np.array([[int(x) for x in ln] for ln in lines[1:1 + r]], dtype=np.uint32)
    hdr = lines[1 + r]
    assert hdr[0] == "output" and (int(hdr[1]), int(hdr[2])) == (c, r)
    want = np.array([[int(x) for x in ln] for ln in lines[2 + r:2 + r + c]],
                    dtype=np.uint32)
    assert np.array_equal(fn(a), want)


def check_index_valued(fn, rows=1024, cols=1024):
    """Every element holds its own row-major index, so out[r][c] must hold
    c * cols + r ("Shared memory and the bank conflict", "The barrier":
    when each element carries its index, a single misplaced element shows)."""
    a = np.arange(rows * cols, dtype=np.float32).reshape(rows, cols)
    out = fn(a)
    want = (np.arange(rows, dtype=np.float32)[None, :] * np.float32(cols)
            + np.arange(cols, dtype=np.float32)[:, None])
    assert out.shape == (cols, rows)
    assert out.dtype == np.float32
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def check_planes(fn, shapes=((37, 53), (53, 37), (1, 100), (100, 1), (64, 65))):
    """Coordinate planes: with in[i][j] = i the output must hold its column
    index everywhere, and with in[i][j] = j its row index.  Together they fix
    every element's destination uniquely."""
    for s in (2, 4, 8):
        for shape in shapes:
            rows_plane = wl.index_plane(shape, 0, s)
            cols_plane = wl.index_plane(shape, 1, s)
            out_r = fn(rows_plane)
            out_c = fn(cols_plane)
            r_out, c_out = shape[1], shape[0]
            assert out_r.shape == (r_out, c_out)
            assert np.array_equal(out_r, wl.index_plane((r_out, c_out), 1, s))
            assert np.array_equal(out_c, wl.index_plane((r_out, c_out), 0, s))


def check_involution(fn):
    """Transposing twice gives back the input, bit for bit, NaN payloads
    and all."""
    for s in SIZES:
        for shape in ((7, 300), (129, 65), (3, 17, 31)):
            a = wl.random_bits(shape, s, seed=77 + s)
            assert np.array_equal(fn(fn(a)), a), (s, shape)


def check_numpy(fn):
    """numpy's own transpose on medium shapes (a textbook routine used only
    to check the oracle)."""
    for s in SIZES:
        a = wl.random_bits((300, 517), s, seed=5 + s)
        assert np.array_equal(fn(a), np.ascontiguousarray(a.T)), s
        b = wl.random_bits((5, 33, 70), s, seed=9 + s)
        assert np.array_equal(fn(b), np.ascontiguousarray(np.swapaxes(b, 1, 2))), s


def check_invariants(fn):
    """Multiset of bit patterns preserved; a single row or column keeps its
    byte order; a symmetric matrix is a fixed point."""
    a = wl.random_bits((41, 77), 4, seed=3)
    out = fn(a)
    assert np.array_equal(np.sort(out, axis=None), np.sort(a, axis=None))
    row = wl.random_bits((1, 1000), 2, seed=4)
    assert fn(row).tobytes() == row.tobytes()
    col = wl.random_bits((1000, 1), 2, seed=4)
    assert fn(col).tobytes() == col.tobytes()
    m = wl.random_bits((50, 50), 4, seed=6)
    sym = np.triu(m) + np.triu(m, 1).T
    assert np.array_equal(fn(sym), sym)


def check_batched(fn):
    """Each matrix of a batch is transposed on its own; the batch axis stays
    first."""
    a = wl.random_bits((6, 19, 23), 4, seed=12)
    out = fn(a)
    assert out.shape == (6, 23, 19)
    for b in range(6):
        assert out[b].tolist() == oracle.transpose_lists(a[b].tolist())


ALL_CHECKS = [check_bruteforce, check_golden_index, check_index_valued,
              check_planes, check_involution, check_numpy, check_invariants,
              check_batched]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle.transpose)


# --------------------------------------------------------------------------
# Strided interface: leading dimensions, batch gaps, zero sizes, bad input.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("s", SIZES)
def test_ld_padding_untouched(s):
    rows, cols, ld_in, ld_out = 29, 45, 51, 33
    t = wl.RAW_UINT[s]
    src = wl.random_bits((rows, ld_in), s, seed=21).reshape(-1)
    sentinel = t(0xA5A5A5A5A5A5A5A5 & ((1 << (8 * s)) - 1))
    guard = 40
    out = np.full(guard + cols * ld_out + guard, sentinel, dtype=t)
    body = out[guard:guard + cols * ld_out]
    oracle.transpose_into(body, src, 1, rows, cols, ld_in, ld_out)
    got = body.reshape(cols, ld_out)
    want = np.ascontiguousarray(src.reshape(rows, ld_in)[:, :cols].T)
    assert np.array_equal(got[:, :rows], want)
    assert np.all(got[:, rows:] == sentinel)
    assert np.all(out[:guard] == sentinel) and np.all(out[-guard:] == sentinel)


def test_batch_gaps_untouched():
    batch, rows, cols = 4, 10, 7
    ld_in, ld_out = 9, 12
    stride_in, stride_out = rows * ld_in + 5, cols * ld_out + 11
    src = wl.random_bits((batch * stride_in,), 4, seed=31)
    out = np.full(batch * stride_out, 0xDEADBEEF, dtype=np.uint32)
    oracle.transpose_into(out, src, batch, rows, cols, ld_in, ld_out,
                          stride_in, stride_out)
    written = np.zeros(out.size, dtype=bool)
    for b in range(batch):
        m = src[b * stride_in: b * stride_in + rows * ld_in].reshape(rows, ld_in)
        o = out[b * stride_out: b * stride_out + cols * ld_out].reshape(cols, ld_out)
        assert np.array_equal(o[:, :rows], m[:, :cols].T)
        w = written[b * stride_out: b * stride_out + cols * ld_out].reshape(cols, ld_out)
        w[:, :rows] = True
    assert np.all(out[~written] == 0xDEADBEEF)


def test_zero_sizes_are_noops():
    out = np.full(16, 7, dtype=np.uint32)
    src = np.arange(16, dtype=np.uint32)
    for b, r, c in ((0, 4, 4), (1, 0, 4), (1, 4, 0)):
        oracle.transpose_into(out, src, b, r, c, max(c, 1), max(r, 1), 16, 16)
    assert np.all(out == 7)
    assert oracle.transpose(np.zeros((0, 5), np.float32)).shape == (5, 0)


def test_bad_arguments_rejected():
    out = np.zeros(64, dtype=np.uint32)
    src = np.zeros(64, dtype=np.uint32)
    with pytest.raises(ValueError):
        oracle.transpose_into(out, src, 1, 8, 8, 7, 8)          # ld_in < cols
    with pytest.raises(ValueError):
        oracle.transpose_into(out, src, 1, 8, 8, 8, 7)          # ld_out < rows
    with pytest.raises(ValueError):
        oracle.transpose_into(out, src, 1, 9, 8, 8, 9)          # past the end
    with pytest.raises(ValueError):
        oracle.transpose_into(out, src.astype(np.uint16), 1, 2, 2, 2, 2)


def test_c1_workload_exact_index_check():
    """The 1024x1024 index-valued workload: out[r][c] == float(c*1024 + r)."""
    w = wl.WORKLOADS["c1_index_1024_f32"]
    a = wl.make_input(w)
    out = oracle.transpose(a)
    r = np.arange(1024)[:, None]
    c = np.arange(1024)[None, :]
    assert np.array_equal(out, (c * 1024 + r).astype(np.float32))


# --------------------------------------------------------------------------
# Planted mistakes: every one must be caught by at least one check.
# --------------------------------------------------------------------------

def _swap_last(a):
    return np.ascontiguousarray(np.swapaxes(a, -1, -2))


MUTANTS = {
    # shape changes but no element moves
    "reshape_only": lambda a: np.ascontiguousarray(a).reshape(
        a.shape[:-2] + (a.shape[-1], a.shape[-2])),
    # output rows in reverse order
    "reversed_rows": lambda a: np.ascontiguousarray(_swap_last(a)[..., ::-1, :]),
    # one-element slip along the output row
    "off_by_one": lambda a: np.roll(_swap_last(a), 1, axis=-1),
    # batch axis exchanged with the row axis
    "wrong_axes": lambda a: (np.ascontiguousarray(np.swapaxes(a, 0, 1))
                             if a.ndim == 3 else _swap_last(a)),
    # last input column dropped (edge not handled)
    "dropped_edge": lambda a: np.concatenate(
        [_swap_last(a)[..., :-1, :], np.zeros_like(_swap_last(a)[..., -1:, :])],
        axis=-2) if a.shape[-1] > 1 else _swap_last(a),
    # square blocks only: the ragged part of the matrix is left behind
    "square_part_only": lambda a: _square_only(a),
}


def _square_only(a):
    out = np.zeros(a.shape[:-2] + (a.shape[-1], a.shape[-2]), dtype=a.dtype)
    n = min(a.shape[-1], a.shape[-2])
    out[..., :n, :n] = _swap_last(a[..., :n, :n])
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    fn = MUTANTS[name]
    caught = []
    for check in ALL_CHECKS:
        try:
            check(fn)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every check"


def test_overlapping_inputs_allowed_outputs_not():
    """Input matrices may coincide (they are only read); output matrices may
    not overlap."""
    src = wl.random_bits((12 * 9,), 4, seed=40)
    out = np.zeros(3 * 9 * 12, dtype=np.uint32)
    oracle.transpose_into(out, src, 3, 12, 9, 9, 12, 0, 9 * 12)
    one = np.ascontiguousarray(src.reshape(12, 9).T).reshape(-1)
    assert np.array_equal(out.reshape(3, -1), np.stack([one] * 3))
    with pytest.raises(ValueError):
        oracle.transpose_into(out, src, 3, 12, 9, 9, 12, 0, 9 * 12 - 1)
