"""The race detector's own check (CPU): the index check must catch a
missing barrier.

The tiled transpose's second phase reads LDS words that other waves wrote
in the first, so the barrier between the phases is what makes it correct
("Shared memory and the bank conflict", section "The barrier"; the index
check of the same page is the detector).  A kernel with the barrier taken
out is not run on the GPU; instead this models one workgroup of the tiled
transpose on the CPU: four waves, each loading a quarter of the tile's rows
into a shared tile that still holds the previous tile's data, then
gathering a quarter of the tile's columns.  With the barrier every load
precedes every gather and the index check passes on every schedule; with
it removed, a schedule that lets one wave gather before the others have
loaded must fail the index check."""
import itertools

import numpy as np

import oracle
import workloads as wl

T = 32      # tile edge
WAVES = 4   # waves per workgroup; wave w loads rows and gathers columns w*8..


def run_tile(src, stale, schedule):
    """Execute one workgroup under `schedule`, a sequence of (wave, phase)
    steps; returns the T x T output tile."""
    lds = stale.copy()
    out = np.zeros((T, T), dtype=src.dtype)
    rows = T // WAVES
    for w, phase in schedule:
        part = slice(w * rows, (w + 1) * rows)
        if phase == 1:
            lds[part, :] = src[part, :]          # coalesced row loads
        else:
            out[part, :] = lds[:, part].T        # column gathers
    return out


def schedules(barrier):
    """Every order of the waves' steps the hardware may produce: each wave
    loads before it gathers; with the barrier, all loads come first."""
    steps = [(w, p) for w in range(WAVES) for p in (1, 2)]
    for perm in itertools.permutations(steps):
        if any(perm.index((w, 1)) > perm.index((w, 2)) for w in range(WAVES)):
            continue
        if barrier and max(perm.index((w, 1)) for w in range(WAVES)) > \
                min(perm.index((w, 2)) for w in range(WAVES)):
            continue
        yield perm


def index_check(out, src):
    return np.array_equal(out, oracle.transpose(src))


def test_barrier_makes_every_schedule_pass():
    src = wl.linear_index_plane((T, T), 4)
    stale = wl.linear_index_plane((T, T), 4)[::-1].copy()  # previous tile
    n = 0
    for sched in schedules(barrier=True):
        assert index_check(run_tile(src, stale, sched), src)
        n += 1
    assert n == 24 * 24  # loads in any order, then gathers in any order


def test_missing_barrier_is_caught():
    src = wl.linear_index_plane((T, T), 4)
    stale = wl.linear_index_plane((T, T), 4)[::-1].copy()
    caught = passed = 0
    for sched in schedules(barrier=False):
        if index_check(run_tile(src, stale, sched), src):
            passed += 1
        else:
            caught += 1
    # The schedules where every wave happens to load before any gathers are
    # the only ones that pass; every other one fails the index check.
    assert passed == 24 * 24
    assert caught > 0
