"""Pins for the bank-conflict model (CPU only): every degree and tile size
the pages print, read from ``golden/bank_examples.txt``, plus planted
mistakes in the model that those values must catch."""
import os

import pytest

from oracle import bankmodel as bm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bank_examples.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for ln in f:
            if not ln.strip() or ln.startswith("#"):
                continue
            pattern, params, expected, source = [x.strip() for x in ln.split("|")]
            kv = dict(p.split("=") for p in params.split())
            rows.append((pattern, {k: int(v) for k, v in kv.items()},
                         int(expected), source))
    return rows


GOLDEN_ROWS = _golden()


def evaluate(pattern, p, model=bm):
    """Evaluate one golden pattern with a model module (or a planted-mistake
    stand-in exposing the same functions)."""
    if pattern == "column_read":
        return model.conflict_degree(bm.column_read(p["stride"], p["col"]))
    if pattern == "row_write":
        return model.conflict_degree(bm.row_write(p["stride"], p["row"]))
    if pattern == "broadcast":
        return model.conflict_degree(bm.scalar_words([p["addr"]] * 32))
    if pattern == "sgemm_as_store":
        # The pages quote one degree for all four component stores.
        degs = {model.conflict_degree(bm.sgemm_as_store(p["bk"], p["a_stride"], j))
                for j in range(4)}
        assert len(degs) == 1
        return degs.pop()
    if pattern == "sgemm_a_pad":
        return bm.sgemm_a_pad(p["bk"])
    if pattern == "tile_bytes":
        return bm.tile_bytes(p["rows"], p["cols"], p["pad"], p["elem"])
    raise KeyError(pattern)


def test_golden_file_covers_each_pattern():
    kinds = {r[0] for r in GOLDEN_ROWS}
    assert kinds == {"column_read", "row_write", "broadcast", "sgemm_as_store",
                     "sgemm_a_pad", "tile_bytes"}


@pytest.mark.parametrize("row", GOLDEN_ROWS, ids=lambda r: f"{r[0]}:{r[1]}")
def test_pages_printed_values(row):
    pattern, params, expected, _ = row
    assert evaluate(pattern, params) == expected


def test_half_wave_caveat():
    """A 64-lane column read of a 33-stride tile: conflict-free when the
    hardware resolves it per 32-lane half ("Shared Memory and Bank
    Conflicts", "the wave size complication"), but 2-way if 64 lanes shared
    32 banks at once -- the reason a 32-lane padding does not port blindly."""
    lanes = bm.column_read(33, lanes=64)
    assert bm.conflict_degree(lanes, banks=32, group=32) == 1
    assert bm.conflict_degree(lanes, banks=32, group=64) == 2
    assert bm.conflict_degree(lanes, banks=64, group=64) == 1
    assert bm.access_cycles(lanes, banks=32, group=32) == [1, 1]


def test_wide_access_occupies_each_word():
    # Eight lanes of 16-byte accesses over one 128-byte stretch: 32 distinct
    # words in 32 banks.  The same eight lanes at a 128-byte stride collide.
    flat = bm.vector_words((16 * l for l in range(8)), 16)
    assert bm.conflict_degree(flat, banks=32, group=8) == 1
    strided = bm.vector_words((128 * l for l in range(8)), 16)
    assert bm.conflict_degree(strided, banks=32, group=8) == 8
    with pytest.raises(ValueError):
        bm.vector_words([2], 4)


# ----- planted mistakes in the model -------------------------------------

class _NoBroadcast:
    """Counts every lane, even lanes reading the same word."""
    @staticmethod
    def conflict_degree(lane_words, banks=32, group=32):
        worst = 0
        for g in range(0, len(lane_words), group):
            count = {}
            for words in lane_words[g:g + group]:
                for w in words:
                    count[w % banks] = count.get(w % banks, 0) + 1
            worst = max(worst, max(count.values(), default=0))
        return worst


class _WrongBankCount:
    """Interleaves over 33 banks instead of 32."""
    @staticmethod
    def conflict_degree(lane_words, banks=32, group=32):
        return bm.conflict_degree(lane_words, banks=33, group=group)


class _ByteBanks:
    """Banks interleaved every byte instead of every 4-byte word."""
    @staticmethod
    def conflict_degree(lane_words, banks=32, group=32):
        as_bytes = [[4 * w for w in words] for words in lane_words]
        return bm.conflict_degree(as_bytes, banks=banks, group=group)


@pytest.mark.parametrize("mutant", [_NoBroadcast, _WrongBankCount, _ByteBanks],
                         ids=lambda m: m.__name__)
def test_planted_model_mistakes_are_caught(mutant):
    misses = [r for r in GOLDEN_ROWS
              if r[0] in ("column_read", "row_write", "broadcast", "sgemm_as_store")
              and evaluate(r[0], r[1], mutant) != r[2]]
    assert misses, f"{mutant.__name__} reproduces every printed value"
