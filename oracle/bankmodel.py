"""LDS / shared-memory bank-conflict model -- TEST INFRASTRUCTURE ONLY.

The rules, as the pages state them:

* Memory is split into banks interleaved every 4-byte word: word ``w`` lives
  in bank ``w mod NB``; the pages' hardware has NB = 32.  ("Padded Shared
  Memory: Eliminating Bank Conflicts", section "How Shared Memory Is
  Addressed"; "Shared Memory and Bank Conflicts", section "how banking
  works"; "Shared memory and the bank conflict", section "Banks";
  "Shared-memory tiling and bank conflicts", section "Calculate the bank
  mapping".)
* Lanes asking for the *same* word are served by one broadcast: a repeated
  bank alone is not a conflict, compare complete addresses.  ("how banking
  works"; "Calculate the bank mapping"; "Common errors".)
* ``n`` distinct words that share a bank are served serially, so such a
  request takes ``n`` steps.  ("How Shared Memory Is Addressed"; "Banks".)
* The lanes that compete for banks form one group; on the pages' hardware
  that is a 32-lane warp, and for 64-lane wavefronts they state that each
  half of the wavefront is analysed on its own, so the group is 32 lanes.
  ("Shared Memory and Bank Conflicts", section "the wave size
  complication".)

The pages leave wider accesses to the target's documentation ("Calculate the
bank mapping").  Reading adopted here: a lane whose access spans ``k``
consecutive words occupies all ``k`` banks, and the group size for a given
access width is a parameter, so the same model can be evaluated under
several hypotheses about gfx950 (the hardware decides; the model only
predicts which layouts should measure conflict-free).
"""
from __future__ import annotations

from typing import Iterable, Sequence

WORD_BYTES = 4


def bank_of(word_addr: int, banks: int = 32) -> int:
    """Bank holding a 4-byte word: the word address modulo the bank count."""
    return word_addr % banks


def group_degree(lane_words: Sequence[Iterable[int]], banks: int = 32) -> int:
    """Conflict degree of one execution group.

    ``lane_words[l]`` lists the word addresses lane ``l`` touches (one word for
    a 32-bit access, several consecutive words for a wider one; an inactive
    lane passes an empty list).  Equal addresses are merged (broadcast); the
    degree is the largest number of *distinct* words any single bank must
    serve.  1 means conflict-free, 0 means no lane was active.
    """
    per_bank: dict[int, set] = {}
    for words in lane_words:
        for w in words:
            per_bank.setdefault(bank_of(w, banks), set()).add(w)
    return max((len(s) for s in per_bank.values()), default=0)


def access_cycles(lane_words: Sequence[Iterable[int]], banks: int = 32,
                  group: int = 32) -> list[int]:
    """Per-group degrees for one instruction: lanes are split into
    consecutive groups of ``group`` lanes, each served on its own."""
    return [group_degree(lane_words[g:g + group], banks)
            for g in range(0, len(lane_words), group)]


def conflict_degree(lane_words: Sequence[Iterable[int]], banks: int = 32,
                    group: int = 32) -> int:
    """Worst per-group degree of one instruction (1 = conflict-free)."""
    return max(access_cycles(lane_words, banks, group), default=0)


def scalar_words(word_addrs: Iterable[int]) -> list[list[int]]:
    """Wrap one 32-bit word address per lane into ``lane_words`` form."""
    return [[w] for w in word_addrs]


def vector_words(byte_addrs: Iterable[int], width_bytes: int) -> list[list[int]]:
    """``lane_words`` for lanes that each access ``width_bytes`` consecutive
    bytes starting at the given byte address (4-byte aligned)."""
    out = []
    for a in byte_addrs:
        if a % WORD_BYTES:
            raise ValueError("LDS accesses in this model are word-aligned")
        first = a // WORD_BYTES
        out.append(list(range(first, first + width_bytes // WORD_BYTES)))
    return out


def tile_bytes(rows: int, cols: int, pad_cols: int, elem_bytes: int) -> int:
    """Storage of a ``rows x (cols + pad_cols)`` tile.  Padding exists only in
    on-chip storage; the logical tile is unchanged ("Shared-memory tiling and
    bank conflicts", worked example)."""
    return rows * (cols + pad_cols) * elem_bytes


# --------------------------------------------------------------------------
# The access patterns the pages analyse, so their printed results can pin the
# model.  Each returns one instruction's lane_words for a 32-lane warp.
# --------------------------------------------------------------------------

def column_read(stride_words: int, col: int = 0, lanes: int = 32):
    """Lane t reads tile[t][col] of a row-major tile whose row stride is
    ``stride_words`` ("Shared Memory and Bank Conflicts", "the classic case";
    "Shared memory and the bank conflict", "Banks")."""
    return scalar_words(t * stride_words + col for t in range(lanes))


def row_write(stride_words: int, row: int = 0, lanes: int = 32):
    """Lane t writes tile[row][t] ("Shared memory and the bank conflict",
    "Banks": the load phase stores one tile row per warp)."""
    return scalar_words(row * stride_words + t for t in range(lanes))


def sgemm_as_store(bk: int, a_stride: int, j: int, offset: int = 0,
                   lanes: int = 32):
    """The transposed store of A into the shared buffer As in the SGEMM
    kernel of "Padded Shared Memory: Eliminating Bank Conflicts" (section
    "How Shared Memory Is Addressed"): a thread loads four consecutive
    floats of one row of A and stores component j at
    (col * 4 + j) * stride + row + offset, with row = tid / (BK / 4) and
    col = tid % (BK / 4)."""
    per_row = bk // 4
    return scalar_words((t % per_row * 4 + j) * a_stride + t // per_row + offset
                        for t in range(lanes))


def sgemm_a_pad(bk: int) -> int:
    """Pad the SGEMM page adds to the As row stride for a given BK ("Padded
    Shared Memory", section "The Fix Is One Constant"; values listed in
    "Mechanics", item 1)."""
    return (32 // bk) % 8
