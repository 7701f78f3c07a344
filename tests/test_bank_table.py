"""The committed half-wave address-to-bank table
(profiles/lds_bank_table_c2_column_gather.md) is exactly what
tests/bank_table.py computes from the kernels' current lane maps, and it
shows the pages' contrast: the default and the one-word-pad tiles
conflict-free, the unpadded ones conflicted."""
import os

import pytest

pytest.importorskip("lds_tiled_matrix_amd")

import bank_table  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = os.path.join(ROOT, "profiles", "lds_bank_table_c2_column_gather.md")


def test_committed_table_is_current():
    text = bank_table.render(bank_table.address_lines())
    with open(PROFILE) as f:
        assert f.read() == text, "regenerate: python tests/bank_table.py > " + PROFILE
    degrees = [ln.split("**")[1] for ln in text.splitlines() if "**" in ln]
    assert degrees == ["1-way", "8-way", "1-way", "8-way", "1-way"]
