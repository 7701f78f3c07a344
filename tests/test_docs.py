"""The documents cite files by path (tests, profiles, kernels, headers):
every such path must exist, so a rename or a removed profile shows up
here instead of as a dangling reference."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = re.compile(r"`((?:tests|profiles|oracle|include|lds_tiled_matrix_amd|csrc)/[\w./-]+)`")


@pytest.mark.parametrize("doc", ["DESIGN.md", "README.md", "BASELINE.md"])
def test_cited_paths_exist(doc):
    with open(os.path.join(ROOT, doc)) as f:
        cited = set(PATH.findall(f.read()))
    missing = [p for p in sorted(cited)
               if not any(os.path.exists(os.path.join(ROOT, base, p))
                          for base in ("", "lds_tiled_matrix_amd"))]
    assert not missing, missing


def test_every_profile_is_cited():
    """Each committed profile summary is referred to by the design doc or by
    another profile, so none is left unexplained."""
    with open(os.path.join(ROOT, "DESIGN.md")) as f:
        design = f.read()
    names = sorted(os.listdir(os.path.join(ROOT, "profiles")))
    assert names
    uncited = [n for n in names if n not in design]
    assert not uncited, uncited
