"""Build the oracle's shared library (test infrastructure only).

    python oracle/build.py

Compiles ``xpose_ref.c`` with the host C compiler into ``liboracle.so`` next
to it.  No HIP headers or libraries are involved.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "xpose_ref.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC", "gcc")
    tmp = LIB + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC",
           "-shared", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
