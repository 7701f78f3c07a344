"""Build libxpose.so for gfx950 in-tree.

    python lds_tiled_matrix_amd/build.py

hipcc cross-compiles without a GPU.  The library is written next to this
file so it travels with the source tree.  Run as a script (not with -m):
importing the package loads the library, which may be stale or missing.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libxpose.so")
SOURCES = ["xpose_kernels.hip", "xpose_api.cpp", "sgemm_kernels.hip",
           "sgemm_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-variable",
        # No packed-fp32 instructions anywhere in device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (the kernel files take
    most of the time), then link the shared library."""
    import tempfile
    compile_flags = [f for f in flags() if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="xpose_build_") as tmpdir:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc()] + compile_flags + ["-c", "-o", obj,
                                               os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd)))
            objs.append(obj)
        failed = [src for src, p in procs if p.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, f"hipcc -c {failed}")
        tmp = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o",
               tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def dump_isa(out_dir: str) -> None:
    """Write the gfx950 assembly of the kernels (for checking instruction
    selection: LDS widths, global access widths, waits)."""
    os.makedirs(out_dir, exist_ok=True)
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = [hipcc()] + [f for f in flags()
                           if f not in ("-shared", "-fPIC")] + [
            "--cuda-device-only", "-S", "-o",
            os.path.join(out_dir, src.replace(".hip", ".s")),
            os.path.join(CSRC, src)]
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
