"""The transpose edge path moves the partial 16-byte vectors of 1- and
2-byte elements in pieces of 8, 4, 2 and 1 bytes (load_head and store_head
in xpose_lanes.h), and edge tiles load every chunk with one 16-byte access
from an address picked without a branch (edge_chunk_src, edge_chunk_fix);
host programs built from the same header check, against a no-access guard
page, that every length and alignment reads and writes exactly its bytes
and that every chunk load stays in its row and yields the chunk."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def _run(name):
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, name)
        subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17",
                        "--offload-arch=gfx950", "-o", exe,
                        os.path.join(HERE, "native", name + ".cpp")],
                       check=True, capture_output=True, timeout=300)
        out = subprocess.run([exe], capture_output=True, text=True,
                             timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout)


def test_partial_vector_pieces_touch_exactly_their_bytes():
    _run("edge_pieces")


def test_edge_chunk_loads_stay_in_the_row():
    _run("edge_chunks")
