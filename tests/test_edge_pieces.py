"""The transpose edge path moves the partial 16-byte vectors of 1- and
2-byte elements in pieces of 8, 4, 2 and 1 bytes (load_head and store_head
in xpose_lanes.h); a host program built from the same header checks,
against a no-access guard page, that every length and alignment reads and
writes exactly its bytes."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_partial_vector_pieces_touch_exactly_their_bytes():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "edge_pieces")
        subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17",
                        "--offload-arch=gfx950", "-o", exe,
                        os.path.join(HERE, "native", "edge_pieces.cpp")],
                       check=True, capture_output=True, timeout=300)
        out = subprocess.run([exe], capture_output=True, text=True,
                             timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout)
