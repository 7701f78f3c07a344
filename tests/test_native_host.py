"""Host-compiled checks of index math the kernels use (CPU only)."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tile_order_is_a_bijection():
    """Every workgroup maps to a tile inside the grid and every tile is hit
    exactly once, for many grid and super-tile shapes, batches, and with and
    without the per-XCD remap (xpose::tile_coords, compiled for the host)."""
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "test_tile_order")
        subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17",
                        "--offload-arch=gfx950", "-o", exe,
                        os.path.join(HERE, "native", "test_tile_order.cpp")],
                       check=True, capture_output=True, timeout=300)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
