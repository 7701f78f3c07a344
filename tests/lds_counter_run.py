"""Launch, once each, the default kernel of every workload and the LDS-layout
ablation of the headline and fp16 workloads, for a rocprofv3 counter pass
(tests/test_gpu_lds_counters.py runs this file under
``rocprofv3 --pmc SQ_LDS_BANK_CONFLICT ...``).

Prints one line per launch, in launch order: ``launch <tag> <kernel kind>``.
Each call enqueues exactly one kernel (checked with xpose_plan), so the
n-th transpose dispatch in the counter file belongs to the n-th line.
Values are not initialised: bank conflicts depend on addresses only.
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

# (tag, workload key, layout) -- layout 0 is the library default.
LAUNCHES = [
    ("c1 default", "c1_index_1024_f32", 0),
    ("c2 default", "c2_8192_f32", 0),
    ("c3 default", "c3_ragged_12345x6789_f32", 0),
    ("c4 default", "c4_16384_f16", 0),
    ("c5 default", "c5_batched_64x2048x1024_f32", 0),
    ("c2 unpadded", "c2_8192_f32", 1),
    ("c2 pad1", "c2_8192_f32", 2),
    ("c2 swizzle", "c2_8192_f32", 3),
    ("c4 unpadded", "c4_16384_f16", 1),
    ("c4 pad1", "c4_16384_f16", 2),
]


def main() -> int:
    import torch

    import lds_tiled_matrix_amd as X
    dev = torch.device("cuda", 0)
    torch_dtype = {"f32": torch.float32, "f16": torch.float16}
    for tag, key, layout in LAUNCHES:
        w = wl.WORKLOADS[key]
        x = torch.empty(w.in_shape, dtype=torch_dtype[w.dtype], device=dev)
        y = torch.empty((w.batch, w.cols, w.rows) if w.batch > 1
                        else (w.cols, w.rows), dtype=x.dtype, device=dev)
        code = X.dtype_code(x.dtype)
        opts = X.make_opts(layout) if layout else None
        args = (y.data_ptr(), x.data_ptr(), w.batch, w.rows, w.cols, w.cols,
                w.rows, w.rows * w.cols, w.cols * w.rows, code)
        rc, info = X.xpose_plan(*args, opts)
        if rc or info.launches != 1 or info.packed:
            raise RuntimeError(f"{tag}: expected one tile-kernel launch "
                               f"({X.strerror(rc)}, {info.launches})")
        kind = ("shift" if info.aligned_out else "tr" if info.tr_read
                else "tile")
        print(f"launch {tag} {kind} {info.tile_rows}x{info.tile_cols} "
              f"layout={info.layout}", flush=True)
        rc = X.xpose_batched_ex(*args, opts, 0)
        if rc:
            raise RuntimeError(f"{tag}: {X.strerror(rc)}")
        torch.cuda.synchronize()
        del x, y
    return 0


if __name__ == "__main__":
    sys.exit(main())
