"""LDS bank microbenchmark driver for gfx950.

    python -m lds_tiled_matrix_amd.ldsprobe [--transposes] [--iters N]

Runs xpose_lds_probe over a fixed list of lane -> address patterns, each as
a read and as a write, and prints the issue cost in shader cycles per
64-lane instruction.  With --transposes it then runs the 8192 x 8192 fp32
and 16384 x 16384 fp16 transposes once per LDS layout, so that one
rocprofv3 counter pass (SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE) covers both
the probe patterns and the real kernels, in the order printed.

Why: conflicts are resolved per group of lanes whose size on 64-lane
hardware has to be measured ("Shared Memory and Bank Conflicts", section
"the wave size complication"), and the pages' 32-bank arithmetic is for
32-lane hardware.  The patterns below separate the candidate models: which
bank count, which lane group per access width.
"""
from __future__ import annotations

import argparse
import sys

LANES = range(64)


def _split_lane(l: int):
    """The store-phase lane map of the 64 x 64 fp32 tile kernel: a half-wave
    covers 8 row groups (q) of 4 columns (c)."""
    h, m = l >> 5, l & 31
    return (m & 7) + 8 * h, m >> 3


def transpose_gather(layout: str):
    """Byte addresses one column-gather instruction of the 64 x 64 fp32 tile
    kernel touches (first of the four words each lane gathers)."""
    out = []
    for l in LANES:
        q, c = _split_lane(l)
        p = 4 * q
        if layout == "swizzle":
            w = p * 64 + (((c // 4) ^ (q & 15)) * 4) + c % 4
        elif layout == "pad1":
            w = p * 65 + c
        else:
            w = p * 64 + c
        out.append(4 * w)
    return out


# (name, access width in bytes, byte address of each of the 64 lanes)
PATTERNS = [
    ("b32 linear", 4, [4 * l for l in LANES]),
    ("b32 broadcast", 4, [0] * 64),
    ("b32 stride 2 words", 4, [8 * l for l in LANES]),
    ("b32 halves 64 words apart", 4, [4 * ((l % 32) + (l // 32) * 64) for l in LANES]),
    ("b32 column, stride 32 words", 4, [(128 * l) % 16384 for l in LANES]),
    ("b32 column, stride 33 words", 4, [132 * l for l in LANES]),
    ("b32 column, stride 64 words", 4, [(256 * l) % 16384 for l in LANES]),
    ("b32 column, stride 65 words", 4, [260 * l for l in LANES]),
    ("b64 linear", 8, [8 * l for l in LANES]),
    ("b64 16-lane groups 256 B apart", 8, [8 * (l % 16) + 256 * (l // 16) for l in LANES]),
    ("b64 stride 256 B", 8, [(256 * l) % 16384 for l in LANES]),
    ("b128 linear", 16, [16 * l for l in LANES]),
    ("b128 8-lane groups 256 B apart", 16, [16 * (l % 8) + 256 * (l // 8) for l in LANES]),
    ("b128 stride 256 B", 16, [(256 * l) % 16384 for l in LANES]),
    ("transpose gather, unpadded", 4, transpose_gather("unpadded")),
    ("transpose gather, pad1", 4, transpose_gather("pad1")),
    ("transpose gather, swizzle", 4, transpose_gather("swizzle")),
]


def measure(X, torch, buf, width, lanes, is_write, iters):
    """Cycles per instruction for one pattern (one wavefront, 8 instructions
    per iteration, no waits between them)."""
    rc = X.xpose_lds_probe(buf.data_ptr(), lanes, width, is_write, iters, 0)
    if rc:
        raise RuntimeError(X.strerror(rc))
    torch.cuda.synchronize()
    return float(buf[0].item()) / (iters * 8)


def run_patterns(iters=1000, out=sys.stdout):
    import torch
    import lds_tiled_matrix_amd as X
    buf = torch.zeros(2, dtype=torch.int64, device="cuda")
    results = []
    for name, width, lanes in PATTERNS:
        for is_write in (0, 1):
            cyc = measure(X, torch, buf, width, lanes, is_write, iters)
            results.append((name, width, is_write, cyc))
            print(f"probe  {name:34s} {'write' if is_write else 'read '}  "
                  f"{cyc:7.2f} cycles/instr", file=out, flush=True)
    return results


def run_transposes(out=sys.stdout):
    """Each LDS layout once on the 8192 x 8192 fp32 and 16384 x 16384 fp16
    transposes, with the default tile shape and with a 64 x 64 tile (for
    fp16 also read back with LDS transpose reads), and the default on the
    odd-pitch 12345 x 6789 fp32 transpose."""
    import torch
    import lds_tiled_matrix_amd as X
    for rows, cols, dt in ((8192, 8192, torch.float32),
                           (16384, 16384, torch.int16)):
        x = torch.zeros((rows, cols), dtype=dt, device="cuda")
        for tile in (None, (64, 64)):
            for layout in (X.LAYOUT_UNPADDED, X.LAYOUT_PAD1, X.LAYOUT_SWIZZLE):
                plan = X.plan_for(x, layout=layout, tile=tile)
                X.transpose(x, layout=layout, tile=tile)
                torch.cuda.synchronize()
                print(f"xpose  {rows}x{cols} {str(dt).split('.')[-1]} tile "
                      f"{plan['tile_rows']}x{plan['tile_cols']} "
                      f"{X.LAYOUT_NAMES[layout]}", file=out, flush=True)
            if dt == torch.int16:
                # the swizzled tile read back with LDS transpose reads
                plan = X.plan_for(x, tile=tile, flags=X.FLAG_TR_READ)
                X.transpose(x, tile=tile, flags=X.FLAG_TR_READ)
                torch.cuda.synchronize()
                print(f"xpose  {rows}x{cols} {str(dt).split('.')[-1]} tile "
                      f"{plan['tile_rows']}x{plan['tile_cols']} swizzle, "
                      f"transpose reads", file=out, flush=True)
        del x
    # Odd pitches: the default there is the line-aligned output tile, whose
    # column gathers start at a different row offset for every column.
    x = torch.zeros((12345, 6789), dtype=torch.float32, device="cuda")
    plan = X.plan_for(x)
    X.transpose(x)
    torch.cuda.synchronize()
    print(f"xpose  12345x6789 float32 tile {plan['tile_rows']}x"
          f"{plan['tile_cols']} swizzle, line-aligned output "
          f"({plan['aligned_out']})", file=out, flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--iters", type=int, default=1000)
    ap.add_argument("--transposes", action="store_true")
    args = ap.parse_args(argv)
    run_patterns(args.iters)
    if args.transposes:
        run_transposes()
    return 0


if __name__ == "__main__":
    sys.exit(main())
