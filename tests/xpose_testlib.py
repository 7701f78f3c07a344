"""Shared helpers for the GPU tests: run one transpose through the C ABI on
raw byte buffers with sentinel guard bands, and compute what the oracle says
the same buffer must hold afterwards."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads as wl

DTYPE_OF_SIZE = {4: 0, 2: 1, 1: 3, 8: 4}   # xpose_dtype by element size
GUARD = 256                                  # guard elements on each side


def say(*a):
    """Name the case before a GPU step, flushed, so a fault can be placed."""
    print(*a, flush=True)
    sys.stdout.flush()


def sentinel_for(s: int):
    return wl.RAW_UINT[s](0xA5C3A5C3A5C3A5C3 & ((1 << (8 * s)) - 1))


def layout_sizes(batch, rows, cols, ld_in, ld_out, stride_in, stride_out):
    if batch <= 1:
        stride_in, stride_out = rows * ld_in, cols * ld_out
    n_in = (batch - 1) * stride_in + rows * ld_in if batch else 0
    n_out = (batch - 1) * stride_out + cols * ld_out if batch else 0
    return n_in, n_out, stride_in, stride_out


def expected_output(src_flat, s, batch, rows, cols, ld_in, ld_out, stride_in,
                    stride_out, n_out):
    """The whole output buffer (with guards) the oracle says must result."""
    t = wl.RAW_UINT[s]
    exp = np.full(GUARD + n_out + GUARD, sentinel_for(s), dtype=t)
    body = exp[GUARD:GUARD + n_out]
    oracle.transpose_into(body, src_flat, batch, rows, cols, ld_in, ld_out,
                          stride_in, stride_out)
    return exp


def gpu_transpose(src_flat, s, batch, rows, cols, ld_in, ld_out, stride_in,
                  stride_out, n_out, opts=None, in_shift=0, out_shift=0,
                  stream=None, entry="batched"):
    """Run the library on ``src_flat`` (raw uint array) and return the whole
    output buffer including GUARD sentinel elements on each side.

    in_shift / out_shift move the base pointers by that many elements past an
    allocation boundary (to exercise unaligned rows)."""
    import torch
    import lds_tiled_matrix_amd as X
    dev = torch.device("cuda", 0)
    t = wl.RAW_UINT[s]
    in_bytes = (in_shift + src_flat.size) * s
    d_in = torch.empty(max(in_bytes, 1), dtype=torch.uint8, device=dev)
    if src_flat.size:
        d_in[in_shift * s:].copy_(torch.from_numpy(src_flat.view(np.uint8)))
    host_out = np.full(GUARD + n_out + GUARD, sentinel_for(s), dtype=t)
    d_out = torch.empty(out_shift * s + host_out.nbytes, dtype=torch.uint8,
                        device=dev)
    d_out[out_shift * s:].copy_(torch.from_numpy(host_out.view(np.uint8)))
    pin = d_in.data_ptr() + in_shift * s
    pout = d_out.data_ptr() + (out_shift + GUARD) * s
    sh = 0 if stream is None else int(stream.cuda_stream)
    if entry == "2d":
        assert batch == 1
        rc = X.xpose_2d(pout, pin, rows, cols, ld_in, ld_out,
                        DTYPE_OF_SIZE[s], sh)
    elif entry == "2d_ex":
        assert batch == 1
        rc = X.xpose_2d_ex(pout, pin, rows, cols, ld_in, ld_out,
                           DTYPE_OF_SIZE[s], opts, sh)
    elif opts is None:
        rc = X.xpose_batched(pout, pin, batch, rows, cols, ld_in, ld_out,
                             stride_in, stride_out, DTYPE_OF_SIZE[s], sh)
    else:
        rc = X.xpose_batched_ex(pout, pin, batch, rows, cols, ld_in, ld_out,
                                stride_in, stride_out, DTYPE_OF_SIZE[s], opts,
                                sh)
    assert rc == 0, X.strerror(rc)
    torch.cuda.synchronize()
    got = d_out[out_shift * s:].cpu().numpy().view(t)
    return got


def check_case(s, batch, rows, cols, ld_in=None, ld_out=None, stride_in=None,
               stride_out=None, seed=0, src=None, opts=None, in_shift=0,
               out_shift=0, label="", entry="batched"):
    """Random-bit (or given) input through the library vs the oracle, whole
    output buffer compared bit for bit, guards and padding included."""
    ld_in = cols if ld_in is None else ld_in
    ld_out = rows if ld_out is None else ld_out
    n_in, n_out, st_in, st_out = layout_sizes(
        batch, rows, cols, ld_in, ld_out,
        rows * ld_in if stride_in is None else stride_in,
        cols * ld_out if stride_out is None else stride_out)
    if src is None:
        src = wl.random_bits((max(n_in, 0),), s, seed)
    say(f"case {label} s={s} b={batch} {rows}x{cols} ld={ld_in}/{ld_out} "
        f"st={st_in}/{st_out} shift={in_shift}/{out_shift} seed={seed}")
    got = gpu_transpose(src, s, batch, rows, cols, ld_in, ld_out, st_in,
                        st_out, n_out, opts, in_shift, out_shift, entry=entry)
    exp = expected_output(src, s, batch, rows, cols, ld_in, ld_out, st_in,
                          st_out, n_out)
    if not np.array_equal(got, exp):
        bad = np.flatnonzero(got != exp)
        raise AssertionError(
            f"{label}: {bad.size} elements differ; first at buffer index "
            f"{bad[0]} (guard={GUARD}): got {got[bad[0]]:#x} want {exp[bad[0]]:#x}")
