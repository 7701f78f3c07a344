"""Throughput of the LDS-tiled transpose on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload KEY] [--table]

One step is one transpose of the whole workload (default: 8192 x 8192 fp32,
row-major, ld = cols) with the input already resident in HBM.  Prints ONE
JSON line: effective GB/s = (read + write bytes) / time, with the copy
yardstick, the LDS-layout ablation, the kernel's roofline fraction measured
live with HIP events on the launch stream, and the oracle timed on one host
core.  The line also carries, under "sgemm", the tiled SGEMM whose
transposed LDS store is the pages' second bank-conflict workload (4096^3
fp32, TFLOP/s against the matrix-core peak, its As-layout ablation);
--sgemm-only measures just that.  --table additionally writes a markdown
table over every workload to stderr.

Timing protocol ("Shared memory and the bank conflict", section "What to
record": warm the kernel up first, time it many times, report the median,
and time the copy with the same procedure): W untimed launches, then K
launches back to back bracketed by device synchronisation (the wall-clock
`value`) and by one event pair on the launch stream (the average launch
duration behind `roofline`), then K launches each between an event pair on
the launch stream (median / min / p90 / mean per launch).  A cold mode reads
1 GiB between launches to empty every cache first (`roofline_cold`: the
bytes then come from HBM).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

METRIC = ("effective GB/s (R+W bytes) and % of HBM peak, 8192x8192 fp32 "
          "transpose, 1 GPU")
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "lds_tiled_matrix_amd", "csrc", f)
                  for f in ("xpose_kernels.hip", "xpose_kernels.h", "xpose_lanes.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c2_8192_f32.md")
SIGNED = {1: np.int8, 2: np.int16, 4: np.int32, 8: np.int64}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the device code (kernels and the tile-order header)."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def plan_signature(config: dict) -> str:
    """The launch a bench line's config describes: layout, tile, workgroup
    size, cache policy, tile order, workgroups per compute unit and grid."""
    return (f"{config['layout']} {config['tile']} t{config['threads']} "
            f"{config['cache']} {config['tile_order']} occupancy "
            f"{config['occupancy']} workgroups {config['workgroups']}")


def read_traffic(config: dict | None = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source and, given the bench
    line's config, on the launch that config describes (else None): the
    default's rules live outside the kernel source, so the hash alone does
    not pin the kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln and ln.startswith("- "):
                k, v = ln[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if config is not None and fields.get("plan") != plan_signature(config):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_launches(launch, stream, steps, warmup):
    """W untimed launches; then K launches back to back bracketed by device
    synchronisation and by one event pair on the launch stream (the
    wall-clock time and the timed region's GPU time, nothing else in the
    loop); then K more launches each between an event pair on the launch
    stream (the per-launch durations).  Returns (wall_s, region_s,
    durations_s): region_s / K is the average launch duration, the figure a
    kernel trace's average duration reports."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for _ in range(steps):
        launch()
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = r0.elapsed_time(r1) * 1e-3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        starts[k].record(stream)
        launch()
        ends[k].record(stream)
    torch.cuda.synchronize()
    durs = [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]
    return wall, region, durs


def summarize(durs, nbytes):
    d = sorted(durs)
    med = statistics.median(d)
    p90 = d[min(len(d) - 1, int(0.9 * len(d)))]
    mean = sum(d) / len(d)
    return {"median_us": round(med * 1e6, 2), "min_us": round(d[0] * 1e6, 2),
            "p90_us": round(p90 * 1e6, 2), "mean_us": round(mean * 1e6, 2),
            "median_GBps": round(nbytes / med / 1e9, 1),
            "mean_GBps": round(nbytes / mean / 1e9, 1)}


def cpu_baseline(w, host_in, max_seconds=12.0, max_runs=6):
    """The oracle as it stands, pinned to one host core, on the full
    workload: 1 warm-up, then repeated runs until max_seconds or max_runs;
    median effective GB/s."""
    import oracle
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        oracle.transpose(host_in)  # warm-up (also faults the pages in)
        times = []
        t_start = time.perf_counter()
        while len(times) < max_runs and (time.perf_counter() - t_start) < max_seconds:
            t0 = time.perf_counter()
            out = oracle.transpose(host_in)
            times.append(time.perf_counter() - t0)
    finally:
        os.sched_setaffinity(0, old)
    med = statistics.median(times)
    return out, {
        "value": round(w.rw_bytes / med / 1e9, 3), "unit": "GB/s", "cores": 1,
        "kind": "oracle",
        "sample": (f"full {w.description}; single-threaded C nested loop "
                   f"pinned to core {core}; 1 warm-up + {len(times)} timed "
                   f"runs, median {med * 1e3:.1f} ms"),
    }


def system_info() -> dict:
    """Device, toolchain and host the numbers were measured on."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "hip": torch.version.hip,
            "torch": torch.__version__, "host_cpu": host_cpu_name(),
            "host_cores": len(os.sched_getaffinity(0))}


def host_cpu_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Copy kernels measured for the yardstick: (threads, 16-byte vectors per
# lane, cache policy).  The fastest one is the practical roofline.
COPY_VARIANTS = ((256, 1, 2), (512, 1, 2), (256, 2, 2), (1024, 1, 2),
                 (256, 4, 2), (256, 4, 1))
FLUSH_BYTES = 1 << 30   # > the 256 MB Infinity Cache


def time_cold(launch, stream, reps, flush):
    """Per-launch event times with the caches flushed before every launch:
    1 GiB is READ between launches, outside the events, so every cache holds
    clean lines of another buffer (a written flush would leave dirty lines
    whose write-back the timed kernel would pay for)."""
    import torch
    durs = []
    flat = flush.view(torch.int64)
    for k in range(reps):
        flat.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        b.synchronize()
        durs.append(a.elapsed_time(b) * 1e-3)
    return durs


def bench_workload(X, w, steps, warmup, stream, layouts=True, cold=True):
    """Time the default launch (and each layout) on one workload plus the
    copy yardstick over the same bytes.  Returns a dict, the host input and
    the device output of the default launch."""
    import torch
    dev = torch.device("cuda", 0)
    host = wl.make_input(w)
    if host.dtype.kind == "u" and host.dtype.itemsize > 1:
        host = host.view(SIGNED[host.dtype.itemsize])
    x = torch.from_numpy(host).to(dev)
    out_shape = (w.cols, w.rows) if w.batch == 1 else (w.batch, w.cols, w.rows)
    y = torch.empty(out_shape, dtype=x.dtype, device=dev)
    code = X.dtype_code(x.dtype)
    sh = int(stream.cuda_stream)
    nbytes = w.rw_bytes

    def launch_with(opts):
        def go():
            rc = X.xpose_batched_ex(y.data_ptr(), x.data_ptr(), w.batch,
                                    w.rows, w.cols, w.cols, w.rows,
                                    w.rows * w.cols, w.cols * w.rows, code,
                                    opts, sh)
            if rc:
                raise RuntimeError(X.strerror(rc))
        return go

    def copy_with(opts):
        # Same byte count, same buffers (input -> output).
        def go():
            rc = X.xpose_copy_ex(y.data_ptr(), x.data_ptr(), nbytes // 2, opts,
                                 sh)
            if rc:
                raise RuntimeError(X.strerror(rc))
        return go

    res = {}
    n_small = max(10, min(steps, 50))
    with torch.cuda.stream(stream):
        copies = {}
        for thr, unroll, cache in COPY_VARIANTS:
            o = X.XposeCopyOpts(thr, unroll, cache, 0)
            _, _, d = time_launches(copy_with(o), stream, n_small, warmup)
            copies[f"{thr}x{unroll} {X.CACHE_NAMES[cache]}"] = summarize(d, nbytes)
        best = max(copies, key=lambda k: copies[k]["median_GBps"])
        res["copy_variants_GBps"] = {k: v["median_GBps"] for k, v in copies.items()}
        res["copy"] = dict(copies[best], kernel=best)
        best_opts = X.XposeCopyOpts(*[int(t) for t in best.split()[0].split("x")],
                                    X.CACHE_NT_STORE if "nt_store" in best
                                    else X.CACHE_DEFAULT, 0)
        yb, xb = y.view(-1), x.view(-1)
        _, _, durs_m = time_launches(lambda: yb.copy_(xb), stream, n_small,
                                     warmup)
        res["memcpy_d2d"] = summarize(durs_m, nbytes)
        if layouts:
            # The pages' record set: the copy, the tile with and without the
            # pad (and the swizzle), and the better of the two naive kernels.
            res["ablation"] = {}
            for lay, name in list(X.LAYOUT_NAMES.items()) + list(X.NAIVE_NAMES.items()):
                _, _, d = time_launches(launch_with(X.XposeOpts(lay, 0, 0, 0)),
                                     stream, max(10, n_small // 5) if lay > 3
                                     else n_small, min(warmup, 3) if lay > 3
                                     else warmup)
                res["ablation"][name] = summarize(d, nbytes)
            if w.elem_bytes in (1, 2):
                # The same swizzled tile read back with LDS transpose reads.
                _, _, d = time_launches(
                    launch_with(X.make_opts(flags=X.FLAG_TR_READ)), stream,
                    n_small, warmup)
                res["ablation"]["swizzle_tr_read"] = summarize(d, nbytes)
        if cold:
            flush = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)
            reps = max(5, min(steps, 20))
            res["cold"] = {
                "transpose": summarize(time_cold(launch_with(None), stream,
                                                 reps, flush), nbytes),
                "copy": summarize(time_cold(copy_with(best_opts), stream,
                                            reps, flush), nbytes),
                "note": "1 GiB read between launches, outside the timing",
            }
            del flush
        # The default launch last, so its output stays in y.
        wall, region, durs = time_launches(launch_with(None), stream, steps,
                                           warmup)
    torch.cuda.synchronize()
    res["wall_s"] = wall
    res["region_s"] = region
    res["default"] = summarize(durs, nbytes)
    res["default"]["region_avg_us"] = round(region / steps * 1e6, 2)
    res["plan"] = X.plan_for(x, y)
    return res, host, y


def cold_roofline(cold):
    """The cache-cold transpose against the HBM peak and against the copy
    timed the same way (median per launch)."""
    if not cold:
        return None
    t, c = cold["transpose"]["median_GBps"], cold["copy"]["median_GBps"]
    return {"bound": "hbm", "achieved": t, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(t / HBM_PEAK_GBS, 4),
            "copy": c, "frac_of_copy": round(t / c, 4),
            "statistic": "median of per-launch events, 1 GiB read before "
                         "each launch"}


FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix-core peak


def bench_sgemm(X, steps, warmup, stream, with_cpu=True):
    """The tiled SGEMM with the transposed As store at the size its page
    measures (M = N = K = 4096, C += A B, uniform [-1, 1) inputs): the
    library's default kernel for that shape with its matrix-core roofline,
    the As-layout ablation (unpadded, padded, swizzle) with one and two LDS
    buffers and with 256-row blocks, torch's fp32 addmm for context,
    sampled parity against the oracle, and the oracle timed on a bounded
    sample."""
    import torch
    w = wl.GEMM_WORKLOADS["sgemm_4096"]
    A, B, C = wl.make_gemm_inputs(w)
    dev = torch.device("cuda", 0)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C).to(dev)
    sh = int(stream.cuda_stream)

    def launch_with(opts):
        def go():
            rc = X.xpose_sgemm_ex(w.m, w.n, w.k, w.alpha, dA.data_ptr(), w.k,
                                  dB.data_ptr(), w.n, w.beta, dC.data_ptr(),
                                  w.n, opts, sh)
            if rc:
                raise RuntimeError(X.strerror(rc))
        return go

    def tflops(durs):
        d = sorted(durs)
        med, mean = statistics.median(d), sum(d) / len(d)
        return {"median_us": round(med * 1e6, 1), "min_us": round(d[0] * 1e6, 1),
                "mean_us": round(mean * 1e6, 1),
                "median_TFLOPs": round(w.flops / med / 1e12, 2),
                "mean_TFLOPs": round(w.flops / mean / 1e12, 2)}

    res = {"workload": w.description, "m": w.m, "n": w.n, "k": w.k,
           "alpha": w.alpha, "beta": w.beta, "flops": w.flops}
    if with_cpu:
        # The CPU leg: the oracle on a bounded sample (64 rows of C), timed,
        # and the GPU's rows from one launch on the original C checked
        # against it.
        import oracle.sgemm as og
        with torch.cuda.stream(stream):
            launch_with(None)()
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        rows = np.random.default_rng(7).choice(w.m, 64, replace=False)
        t0 = time.perf_counter()
        ref = og.sgemm(len(rows), w.n, w.k, w.alpha,
                       np.ascontiguousarray(A[rows]).reshape(-1), w.k,
                       B.reshape(-1), w.n, w.beta,
                       np.ascontiguousarray(C[rows]).reshape(-1), w.n)
        t_ref = time.perf_counter() - t0
        mag = abs(w.alpha) * (np.abs(A[rows].astype(np.float64)) @
                              np.abs(B.astype(np.float64)))
        mag += abs(w.beta) * np.abs(C[rows].astype(np.float64))
        err = np.abs(got[rows].astype(np.float64) - ref)
        res["parity_vs_oracle"] = bool(
            (err <= (w.k + 3) * 2.0 ** -24 * mag).all())
        res["parity_sample"] = ("64 sampled rows of C (all columns) against "
                                "the oracle, within (k + 3) 2^-24 "
                                "(|alpha||A||B| + |beta||C|)")
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = 1
        res["cpu_baseline"] = {
            "value": round(2 * len(rows) * w.n * w.k / t_ref / 1e9, 2),
            "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"{len(rows)} rows of C (float64 numpy matmul, "
                       f"{threads} BLAS threads), {t_ref * 1e3:.0f} ms")}
    with torch.cuda.stream(stream):
        ab = {}
        n_ab = max(10, min(steps, 40))
        for lay, name in X.AS_NAMES.items():
            for flags, tile_m, tag in ((0, 0, ""),
                                       (X.SGEMM_DOUBLE_BUFFER, 0, " 2 buffers"),
                                       (0, 256, " 256-row blocks")):
                opts = X.make_sgemm_opts(lay, 0, 0, flags, tile_m)
                _, _, d = time_launches(launch_with(opts), stream, n_ab,
                                     min(warmup, 5))
                ab[name + tag] = tflops(d)["median_TFLOPs"]
        res["ablation_TFLOPs"] = ab
        c2 = torch.empty_like(dC)
        _, _, d = time_launches(lambda: torch.addmm(dC, dA, dB, out=c2),
                                stream, n_ab, min(warmup, 5))
        res["torch_addmm_fp32_TFLOPs"] = tflops(d)["median_TFLOPs"]
        del c2
        n_t = max(10, min(steps, 100))
        _, region, durs = time_launches(launch_with(None), stream, n_t,
                                        min(warmup, 10))
    torch.cuda.synchronize()
    t = tflops(durs)
    rc, info = X.xpose_sgemm_plan(w.m, w.n, w.k, dA.data_ptr(), w.k,
                                  dB.data_ptr(), w.n, dC.data_ptr(), w.n)
    res["kernel"] = {"layout": X.AS_NAMES[info.layout], "bk": info.bk,
                     "as_stride": info.as_stride, "stages": info.stages,
                     "lds_bytes": info.lds_bytes, "workgroups": info.tiles,
                     "tile": f"{info.tile_m}x{info.tile_n}"}
    # The roofline uses the average launch duration over the back-to-back
    # timed region (one event pair on the launch stream), the statistic a
    # kernel trace's average duration reports.
    t["region_avg_us"] = round(region / n_t * 1e6, 1)
    res["timing"] = t
    achieved = round(w.flops / (region / n_t) / 1e12, 2)
    res["roofline"] = {"bound": "mfma", "achieved": achieved,
                       "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
                       "traffic": None}
    return res


SGEMM_SHAPES = ((1024, 1024, 1024), (1536, 1536, 1536), (2048, 2048, 2048),
                (3000, 3000, 3000), (4100, 4100, 4100), (5000, 5000, 5000),
                (1024, 1024, 8192))


def bench_sgemm_shapes(X, shapes, steps, warmup, stream):
    """The SGEMM off the page's size, where the grid of 128 x 128 blocks
    is too small to fill 256 compute units: per shape, the library's
    default with a workspace (xpose_sgemm_ws: its split of k, product and
    sum kernels, timed together), the same without a workspace (no split),
    and torch's fp32 addmm; C += A B on uniform [-1, 1) inputs, medians of
    per-call events."""
    import torch
    dev = torch.device("cuda", 0)
    sh = int(stream.cuda_stream)
    out = []
    n = max(10, min(steps, 50))
    for idx, (m, nn, k) in enumerate(shapes):
        g = torch.Generator(device="cpu").manual_seed(100 + idx)
        dA = (torch.rand(m, k, generator=g) * 2 - 1).to(dev)
        dB = (torch.rand(k, nn, generator=g) * 2 - 1).to(dev)
        dC = (torch.rand(m, nn, generator=g) * 2 - 1).to(dev)
        args = (m, nn, k, dA.data_ptr(), k, dB.data_ptr(), nn, dC.data_ptr(),
                nn)
        rc, info = X.xpose_sgemm_plan_ws(*args, None, 0, 0)
        if rc:
            raise RuntimeError(X.strerror(rc))
        ws = torch.empty(max(info.workspace_wanted // 4, 1),
                         dtype=torch.float32, device=dev)
        rc, info = X.xpose_sgemm_plan_ws(*args, None, ws.data_ptr(),
                                         info.workspace_wanted)

        def split_call():
            rc = X.xpose_sgemm_ws(m, nn, k, 1.0, dA.data_ptr(), k,
                                  dB.data_ptr(), nn, 1.0, dC.data_ptr(), nn,
                                  None, ws.data_ptr(), info.workspace_wanted,
                                  sh)
            if rc:
                raise RuntimeError(X.strerror(rc))

        def plain_call():
            rc = X.xpose_sgemm_ex(m, nn, k, 1.0, dA.data_ptr(), k,
                                  dB.data_ptr(), nn, 1.0, dC.data_ptr(), nn,
                                  None, sh)
            if rc:
                raise RuntimeError(X.strerror(rc))

        c2 = torch.empty_like(dC)
        flops = 2 * m * nn * k
        row = {"m": m, "n": nn, "k": k, "splits": info.splits,
               "split_len": info.split_len,
               "workspace_MiB": round(info.workspace_bytes / 2 ** 20, 1),
               "workgroups": info.tiles}
        variants = (("split", split_call), ("no_split", plain_call),
                    ("torch_addmm", lambda: torch.addmm(dC, dA, dB, out=c2)))
        with torch.cuda.stream(stream):
            # one untimed pass over all three first: the first calls after
            # the inputs are made run while clocks and caches settle
            for _, fn in variants:
                time_launches(fn, stream, n, min(warmup, 5))
            for name, fn in variants:
                _, _, d = time_launches(fn, stream, n, min(warmup, 5))
                row[name + "_TFLOPs"] = round(
                    flops / statistics.median(d) / 1e12, 2)
        torch.cuda.synchronize()
        row["split_vs_torch"] = round(row["split_TFLOPs"] /
                                      row["torch_addmm_TFLOPs"], 3)
        out.append(row)
        del dA, dB, dC, c2, ws
    return out


# The library's defaults off the five workloads: (element bytes, rows,
# cols) -- square, wide, tall, odd (line-aligned output) and large shapes of
# every element size.
SWEEP_SHAPES = (
    (4, 2048, 2048), (4, 4096, 4096), (4, 6144, 6144), (4, 8192, 8192),
    (4, 12288, 12288), (4, 16384, 16384), (4, 1024, 8192), (4, 8192, 1024),
    (4, 8192, 4096), (4, 16384, 2048), (4, 16384, 8192), (4, 32768, 8192),
    (4, 12345, 6789), (4, 9999, 9999),
    (2, 4096, 4096), (2, 8192, 8192), (2, 16384, 16384), (2, 32768, 16384),
    (2, 12345, 6789), (2, 16383, 16383),
    (1, 8192, 8192), (1, 16384, 16384), (1, 12345, 6789),
    (8, 4096, 4096), (8, 6000, 6000), (8, 8192, 8192), (8, 16384, 8192),
    (8, 8191, 8191))


def bench_sweep(X, stream, shapes=SWEEP_SHAPES, steps=20, cold_reps=4):
    """The default launch on each (element bytes, rows, cols) matrix of
    ``shapes``, filled with seeded random bytes, against the library's
    default copy over the same bytes, back to back (average over the region
    of ``steps`` launches) and with the caches flushed before each launch
    (median of ``cold_reps``).  Returns a list of rows.

    The bytes must be random: the kernels never look at them, but on MI355X
    back-to-back launches over zero-filled buffers (what a fresh, untouched
    allocation holds) run about 17% faster than over random data, the copy
    as much as the transpose, while cache-cold launches do not change."""
    import torch
    dev = torch.device("cuda", 0)
    sh = int(stream.cuda_stream)
    flush = torch.empty(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
    flush.zero_()
    rows = []
    for s, r, c in shapes:
        nbytes = r * c * s
        x = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.int32,
                        device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(s * 1_000_003 + r * 1009 + c)
        x.view(torch.uint8).random_(0, 256, generator=gen)
        y = torch.empty_like(x)
        y.view(torch.uint8).random_(0, 256, generator=gen)
        dt = {1: X.XPOSE_U8, 2: X.XPOSE_F16, 4: X.XPOSE_F32, 8: X.XPOSE_F64}[s]
        rc, info = X.xpose_plan(y.data_ptr(), x.data_ptr(), 1, r, c, c, r, 0,
                                0, dt, None)
        if rc:
            raise RuntimeError(X.strerror(rc))

        def tr():
            rc = X.xpose_2d(y.data_ptr(), x.data_ptr(), r, c, c, r, dt, sh)
            if rc:
                raise RuntimeError(X.strerror(rc))

        def cp():
            rc = X.xpose_copy(y.data_ptr(), x.data_ptr(), nbytes, sh)
            if rc:
                raise RuntimeError(X.strerror(rc))

        res = {}
        with torch.cuda.stream(stream):
            for name, fn in (("transpose", tr), ("copy", cp)):
                _, region, _ = time_launches(fn, stream, steps, 3)
                cold = statistics.median(time_cold(fn, stream, cold_reps, flush))
                res[name] = (2 * nbytes / (region / steps) / 1e9,
                             2 * nbytes / cold / 1e9)
        torch.cuda.synchronize()
        order = {X.ORDER_SUPER_TILES: f"super {info.group_rows}x{info.group_cols}",
                 X.ORDER_DIAGONAL: "diagonal",
                 X.ORDER_COLUMN_BANDS: f"bands {info.group_cols}"}.get(
                     info.order, f"order {info.order}")
        rows.append({
            "elem_bytes": s, "rows": r, "cols": c, "rw_bytes": 2 * nbytes,
            "kernel": f"{info.tile_rows}x{info.tile_cols}"
                      + (" line-aligned" if info.aligned_out else "")
                      + f", {order}" + (f", {info.occupancy}/CU" if info.occupancy else ""),
            "hot_GBps": round(res["transpose"][0], 1),
            "hot_of_copy": round(res["transpose"][0] / res["copy"][0], 3),
            "cold_GBps": round(res["transpose"][1], 1),
            "cold_of_copy": round(res["transpose"][1] / res["copy"][1], 3)})
        log(f"sweep: s{s} {r}x{c} {rows[-1]['kernel']}: "
            f"{rows[-1]['hot_GBps']:.0f} ({rows[-1]['hot_of_copy']:.3f}) / "
            f"{rows[-1]['cold_GBps']:.0f} ({rows[-1]['cold_of_copy']:.3f})")
        del x, y
        torch.cuda.empty_cache()
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=wl.HEADLINE, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle CPU baseline and the parity check")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache (flushed) timing")
    ap.add_argument("--table", action="store_true",
                    help="also measure every workload; markdown table to stderr")
    ap.add_argument("--no-sgemm", action="store_true",
                    help="skip the tiled SGEMM (padded transposed As store)")
    ap.add_argument("--sgemm-only", action="store_true",
                    help="measure only the tiled SGEMM; print its JSON line")
    ap.add_argument("--sweep", action="store_true",
                    help="measure only the library's default over a sweep of "
                         "shapes and element sizes against the copy, hot and "
                         "cold; JSON line on stdout, markdown table on stderr")
    ap.add_argument("--sgemm-shapes", default=None,
                    help="comma-separated MxNxK list for the SGEMM's small-grid "
                         "table (split of k against none and torch); 'none' "
                         "skips it; default: " +
                         ",".join("x".join(map(str, t)) for t in SGEMM_SHAPES))
    args = ap.parse_args(argv)
    if args.sgemm_shapes is None:
        shapes = SGEMM_SHAPES
    elif args.sgemm_shapes == "none":
        shapes = ()
    else:
        try:
            shapes = tuple(tuple(int(v) for v in t.split("x"))
                           for t in args.sgemm_shapes.split(","))
            assert all(len(t) == 3 and min(t) > 0 for t in shapes)
        except (ValueError, AssertionError):
            ap.error("--sgemm-shapes takes MxNxK[,MxNxK...] of positive sizes")

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for "
              f"--gpus {args.gpus}); the transpose has no multi-GPU path.",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import torch
    import lds_tiled_matrix_amd as X
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    stream = torch.cuda.Stream()
    if args.sweep:
        log("bench: default kernels over a shape sweep")
        rows = bench_sweep(X, stream)
        print(json.dumps({"sweep": rows, "system": system_info()}), flush=True)
        print("| element bytes | rows x cols | default kernel | hot GB/s | of copy | "
              "cold GB/s | of copy |", file=sys.stderr)
        print("|---|---|---|---|---|---|---|", file=sys.stderr)
        for r in rows:
            print(f"| {r['elem_bytes']} | {r['rows']} x {r['cols']} | {r['kernel']} | "
                  f"{r['hot_GBps']:,.0f} | {r['hot_of_copy']:.3f} | "
                  f"{r['cold_GBps']:,.0f} | {r['cold_of_copy']:.3f} |",
                  file=sys.stderr)
        return 0
    if args.sgemm_only:
        log("bench: tiled SGEMM only")
        sg = bench_sgemm(X, args.steps, args.warmup, stream,
                         with_cpu=not args.no_cpu)
        if shapes:
            log("bench: SGEMM small grids")
            sg["shapes"] = bench_sgemm_shapes(X, shapes, args.steps,
                                              args.warmup, stream)
        print(json.dumps({"sgemm": sg}), flush=True)
        return 0
    w = wl.WORKLOADS[args.workload]
    log(f"bench: {w.description}; steps={args.steps} warmup={args.warmup}")
    res, host, y = bench_workload(X, w, args.steps, args.warmup, stream,
                                  layouts=not args.no_ablation,
                                  cold=not args.no_cold)
    nbytes = w.rw_bytes
    wall = res["wall_s"]
    value = args.steps * nbytes / wall / 1e9
    d = res["default"]
    # Average launch duration over the back-to-back timed region (one event
    # pair on the launch stream): the statistic a kernel trace's average
    # duration reports, so the two agree.
    achieved = nbytes / (res["region_s"] / args.steps) / 1e9
    copy_gbps = res["copy"]["median_GBps"]

    cpu = None
    parity = None
    if not args.no_cpu:
        log("bench: oracle on one host core (CPU baseline + parity)")
        want, cpu = cpu_baseline(w, host)
        got = y.cpu().numpy()
        parity = bool(np.array_equal(got, want))
        cpu["host_cpu"] = host_cpu_name()
        # threads this process may run on (the machine's CPU share), for context:
        # the oracle itself is pinned to one of them
        cpu["host_threads_available"] = len(os.sched_getaffinity(0))
        if not parity:
            log("bench: PARITY FAILURE against the oracle")

    sgemm = None
    if not args.no_sgemm:
        log("bench: tiled SGEMM")
        del y
        torch.cuda.empty_cache()
        sgemm = bench_sgemm(X, args.steps, args.warmup, stream,
                            with_cpu=not args.no_cpu)
        if shapes:
            log("bench: SGEMM small grids")
            sgemm["shapes"] = bench_sgemm_shapes(X, shapes, args.steps,
                                                 args.warmup, stream)

    plan = res["plan"]
    config = {
        "workload": w.description, "batch": w.batch, "rows": w.rows,
        "cols": w.cols, "ld_in": w.cols, "ld_out": w.rows,
        "rw_bytes": nbytes,
        "layout": X.LAYOUT_NAMES[plan["layout"]],
        "tile": f"{plan['tile_rows']}x{plan['tile_cols']}",
        "threads": plan["threads"], "workgroups": plan["tiles"],
        "cache": X.CACHE_NAMES[plan["cache"]],
        "tile_order": {
            X.ORDER_SUPER_TILES:
                f"super-tiles {plan['group_rows']}x{plan['group_cols']}",
            X.ORDER_DIAGONAL: "diagonal",
            X.ORDER_COLUMN_BANDS: f"column bands {plan['group_cols']}",
        }[plan["order"]]
                      + (", per-XCD ranges" if plan["xcd_remap"] else ""),
        "occupancy": plan["occupancy"],
    }
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": config,
        "system": system_info(),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "frac_of_copy": round(d["median_GBps"] / copy_gbps, 4),
        "timing": d,
        "copy": res["copy"],
        "copy_variants_GBps": res["copy_variants_GBps"],
        "memcpy_d2d": res["memcpy_d2d"],
        "cold": res.get("cold"),
        "ablation": res.get("ablation"),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(config) if w.key == wl.HEADLINE else None,
        },
        # HBM-served figures: every cache (L2 and the 256 MB memory-side
        # cache) is emptied before each launch, so the bytes come from HBM.
        "roofline_cold": cold_roofline(res.get("cold")),
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "sgemm": sgemm,
    }
    print(json.dumps(line), flush=True)

    if args.table:
        rows = []
        for key in sorted(wl.WORKLOADS):
            wk = wl.WORKLOADS[key]
            log(f"bench: table {key}")
            r, _, _ = bench_workload(X, wk, min(args.steps, 100),
                                     min(args.warmup, 10), stream,
                                     layouts=True, cold=True)
            dd = r["default"]
            rows.append((key, wk.rw_bytes, dd, r["copy"], r["ablation"],
                         r["cold"], r["plan"]))
            del r
            torch.cuda.empty_cache()
        log("| workload | kernel | R+W bytes | median us | GB/s | % 8 TB/s | "
            "copy GB/s | % copy | cold GB/s | cold copy GB/s | unpadded | "
            "pad1 | swizzle | swizzle, transpose reads | naive (best) |")
        log("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
        for key, b, dd, cp, ab, cd, pl in rows:
            g = dd["median_GBps"]
            kern = (f"{pl['tile_rows']}x{pl['tile_cols']} "
                    f"{X.CACHE_NAMES[pl['cache']]}")
            log(f"| {key} | {kern} | {b:,} | {dd['median_us']} | {g} | "
                f"{100 * g / HBM_PEAK_GBS:.1f} | {cp['median_GBps']} | "
                f"{100 * g / cp['median_GBps']:.1f} | "
                f"{cd['transpose']['median_GBps']} | {cd['copy']['median_GBps']} | "
                f"{ab['unpadded']['median_GBps']} | {ab['pad1']['median_GBps']} | "
                f"{ab['swizzle']['median_GBps']} | "
                f"{ab['swizzle_tr_read']['median_GBps'] if 'swizzle_tr_read' in ab else '—'} | "
                f"{max(ab['naive_read_coalesced']['median_GBps'], ab['naive_write_coalesced']['median_GBps'])} |")
    return 0 if parity is not False else 3


if __name__ == "__main__":
    sys.exit(main())
