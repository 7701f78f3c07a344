"""Python binding of libxpose.so, the LDS-tiled transpose for MI355X.

Every function here marshals arguments and calls the C ABI declared in
``include/xpose.h``; the transpose itself runs only in the library's gfx950
kernels.  The library must have been built (``python lds_tiled_matrix_amd/build.py``);
importing this package without it raises ImportError rather than falling
back to anything else.

Low-level names mirror the C ABI (``xpose_2d``, ``xpose_2d_ex``,
``xpose_batched``,
``xpose_batched_ex``, ``xpose_copy``, ``xpose_plan``, ``xpose_lds_probe``,
and the tiled SGEMM's ``xpose_sgemm``, ``xpose_sgemm_ex``,
``xpose_sgemm_plan``, ``xpose_sgemm_ws``, ``xpose_sgemm_noalloc``,
``xpose_sgemm_plan_ws`` of
``include/xpose_sgemm.h``) and take raw device
addresses as integers.  ``transpose``, ``copy`` and ``sgemm`` are
conveniences over torch tensors: torch supplies the device memory and the
stream, nothing else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libxpose.so")

XPOSE_F32, XPOSE_F16, XPOSE_BF16, XPOSE_U8, XPOSE_F64 = 0, 1, 2, 3, 4
XPOSE_OK = 0
XPOSE_EINVAL, XPOSE_EALIAS, XPOSE_EDTYPE = -1, -2, -3
XPOSE_EHIP, XPOSE_EALIGN, XPOSE_ENOTILE = -4, -5, -6
XPOSE_EWORKSPACE = -7
SGEMM_SCRATCH_BYTES = 64 << 20   # xpose_sgemm_noalloc's device array, per GPU
LAYOUT_AUTO, LAYOUT_UNPADDED, LAYOUT_PAD1, LAYOUT_SWIZZLE = 0, 1, 2, 3
LAYOUT_NAIVE_READ, LAYOUT_NAIVE_WRITE = 4, 5
LAYOUT_NAMES = {LAYOUT_UNPADDED: "unpadded", LAYOUT_PAD1: "pad1",
                LAYOUT_SWIZZLE: "swizzle"}
NAIVE_NAMES = {LAYOUT_NAIVE_READ: "naive_read_coalesced",
               LAYOUT_NAIVE_WRITE: "naive_write_coalesced"}
FLAG_ELEMENTWISE, FLAG_XCD_REMAP, FLAG_NO_XCD_REMAP = 1, 2, 4
FLAG_DIRECT_LDS, FLAG_ALIGN_OUT, FLAG_NO_ALIGN_OUT = 8, 16, 32
FLAG_TR_READ = 64
FLAG_PACKED, FLAG_NO_PACKED = 128, 256
CACHE_AUTO, CACHE_DEFAULT, CACHE_NT_STORE, CACHE_NT_ALL = 0, 1, 2, 3
ORDER_AUTO, ORDER_SUPER_TILES, ORDER_DIAGONAL, ORDER_COLUMN_BANDS = 0, 1, 2, 3
CACHE_NAMES = {CACHE_DEFAULT: "default", CACHE_NT_STORE: "nt_store",
               CACHE_NT_ALL: "nt_all"}

AS_AUTO, AS_UNPADDED, AS_PADDED, AS_SWIZZLE = 0, 1, 2, 3
AS_NAMES = {AS_UNPADDED: "unpadded", AS_PADDED: "padded",
            AS_SWIZZLE: "swizzle"}
SGEMM_NO_XCD_REMAP, SGEMM_DOUBLE_BUFFER, SGEMM_NO_BUFFER_LOADS = 1, 2, 4

# Every exported entry point, in header order (include/xpose.h, then
# include/xpose_sgemm.h).
EXPORTS = ("xpose_2d", "xpose_2d_ex", "xpose_batched", "xpose_batched_ex",
           "xpose_plan",
           "xpose_copy", "xpose_copy_ex", "xpose_lds_probe",
           "xpose_last_hip_error", "xpose_strerror",
           "xpose_sgemm", "xpose_sgemm_ex", "xpose_sgemm_plan",
           "xpose_sgemm_ws", "xpose_sgemm_noalloc", "xpose_sgemm_plan_ws")


class XposeOpts(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("tile_cols", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("cache", ctypes.c_int32), ("group_rows", ctypes.c_int32),
                ("group_cols", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("order", ctypes.c_int32), ("persistent", ctypes.c_int32),
                ("occupancy", ctypes.c_int32)]


class XposeCopyOpts(ctypes.Structure):
    _fields_ = [("threads", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("cache", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class XposePlanInfo(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("tile_cols", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("vector_path", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("launches", ctypes.c_int32),
                ("cache", ctypes.c_int32), ("group_rows", ctypes.c_int32),
                ("group_cols", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("order", ctypes.c_int32), ("persistent", ctypes.c_int32),
                ("direct_lds", ctypes.c_int32), ("aligned_out", ctypes.c_int32),
                ("tr_read", ctypes.c_int32), ("packed", ctypes.c_int32),
                ("occupancy", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class XposeSgemmOpts(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("split_k", ctypes.c_int32)]


class XposeSgemmInfo(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("as_stride", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("vector_loads", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("buffer_loads", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("whole_matrix", ctypes.c_int32),
                ("edge_buffer_loads", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("split_len", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64),
                ("workspace_wanted", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


def _load() -> ctypes.CDLL:
    # libxpose.so needs libamdhip64.so.7.  PyTorch's ROCm wheel ships its own
    # HIP and HSA runtimes under that same soname; if libxpose.so were loaded
    # first, the process would end up with two HIP runtimes (ROCm's and
    # torch's), each with its own device context, and launches on torch
    # memory fail or crash.  Importing torch first makes the dynamic loader
    # resolve libamdhip64.so.7 to the runtime torch already loaded.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python lds_tiled_matrix_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f32 = ctypes.c_float
    opts_p, info_p = ctypes.POINTER(XposeOpts), ctypes.POINTER(XposePlanInfo)
    sig = {
        "xpose_2d": [p, p, i64, i64, i64, i64, i32, p],
        "xpose_2d_ex": [p, p, i64, i64, i64, i64, i32, opts_p, p],
        "xpose_batched": [p, p, i64, i64, i64, i64, i64, i64, i64, i32, p],
        "xpose_batched_ex": [p, p, i64, i64, i64, i64, i64, i64, i64, i32,
                             opts_p, p],
        "xpose_plan": [p, p, i64, i64, i64, i64, i64, i64, i64, i32, opts_p,
                       info_p],
        "xpose_copy": [p, p, i64, p],
        "xpose_copy_ex": [p, p, i64, ctypes.POINTER(XposeCopyOpts), p],
        "xpose_lds_probe": [p, ctypes.POINTER(i32), i32, i32, i32, p],
        "xpose_last_hip_error": [],
        "xpose_strerror": [ctypes.c_int],
        "xpose_sgemm": [i64, i64, i64, f32, p, i64, p, i64, f32, p, i64, p],
        "xpose_sgemm_ex": [i64, i64, i64, f32, p, i64, p, i64, f32, p, i64,
                           ctypes.POINTER(XposeSgemmOpts), p],
        "xpose_sgemm_plan": [i64, i64, i64, p, i64, p, i64, p, i64,
                             ctypes.POINTER(XposeSgemmOpts),
                             ctypes.POINTER(XposeSgemmInfo)],
        "xpose_sgemm_ws": [i64, i64, i64, f32, p, i64, p, i64, f32, p, i64,
                           ctypes.POINTER(XposeSgemmOpts), p, i64, p],
        "xpose_sgemm_noalloc": [i64, i64, i64, f32, p, i64, p, i64, f32, p,
                                i64, ctypes.POINTER(XposeSgemmOpts), p],
        "xpose_sgemm_plan_ws": [i64, i64, i64, p, i64, p, i64, p, i64,
                                ctypes.POINTER(XposeSgemmOpts), p, i64,
                                ctypes.POINTER(XposeSgemmInfo)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "xpose_strerror" else ctypes.c_int
    return lib


_lib = _load()


class XposeError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = f"{what}: {strerror(code)} ({code})"
        if code == XPOSE_EHIP:
            msg += f", hipError {_lib.xpose_last_hip_error()}"
        super().__init__(msg)


def _check(code: int, what: str) -> int:
    if code != XPOSE_OK:
        raise XposeError(code, what)
    return code


def make_opts(layout=LAYOUT_AUTO, tile=None, flags=0, cache=CACHE_AUTO,
              group_rows=0, group_cols=0, threads=0, order=ORDER_AUTO,
              persistent=0, occupancy=0) -> XposeOpts:
    tr, tc = tile if tile else (0, 0)
    return XposeOpts(layout, tr, tc, flags, cache, group_rows, group_cols,
                     threads, order, persistent, occupancy)


# ----- C ABI, one to one -----------------------------------------------------

def xpose_2d(out: int, inp: int, rows: int, cols: int, ld_in: int,
             ld_out: int, dtype: int, stream: int = 0) -> int:
    return _lib.xpose_2d(out, inp, rows, cols, ld_in, ld_out, dtype, stream)


def xpose_2d_ex(out: int, inp: int, rows: int, cols: int, ld_in: int,
                ld_out: int, dtype: int, opts: XposeOpts | None = None,
                stream: int = 0) -> int:
    return _lib.xpose_2d_ex(out, inp, rows, cols, ld_in, ld_out, dtype,
                            ctypes.byref(opts) if opts else None, stream)


def xpose_batched(out: int, inp: int, batch: int, rows: int, cols: int,
                  ld_in: int, ld_out: int, stride_in: int, stride_out: int,
                  dtype: int, stream: int = 0) -> int:
    return _lib.xpose_batched(out, inp, batch, rows, cols, ld_in, ld_out,
                              stride_in, stride_out, dtype, stream)


def xpose_batched_ex(out: int, inp: int, batch: int, rows: int, cols: int,
                     ld_in: int, ld_out: int, stride_in: int, stride_out: int,
                     dtype: int, opts: XposeOpts | None = None,
                     stream: int = 0) -> int:
    return _lib.xpose_batched_ex(out, inp, batch, rows, cols, ld_in, ld_out,
                                 stride_in, stride_out, dtype,
                                 ctypes.byref(opts) if opts else None, stream)


def xpose_plan(out: int, inp: int, batch: int, rows: int, cols: int,
               ld_in: int, ld_out: int, stride_in: int, stride_out: int,
               dtype: int, opts: XposeOpts | None = None):
    """Returns (status, XposePlanInfo)."""
    info = XposePlanInfo()
    rc = _lib.xpose_plan(out, inp, batch, rows, cols, ld_in, ld_out,
                         stride_in, stride_out, dtype,
                         ctypes.byref(opts) if opts else None,
                         ctypes.byref(info))
    return rc, info


def xpose_copy(dst: int, src: int, nbytes: int, stream: int = 0) -> int:
    return _lib.xpose_copy(dst, src, nbytes, stream)


def xpose_copy_ex(dst: int, src: int, nbytes: int,
                  opts: XposeCopyOpts | None = None, stream: int = 0) -> int:
    return _lib.xpose_copy_ex(dst, src, nbytes,
                              ctypes.byref(opts) if opts else None, stream)


def xpose_lds_probe(cycles_out: int, lane_bytes, width: int, is_write: int,
                    iters: int, stream: int = 0) -> int:
    arr = (ctypes.c_int32 * 64)(*[int(x) for x in lane_bytes])
    return _lib.xpose_lds_probe(cycles_out, arr, width, is_write, iters,
                                stream)


def make_sgemm_opts(layout=AS_AUTO, bk=0, group_m=0, flags=0,
                    tile_m=0, split_k=0) -> XposeSgemmOpts:
    return XposeSgemmOpts(layout, bk, group_m, flags, tile_m, split_k)


def xpose_sgemm(m: int, n: int, k: int, alpha: float, a: int, lda: int,
                b: int, ldb: int, beta: float, c: int, ldc: int,
                stream: int = 0) -> int:
    return _lib.xpose_sgemm(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc,
                            stream)


def xpose_sgemm_ex(m: int, n: int, k: int, alpha: float, a: int, lda: int,
                   b: int, ldb: int, beta: float, c: int, ldc: int,
                   opts: XposeSgemmOpts | None = None,
                   stream: int = 0) -> int:
    return _lib.xpose_sgemm_ex(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc,
                               ctypes.byref(opts) if opts else None, stream)


def xpose_sgemm_plan(m: int, n: int, k: int, a: int, lda: int, b: int,
                     ldb: int, c: int, ldc: int,
                     opts: XposeSgemmOpts | None = None):
    """Returns (status, XposeSgemmInfo)."""
    info = XposeSgemmInfo()
    rc = _lib.xpose_sgemm_plan(m, n, k, a, lda, b, ldb, c, ldc,
                               ctypes.byref(opts) if opts else None,
                               ctypes.byref(info))
    return rc, info


def xpose_sgemm_ws(m: int, n: int, k: int, alpha: float, a: int, lda: int,
                   b: int, ldb: int, beta: float, c: int, ldc: int,
                   opts: XposeSgemmOpts | None = None, workspace: int = 0,
                   workspace_bytes: int = 0, stream: int = 0) -> int:
    return _lib.xpose_sgemm_ws(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc,
                               ctypes.byref(opts) if opts else None,
                               workspace, workspace_bytes, stream)


def xpose_sgemm_noalloc(m: int, n: int, k: int, alpha: float, a: int,
                        lda: int, b: int, ldb: int, beta: float, c: int,
                        ldc: int, opts: XposeSgemmOpts | None = None,
                        stream: int = 0) -> int:
    return _lib.xpose_sgemm_noalloc(m, n, k, alpha, a, lda, b, ldb, beta, c,
                                    ldc, ctypes.byref(opts) if opts else None,
                                    stream)


def xpose_sgemm_plan_ws(m: int, n: int, k: int, a: int, lda: int, b: int,
                        ldb: int, c: int, ldc: int,
                        opts: XposeSgemmOpts | None = None,
                        workspace: int = 0, workspace_bytes: int = 0):
    """Returns (status, XposeSgemmInfo)."""
    info = XposeSgemmInfo()
    rc = _lib.xpose_sgemm_plan_ws(m, n, k, a, lda, b, ldb, c, ldc,
                                  ctypes.byref(opts) if opts else None,
                                  workspace, workspace_bytes,
                                  ctypes.byref(info))
    return rc, info


def xpose_last_hip_error() -> int:
    return _lib.xpose_last_hip_error()


def strerror(code: int) -> str:
    return _lib.xpose_strerror(code).decode()


# ----- torch conveniences (memory and streams only) --------------------------

def dtype_code(t) -> int:
    """xpose_dtype for a torch dtype, by element size."""
    import torch
    table = {torch.float32: XPOSE_F32, torch.int32: XPOSE_F32,
             torch.uint32: XPOSE_F32, torch.float16: XPOSE_F16,
             torch.bfloat16: XPOSE_BF16, torch.int16: XPOSE_F16,
             torch.uint16: XPOSE_F16, torch.uint8: XPOSE_U8,
             torch.int8: XPOSE_U8, torch.float64: XPOSE_F64,
             torch.int64: XPOSE_F64, torch.uint64: XPOSE_F64}
    if t not in table:
        raise TypeError(f"unsupported dtype {t}")
    return table[t]


def _require_device(*tensors) -> None:
    """The library dereferences its pointers on the GPU only: every tensor
    must live in device memory, all on one device.  Checked before anything
    is launched, so a host tensor is a Python error, not a GPU fault."""
    devs = set()
    for t in tensors:
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"expected a CUDA tensor, got one on {t.device}")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def transpose(x, out=None, *, layout: int = LAYOUT_AUTO, tile=None,
              flags: int = 0, cache: int = CACHE_AUTO, group_rows: int = 0,
              order: int = ORDER_AUTO, persistent: int = 0, stream=None):
    """Transpose the last two dims of a 2-D or 3-D CUDA tensor whose last dim
    is contiguous.  Row pitches and the batch stride are taken from the
    tensor's strides.  Returns ``out`` (allocated contiguous if None)."""
    import torch
    _require_device(x)
    if x.dim() not in (2, 3):
        raise ValueError("expected a 2-D or 3-D tensor")
    if x.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    batch = x.shape[0] if x.dim() == 3 else 1
    rows, cols = x.shape[-2], x.shape[-1]
    if out is None:
        shape = (cols, rows) if x.dim() == 2 else (batch, cols, rows)
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _require_device(x, out)
    if out.dtype != x.dtype or out.stride(-1) != 1:
        raise ValueError("out must match dtype and have a contiguous last dim")
    if tuple(out.shape[-2:]) != (cols, rows):
        raise ValueError("out has the wrong shape")
    ld_in = x.stride(-2) if rows > 1 else cols
    ld_out = out.stride(-2) if cols > 1 else rows
    stride_in = x.stride(0) if x.dim() == 3 else 0
    stride_out = out.stride(0) if out.dim() == 3 else 0
    code = dtype_code(x.dtype)
    opts = (make_opts(layout, tile, flags, cache, group_rows, 0, 0, order,
                      persistent)
            if (layout or tile or flags or cache or group_rows or order
                or persistent) else None)
    _check(xpose_batched_ex(out.data_ptr(), x.data_ptr(), batch, rows, cols,
                            ld_in, ld_out, stride_in, stride_out, code, opts,
                            _stream_handle(stream)), "xpose_batched_ex")
    return out


def copy(dst, src, stream=None):
    """Byte copy between two contiguous CUDA tensors of equal byte size, by
    the library's 128-bit copy kernel."""
    _require_device(dst, src)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("byte sizes differ")
    _check(xpose_copy(dst.data_ptr(), src.data_ptr(), nbytes,
                      _stream_handle(stream)), "xpose_copy")
    return dst


def plan_for(x, out=None, *, layout: int = LAYOUT_AUTO, tile=None,
             flags: int = 0, cache: int = CACHE_AUTO,
             group_rows: int = 0) -> dict:
    """The kernel ``transpose`` would launch for these tensors (host only)."""
    batch = x.shape[0] if x.dim() == 3 else 1
    rows, cols = x.shape[-2], x.shape[-1]
    ld_in = x.stride(-2) if rows > 1 else cols
    stride_in = x.stride(0) if x.dim() == 3 else 0
    if out is None:
        out_ptr, ld_out, stride_out = 0x100000000000, rows, rows * cols
    else:
        out_ptr = out.data_ptr()
        ld_out = out.stride(-2) if cols > 1 else rows
        stride_out = out.stride(0) if out.dim() == 3 else 0
    opts = (make_opts(layout, tile, flags, cache, group_rows)
            if (layout or tile or flags or cache or group_rows) else None)
    rc, info = xpose_plan(out_ptr, x.data_ptr(), batch, rows, cols, ld_in,
                          ld_out, stride_in, stride_out, dtype_code(x.dtype),
                          opts)
    _check(rc, "xpose_plan")
    return info.as_dict()


def sgemm(a, b, c=None, *, alpha: float = 1.0, beta: float = 0.0,
          layout: int = AS_AUTO, bk: int = 0, split_k: int = 0, stream=None):
    """c = alpha * a @ b + beta * c for 2-D float32 CUDA tensors whose last
    dimension is contiguous (pitches come from the row strides).  With c
    None, a new tensor is allocated and beta must be 0.  Where the library
    splits k (split_k 0: its own rule; >= 2: that split), torch allocates
    the workspace for the partial sums.  Returns c."""
    import torch
    _require_device(a, b, *(() if c is None else (c,)))
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("expected 2-D tensors")
    m, k = a.shape
    if b.shape[0] != k:
        raise ValueError("inner dimensions differ")
    n = b.shape[1]
    if c is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs c")
        c = torch.empty((m, n), dtype=torch.float32, device=a.device)
    for t in (a, b, c):
        if t.dtype != torch.float32 or (t.numel() > 1 and t.stride(-1) != 1):
            raise ValueError("float32 tensors with a contiguous last dim")
    if tuple(c.shape) != (m, n):
        raise ValueError("c has the wrong shape")
    lda = a.stride(0) if m > 1 else max(k, 1)
    ldb = b.stride(0) if k > 1 else max(n, 1)
    ldc = c.stride(0) if m > 1 else max(n, 1)
    opts = make_sgemm_opts(layout, bk, split_k=split_k)
    args = (m, n, k, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc)
    rc, info = xpose_sgemm_plan_ws(*args, opts)   # the size query
    if rc != XPOSE_EWORKSPACE:
        _check(rc, "xpose_sgemm_plan_ws")
    ws = None
    if info.workspace_wanted:
        ws = torch.empty(info.workspace_wanted // 4, dtype=torch.float32,
                         device=a.device)
    _check(xpose_sgemm_ws(m, n, k, alpha, a.data_ptr(), lda, b.data_ptr(),
                          ldb, beta, c.data_ptr(), ldc, opts,
                          ws.data_ptr() if ws is not None else 0,
                          info.workspace_wanted, _stream_handle(stream)),
           "xpose_sgemm_ws")
    if ws is not None and stream is not None:
        # allocated on the current stream, used on `stream`: keep it from
        # being reused before the call's kernels have run there
        ws.record_stream(stream)
    return c
