"""The C ABI from a C99 caller (CPU only): the header compiles as strict C,
and struct layouts, constants and host-only plans agree with the Python
binding."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

X = pytest.importorskip("lds_tiled_matrix_amd")

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.join(ROOT, "lds_tiled_matrix_amd")


@pytest.fixture(scope="module")
def c_output():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_c")
        subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(HERE, "native", "abi_c.c"), "-o", exe,
                        "-L", LIBDIR, "-lxpose", f"-Wl,-rpath,{LIBDIR}"],
                       check=True, capture_output=True, timeout=120)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                             check=True).stdout
    return out.splitlines()


def _entries(lines, kind):
    return [ln.split(" ", 2)[1:] for ln in lines if ln.startswith(kind + " ")]


def test_struct_layouts_match_ctypes(c_output):
    structs = {"xpose_opts": X.XposeOpts, "xpose_plan_info": X.XposePlanInfo,
               "xpose_copy_opts": X.XposeCopyOpts,
               "xpose_sgemm_opts": X.XposeSgemmOpts,
               "xpose_sgemm_info": X.XposeSgemmInfo}
    sizes = dict(_entries(c_output, "size"))
    for name, cls in structs.items():
        assert int(sizes[name]) == ctypes.sizeof(cls), name
    offsets = _entries(c_output, "offset")
    assert len(offsets) >= 9
    for field, off in offsets:
        sname, fname = field.split(".")
        assert getattr(structs[sname], fname).offset == int(off), field


def test_constants_match_binding(c_output):
    consts = dict(_entries(c_output, "const"))
    assert len(consts) == 21
    for name, value in consts.items():
        short = name.replace("XPOSE_FLAG_", "FLAG_").replace("XPOSE_AS_", "AS_")
        short = short.replace("XPOSE_SGEMM_", "SGEMM_")
        py = getattr(X, name, None)
        if py is None:
            py = getattr(X, short)
        assert py == int(value), name


def test_plans_match_binding(c_output):
    plans = {}
    for ln in c_output:
        if ln.startswith("plan "):
            f = ln.split()
            plans[f[1]] = (int(f[2]), dict(kv.split("=") for kv in f[3:]))
    out, inp = 0x100000000000, 0x200000000000
    cases = {"c2": (8192, 8192, X.XPOSE_F32, None),
             "c3": (12345, 6789, X.XPOSE_F32, None),
             "c4": (16384, 16384, X.XPOSE_F16, None),
             "c4tr": (16384, 16384, X.XPOSE_F16, X.make_opts(flags=X.FLAG_TR_READ))}
    for tag, (r, c, dt, opts) in cases.items():
        rc, info = X.xpose_plan(out, inp, 1, r, c, c, r, r * c, c * r, dt, opts)
        crc, cinfo = plans[tag]
        assert crc == rc == 0, tag
        for k, v in cinfo.items():
            assert getattr(info, k) == int(v), (tag, k)
    assert plans["null"][0] == X.XPOSE_EINVAL
    assert plans["alias"][0] == X.XPOSE_EALIAS
    assert plans["dtype"][0] == X.XPOSE_EDTYPE
    assert plans["c4tr"][1]["tr_read"] == "1"


def test_2d_ex_from_c(c_output):
    ex = dict(_entries(c_output, "ex"))
    assert int(ex["pitch"]) == X.XPOSE_EINVAL
    assert int(ex["alias"]) == X.XPOSE_EALIAS
    assert int(ex["layout"]) == X.XPOSE_EINVAL
    assert int(ex["dtype"]) == X.XPOSE_EDTYPE
    assert int(ex["empty"]) == X.XPOSE_OK
    out, inp = 0x100000000000, 0x200000000000
    assert X.xpose_2d_ex(out, inp, 64, 64, 63, 64, X.XPOSE_F32) == X.XPOSE_EINVAL
    assert X.xpose_2d_ex(out, inp, 64, 64, 64, 64, X.XPOSE_F32,
                         X.make_opts(layout=9)) == X.XPOSE_EINVAL


def test_strerror_matches_binding(c_output):
    for code, text in _entries(c_output, "strerror"):
        assert X.strerror(int(code)) == text


def test_sgemm_plan_matches_binding(c_output):
    line = [ln for ln in c_output if ln.startswith("sgemm ")]
    assert len(line) == 1
    f = line[0].split()
    fields = dict(kv.split("=") for kv in f[2:])
    rc, info = X.xpose_sgemm_plan(4096, 4096, 4096, 0x300000000000, 4096,
                                  0x310000000000, 4096, 0x320000000000, 4096)
    assert int(f[1]) == rc == 0
    for k, v in fields.items():
        assert getattr(info, k) == int(v), k


def test_sgemm_plan_ws_matches_binding(c_output):
    line = [ln for ln in c_output if ln.startswith("sgemmws ")]
    assert len(line) == 1
    f = line[0].split()
    fields = dict(kv.split("=") for kv in f[2:])
    rc, info = X.xpose_sgemm_plan_ws(1024, 1024, 1024, 0x300000000000, 1024,
                                     0x310000000000, 1024, 0x320000000000,
                                     1024, None, 0x330000000000, 1 << 30)
    assert int(f[1]) == rc == 0
    assert info.splits > 1
    for k, v in fields.items():
        assert getattr(info, k) == int(v), k
