"""The C-ABI library loads and exports every function include/dbs.h declares;
host-side argument checks answer without touching a GPU (CPU only)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dbs.h")
LIB = os.path.join(ROOT, "spmspv_graph_traversal_amd", "libdbs.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dbs_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from spmspv_graph_traversal_amd import build_lib

        build_lib.build()
    return C.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ["dbs_build", "dbs_spmspv", "dbs_spmspv_dense", "dbs_bfs", "dbs_free", "dbs_get_stats",
              "dbs_set_option", "dbs_get_option", "dbs_copy_array", "dbs_status_string",
              "dbs_build_options_default"]:
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in dbs.h but not exported"


def test_binding_covers_every_symbol():
    import spmspv_graph_traversal_amd.binding as b

    assert set(declared_functions()) == set(b.EXPORTED)


def test_host_side_validation_without_gpu(lib):
    lib.dbs_status_string.restype = C.c_char_p
    assert lib.dbs_status_string(0) == b"ok"
    assert lib.dbs_status_string(2) == b"invalid CSR input"
    vp = C.c_void_p
    h = vp()
    # m < 1, null row_ptr, nnz < 0, bad dtype, missing values: rejected before any HIP call
    lib.dbs_build.argtypes = [C.c_int32, C.c_int32, C.c_int64, vp, vp, vp, C.c_int, vp, vp, C.POINTER(vp)]
    assert lib.dbs_build(0, 5, 0, vp(8), vp(8), None, 0, None, None, C.byref(h)) == 1
    assert lib.dbs_build(5, 5, 0, None, vp(8), None, 0, None, None, C.byref(h)) == 1
    assert lib.dbs_build(5, 5, -1, vp(8), vp(8), vp(8), 0, None, None, C.byref(h)) == 1
    assert lib.dbs_build(5, 5, 3, vp(8), vp(8), vp(8), 7, None, None, C.byref(h)) == 1
    assert lib.dbs_build(5, 5, 3, vp(8), vp(8), None, 0, None, None, C.byref(h)) == 1
    assert lib.dbs_build(5, 5, 3, vp(8), vp(8), None, 2, None, None, None) == 1
    lib.dbs_spmspv.argtypes = [vp, C.c_int32, vp, vp, C.c_int, vp, vp]
    assert lib.dbs_spmspv(None, 0, None, None, 0, vp(8), None) == 1
    lib.dbs_bfs.argtypes = [vp, C.c_int32, vp, vp]
    assert lib.dbs_bfs(None, 0, vp(8), None) == 1
    lib.dbs_set_option.argtypes = [vp, C.c_int32, C.c_int64]
    assert lib.dbs_set_option(None, 0, 0) == 1
    lib.dbs_free.argtypes = [vp]
    assert lib.dbs_free(None) == 0
    # the read probe: null buffer or sink, a size that is not a positive multiple
    # of 16, a buffer not 16-byte aligned
    lib.dbs_probe_read.argtypes = [vp, C.c_int64, vp, C.c_uint32, vp]
    assert lib.dbs_probe_read(None, 64, vp(16), 0, None) == 1
    assert lib.dbs_probe_read(vp(16), 64, None, 0, None) == 1
    assert lib.dbs_probe_read(vp(16), 40, vp(16), 0, None) == 1
    assert lib.dbs_probe_read(vp(16), 0, vp(16), 0, None) == 1
    assert lib.dbs_probe_read(vp(24), 64, vp(16), 0, None) == 1


def test_default_build_options(lib):
    from spmspv_graph_traversal_amd.binding import dbs_build_options

    o = dbs_build_options()
    assert lib.dbs_build_options_default(C.byref(o)) == 0
    # section 3.2.1 thresholds, section 3.3.2 weights; cap 64 for one 64-lane wave
    assert (o.th0, o.th1, o.th2_num, o.th2_den, o.force_format) == (32, 128, 2, 1, -1)
    assert (o.seg_w_dense, o.seg_w_csr, o.seg_w_coo, o.seg_cap) == (4, 2, 1, 0)
    assert lib.dbs_build_options_default(None) == 1


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: a request for more exits with a message and status 2,
    # before anything touches a device
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.lstrip().startswith("{")


def test_build_helper_imports_without_the_library():
    """The build helper must import on a tree where libdbs.so is not built yet,
    without loading the binding (which refuses to load without the library)."""
    import subprocess
    import sys

    code = ("import sys; from spmspv_graph_traversal_amd import build_lib; "
            "assert callable(build_lib.build); "
            "assert 'spmspv_graph_traversal_amd.binding' not in sys.modules")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
