"""ctypes binding of ``libdbs.so`` (declared in ``include/dbs.h``).

Argument marshalling only: every step of the computation runs in the HIP
library.  Tensors are torch tensors on the current GPU (torch provides the
device memory and the stream); the functions carry the C names.  Importing
this module without the built library raises ``ImportError`` — there is no
fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdbs.so")

# status codes (dbs_status)
DBS_OK, DBS_ERR_INVALID_ARG, DBS_ERR_BAD_CSR, DBS_ERR_OUT_OF_MEMORY = 0, 1, 2, 3
DBS_ERR_DEVICE, DBS_ERR_UNSUPPORTED, DBS_ERR_BAD_VECTOR, DBS_ERR_TOO_LARGE = 4, 5, 6, 7
DBS_NOALLOC_SCRATCH_BYTES = 32 << 20
# dtypes, semirings, tile formats
DBS_F32, DBS_BF16, DBS_PATTERN = 0, 1, 2
DBS_PLUS_TIMES, DBS_OR_AND = 0, 1
DBS_TILE_COO, DBS_TILE_DENSE, DBS_TILE_FORCE_CSR, DBS_TILE_FORCE_CSC, DBS_TILE_CSR = 0, 1, 2, 3, 4
# options
DBS_OPT_PATH, DBS_OPT_TH3_NUM, DBS_OPT_TH3_DEN = 0, 1, 2
DBS_OPT_LOCAL_PUSH_CUTOFF, DBS_OPT_TIMING, DBS_OPT_CHECK = 3, 4, 5
DBS_OPT_PULL_WIDTH, DBS_OPT_PULL_SHARE = 6, 7
# exported arrays
(DBS_ARR_RB_PTR, DBS_ARR_T_CB, DBS_ARR_T_META, DBS_ARR_CB_PTR, DBS_ARR_CSC_RB, DBS_ARR_CSC2CSR,
 DBS_ARR_PAYLOAD, DBS_ARR_SEGMENTS, DBS_ARR_XMASK, DBS_ARR_ACTIVE, DBS_ARR_CSC_CM, DBS_ARR_PAT_SEGS,
 DBS_ARR_T_CBX, DBS_ARR_META2, DBS_ARR_PAT_M2) = range(15)

_ARR_DTYPES = {
    DBS_ARR_RB_PTR: np.uint32, DBS_ARR_T_CB: np.uint32, DBS_ARR_T_META: np.uint64,
    DBS_ARR_CB_PTR: np.uint32, DBS_ARR_CSC_RB: np.uint32, DBS_ARR_CSC2CSR: np.uint32,
    DBS_ARR_PAYLOAD: np.uint8, DBS_ARR_SEGMENTS: np.uint32, DBS_ARR_XMASK: np.uint16,
    DBS_ARR_ACTIVE: np.uint32, DBS_ARR_CSC_CM: np.uint16, DBS_ARR_PAT_SEGS: np.uint32,
    DBS_ARR_T_CBX: np.uint32, DBS_ARR_META2: np.uint64, DBS_ARR_PAT_M2: np.uint32,
}


class dbs_build_options(C.Structure):
    _fields_ = [(name, C.c_int32) for name in (
        "th0", "th1", "th2_num", "th2_den", "force_format", "seg_w_dense", "seg_w_csr",
        "seg_w_coo", "seg_cap")]


class dbs_stats(C.Structure):
    _fields_ = [
        ("m", C.c_int32), ("n", C.c_int32), ("mb", C.c_int32), ("nb", C.c_int32),
        ("nnz", C.c_int64), ("tiles", C.c_int64),
        ("tiles_by_format", C.c_int64 * 5), ("nnz_by_format", C.c_int64 * 5),
        ("segments", C.c_int64), ("payload_bytes", C.c_int64), ("index_bytes", C.c_int64),
        ("format_bytes", C.c_int64), ("build_peak_bytes", C.c_int64),
        ("last_path", C.c_int32), ("last_n_nzblk", C.c_int32), ("last_push_chunks", C.c_int64),
        ("last_meta_ms", C.c_float), ("last_compute_ms", C.c_float),
        ("timed_calls", C.c_int64), ("sum_meta_ms", C.c_double), ("sum_compute_ms", C.c_double),
        ("bfs_levels", C.c_int32), ("bfs_push_levels", C.c_int32), ("bfs_reached", C.c_int64),
        ("bfs_ms", C.c_float), ("bfs_kernel_ms", C.c_float),
    ]


EXPORTED = ["dbs_build_options_default", "dbs_build", "dbs_spmspv", "dbs_spmspv_dense",
            "dbs_spmspv_dense_threshold", "dbs_bfs", "dbs_bfs_noalloc",
            "dbs_set_option", "dbs_get_option", "dbs_get_stats", "dbs_copy_array", "dbs_free",
            "dbs_status_string", "dbs_probe_read"]


def load_library(path: str = LIB_PATH) -> C.CDLL:
    # torch first: its HIP runtime (SONAME libamdhip64.so.7) is then the one
    # the library binds to, so torch's allocations and streams are valid in
    # the library.  Loading the library first would pull in a second runtime.
    import torch  # noqa: F401

    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(path)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    sig = {
        "dbs_build_options_default": [C.POINTER(dbs_build_options)],
        "dbs_build": [i32, i32, i64, vp, vp, vp, C.c_int, C.POINTER(dbs_build_options), vp,
                      C.POINTER(vp)],
        "dbs_spmspv": [vp, i32, vp, vp, C.c_int, vp, vp],
        "dbs_spmspv_dense": [vp, vp, C.c_int, vp, vp],
        "dbs_spmspv_dense_threshold": [vp, vp, C.c_float, C.c_int, vp, vp],
        "dbs_bfs": [vp, i32, vp, vp],
        "dbs_bfs_noalloc": [vp, i32, vp, vp],
        "dbs_set_option": [vp, i32, i64],
        "dbs_get_option": [vp, i32, C.POINTER(i64)],
        "dbs_get_stats": [vp, C.POINTER(dbs_stats)],
        "dbs_copy_array": [vp, i32, vp, i64, C.POINTER(i64)],
        "dbs_free": [vp],
        "dbs_probe_read": [vp, i64, vp, C.c_uint32, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.dbs_status_string.argtypes = [C.c_int]
    lib.dbs_status_string.restype = C.c_char_p
    return lib


_lib = load_library()


class DBSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.dbs_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(st: int, where: str) -> None:
    if st != DBS_OK:
        raise DBSError(st, where)


# torch (imported by load_library before the library) and its raw current
# stream getter, looked up once: the per-call wrappers run at a few us
import torch as _torch  # noqa: E402

_RAW_STREAM = getattr(_torch._C, "_cuda_getCurrentRawStream", None)
_Tensor = _torch.Tensor
_I32, _F32, _U8 = (_torch.int32,), (_torch.float32,), (_torch.uint8,)


def _ptr(t):
    # the argtypes are c_void_p: a plain int (or None) converts on the call
    return None if t is None else t.data_ptr()


def _stream(stream, device=None):
    """Raw HIP stream handle: the given stream, else the current stream of
    `device` (the call's output tensor's device), read without building a
    Stream object where torch offers that."""
    if stream is None:
        if _RAW_STREAM is not None and device is not None:
            idx = device.index
            return _RAW_STREAM(idx if idx is not None else _torch.cuda.current_device())
        stream = _torch.cuda.current_stream(device)
    return stream.cuda_stream


def _need(t, name, dtypes, numel=None):
    if not isinstance(t, _Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


_BF16_DTYPES = (_torch.bfloat16, _torch.int16, _torch.uint16)


def _value_dtypes(dtype):
    if dtype == DBS_F32:
        return _F32
    if dtype == DBS_BF16:
        return _BF16_DTYPES
    return ()


class Matrix:
    """Owner of a dbs_handle; freed with the object or by dbs_free."""

    def __init__(self, handle: C.c_void_p, m: int, n: int, dtype: int):
        self.handle = handle
        self.m, self.n, self.dtype = m, n, dtype

    def __del__(self):
        try:
            dbs_free(self)
        except Exception:
            pass


def default_build_options() -> dbs_build_options:
    o = dbs_build_options()
    _check(_lib.dbs_build_options_default(C.byref(o)), "dbs_build_options_default")
    return o


def dbs_build(m, n, row_ptr, col_idx, val, dtype, options=None, stream=None) -> Matrix:
    import torch

    _need(row_ptr, "row_ptr", (torch.int32,), m + 1)
    _need(col_idx, "col_idx", (torch.int32,))
    nnz = col_idx.numel()
    if dtype != DBS_PATTERN:
        _need(val, "val", _value_dtypes(dtype), nnz)
    h = C.c_void_p()
    opt = C.byref(options) if options is not None else None
    st = _lib.dbs_build(int(m), int(n), int(nnz), _ptr(row_ptr), _ptr(col_idx),
                        _ptr(val) if dtype != DBS_PATTERN else None, int(dtype), opt,
                        _stream(stream), C.byref(h))
    _check(st, "dbs_build")
    return Matrix(h, int(m), int(n), int(dtype))


def dbs_spmspv(A: Matrix, x_idx, x_val, semiring, y, stream=None) -> None:
    _need(x_idx, "x_idx", _I32)
    if semiring == DBS_PLUS_TIMES:
        _need(x_val, "x_val", _value_dtypes(A.dtype), x_idx.numel())
        _need(y, "y", _F32, A.m)
        xv = x_val.data_ptr()
    else:
        _need(y, "y", _U8, A.m)
        xv = None
    st = _lib.dbs_spmspv(A.handle, x_idx.numel(), x_idx.data_ptr(), xv, int(semiring), y.data_ptr(),
                         _stream(stream, y.device))
    if st != DBS_OK:
        raise DBSError(st, "dbs_spmspv")


def dbs_spmspv_dense(A: Matrix, x, semiring, y, stream=None) -> None:
    import torch

    xd = _value_dtypes(A.dtype) if A.dtype != DBS_PATTERN else (torch.float32,)
    _need(x, "x", xd, A.n)
    _need(y, "y", (torch.float32,) if semiring == DBS_PLUS_TIMES else (torch.uint8,), A.m)
    _check(_lib.dbs_spmspv_dense(A.handle, _ptr(x), int(semiring), _ptr(y), _stream(stream, y.device)),
           "dbs_spmspv_dense")


def dbs_spmspv_dense_threshold(A: Matrix, x, threshold: float, semiring, y, stream=None) -> None:
    import torch

    xd = _value_dtypes(A.dtype) if A.dtype != DBS_PATTERN else (torch.float32,)
    _need(x, "x", xd, A.n)
    _need(y, "y", (torch.float32,) if semiring == DBS_PLUS_TIMES else (torch.uint8,), A.m)
    _check(_lib.dbs_spmspv_dense_threshold(A.handle, _ptr(x), float(threshold), int(semiring), _ptr(y),
                                           _stream(stream, y.device)), "dbs_spmspv_dense_threshold")


def dbs_bfs(A: Matrix, src: int, levels, stream=None) -> None:
    import torch

    _need(levels, "levels", (torch.int32,), A.m)
    _check(_lib.dbs_bfs(A.handle, int(src), _ptr(levels), _stream(stream, levels.device)), "dbs_bfs")


def dbs_bfs_noalloc(A: Matrix, src: int, levels, stream=None) -> None:
    """dbs_bfs without allocation: the run's scratch is the library's fixed
    per-device array (DBS_NOALLOC_SCRATCH_BYTES); DBS_ERR_TOO_LARGE above it."""
    import torch

    _need(levels, "levels", (torch.int32,), A.m)
    _check(_lib.dbs_bfs_noalloc(A.handle, int(src), _ptr(levels), _stream(stream, levels.device)),
           "dbs_bfs_noalloc")


def dbs_set_option(A: Matrix, option: int, value: int) -> None:
    _check(_lib.dbs_set_option(A.handle, int(option), int(value)), "dbs_set_option")


def dbs_get_option(A: Matrix, option: int) -> int:
    v = C.c_int64()
    _check(_lib.dbs_get_option(A.handle, int(option), C.byref(v)), "dbs_get_option")
    return int(v.value)


def dbs_get_stats(A: Matrix, allow_bad_vector: bool = False) -> dict:
    s = dbs_stats()
    st = _lib.dbs_get_stats(A.handle, C.byref(s))
    if not (allow_bad_vector and st == DBS_ERR_BAD_VECTOR):
        _check(st, "dbs_get_stats")
    out = {}
    for name, _ in dbs_stats._fields_:
        v = getattr(s, name)
        out[name] = list(v) if isinstance(v, C.Array) else v
    out["status"] = st
    return out


def dbs_copy_array(A: Matrix, which: int) -> np.ndarray:
    nbytes = C.c_int64()
    _check(_lib.dbs_copy_array(A.handle, int(which), None, 0, C.byref(nbytes)), "dbs_copy_array")
    dt = _ARR_DTYPES[which]
    out = np.empty(nbytes.value // np.dtype(dt).itemsize, dtype=dt)
    _check(_lib.dbs_copy_array(A.handle, int(which), out.ctypes.data_as(C.c_void_p), out.nbytes,
                               C.byref(nbytes)), "dbs_copy_array")
    return out


def dbs_probe_read(buf, sink, never: int = 0xFFFFFFFF, stream=None) -> None:
    """Read the CUDA tensor `buf` once through the library's streaming-read
    probe (a measurement helper); `sink` is a one-element int32 CUDA tensor
    written only if some thread's XOR of words equals `never`."""
    if not isinstance(buf, _Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA tensor")
    _need(sink, "sink", _I32, 1)
    _check(_lib.dbs_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                               int(never) & 0xFFFFFFFF, _stream(stream, buf.device)), "dbs_probe_read")


def dbs_free(A: Matrix) -> None:
    if A.handle is not None and A.handle.value:
        _check(_lib.dbs_free(A.handle), "dbs_free")
        A.handle = C.c_void_p()
