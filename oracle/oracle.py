"""ctypes front end of the C oracle (``oracle.c``) — test infrastructure only.

The functions take and return numpy arrays.  The C library is compiled with
gcc into ``oracle/liboracle.so`` by :func:`build_oracle` (called by the repo's
``build()``; loading builds it once if it is missing).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_SRC_OMP = os.path.join(_HERE, "oracle_omp.c")
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")

F32, BF16, PATTERN = 0, 1, 2
COO, DENSE, FORCE_CSR, FORCE_CSC, CSR = 0, 1, 2, 3, 4
TYPE_NAMES = {COO: "COO", DENSE: "Dense", FORCE_CSR: "ForceCSR", FORCE_CSC: "ForceCSC", CSR: "CSR"}

# thresholds and weights as stated in sections 3.2.1, 3.3.1 and 3.3.2 of the paper
TH0, TH1, TH2, TH3 = 32, 128, 2.0, 0.01
W_DENSE, W_CSR, W_COO, SEG_CAP = 4, 2, 1, 16

_lib = None
_lib_omp = None


def build_oracle(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, no OpenMP), and oracle_omp.c (the
    all-core copy of the Boolean pull loop used only as a CPU baseline)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    if force or not os.path.exists(_LIB_OMP):
        tmp = _LIB_OMP + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC_OMP])
        os.replace(tmp, _LIB_OMP)
    return _LIB


def or_and_pull_all_cores(m, n, row_ptr, col_idx, x_idx):
    """orc_or_and_pull on every host core (OpenMP over rows); returns (y, threads)."""
    global _lib_omp
    if _lib_omp is None:
        if not os.path.exists(_LIB_OMP):
            build_oracle(force=True)
        _lib_omp = C.CDLL(_LIB_OMP)
        _lib_omp.orc_or_and_pull_omp.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                                                 C.c_void_p, C.c_void_p]
        _lib_omp.orc_or_and_pull_omp.restype = C.c_int
        _lib_omp.orc_omp_threads.restype = C.c_int
    rp, ci, xi = _i32(row_ptr), _i32(col_idx), _i32(x_idx)
    y = np.empty(m, np.uint8)
    _check(_lib_omp.orc_or_and_pull_omp(m, n, _p(rp), _p(ci), xi.shape[0], _p(xi), _p(y)), "or_and_pull_omp")
    return y, int(_lib_omp.orc_omp_threads())


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_oracle(force=True)
        _lib = C.CDLL(_LIB)
        i32, i64, vp, dbl = C.c_int32, C.c_int64, C.c_void_p, C.c_double
        sig = {
            "orc_csr_to_csc": (C.c_int, [i32, i32, vp, vp, vp, C.c_int, vp, vp, vp]),
            "orc_spmspv_pull": (C.c_int, [i32, i32, vp, vp, vp, C.c_int, i32, vp, vp, C.c_int, vp, vp]),
            "orc_spmspv_push": (C.c_int, [i32, i32, vp, vp, vp, C.c_int, i32, vp, vp, C.c_int, vp, vp]),
            "orc_or_and_pull": (C.c_int, [i32, i32, vp, vp, i32, vp, vp]),
            "orc_or_and_push": (C.c_int, [i32, i32, vp, vp, i32, vp, vp]),
            "orc_masked_or_and": (C.c_int, [i32, i32, vp, vp, i32, vp, vp, vp]),
            "orc_bfs": (C.c_int, [i32, vp, vp, i32, vp]),
            "orc_spmspv_dense_x": (C.c_int, [i32, i32, vp, vp, vp, C.c_int, vp, C.c_int, vp, vp]),
            "orc_threshold_activation": (C.c_int, [i32, vp, C.c_int, C.c_float, vp]),
            "orc_xmeta": (C.c_int, [i32, i32, vp, vp, vp]),
            "orc_xmeta_dense": (C.c_int, [i32, vp, C.c_int, vp, vp]),
            "orc_select_push": (C.c_int, [i32, i32, dbl]),
            "orc_classify": (C.c_int, [i32, i32, i32, i32, i32, dbl]),
            "orc_tile_view": (i64, [i32, i32, vp, vp, i32, i32, dbl] + [vp] * 12),
            "orc_segments": (i64, [i32, vp, vp, i32, i32, i32, i32, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(_lib, name)
            f.restype = res
            f.argtypes = args
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _vals(val, kind):
    if kind == PATTERN or val is None:
        return None
    return np.ascontiguousarray(val, dtype=np.float32 if kind == F32 else np.uint16)


def _check(rc, name):
    if rc < 0:
        raise RuntimeError(f"{name} failed ({rc})")
    return rc


# ------------------------------------------------------------------ SpMSpV
def csr_to_csc(m, n, row_ptr, col_idx, val=None, kind=PATTERN):
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    nnz = int(row_ptr[-1])
    v = _vals(val, kind)
    col_ptr = np.empty(n + 1, np.int32)
    row_idx = np.empty(nnz, np.int32)
    cv = None if v is None else np.empty(nnz, v.dtype)
    _check(lib.orc_csr_to_csc(m, n, _p(row_ptr), _p(col_idx), _p(v), kind, _p(col_ptr),
                              _p(row_idx), _p(cv)), "csr_to_csc")
    return col_ptr, row_idx, cv


def spmspv_pull(m, n, row_ptr, col_idx, val, kind, x_idx, x_val, xkind):
    """(y, s): y = A x over the listed entries (fp64), s = sum |a*x| per row."""
    lib = _load()
    row_ptr, col_idx, x_idx = _i32(row_ptr), _i32(col_idx), _i32(x_idx)
    v, xv = _vals(val, kind), _vals(x_val, xkind)
    y = np.empty(m, np.float64)
    s = np.empty(m, np.float64)
    _check(lib.orc_spmspv_pull(m, n, _p(row_ptr), _p(col_idx), _p(v), kind, x_idx.shape[0],
                               _p(x_idx), _p(xv), xkind, _p(y), _p(s)), "spmspv_pull")
    return y, s


def spmspv_push(m, n, col_ptr, row_idx, csc_val, kind, x_idx, x_val, xkind):
    lib = _load()
    col_ptr, row_idx, x_idx = _i32(col_ptr), _i32(row_idx), _i32(x_idx)
    v, xv = _vals(csc_val, kind), _vals(x_val, xkind)
    y = np.empty(m, np.float64)
    s = np.empty(m, np.float64)
    _check(lib.orc_spmspv_push(m, n, _p(col_ptr), _p(row_idx), _p(v), kind, x_idx.shape[0],
                               _p(x_idx), _p(xv), xkind, _p(y), _p(s)), "spmspv_push")
    return y, s


def or_and_pull(m, n, row_ptr, col_idx, x_idx):
    lib = _load()
    row_ptr, col_idx, x_idx = _i32(row_ptr), _i32(col_idx), _i32(x_idx)
    y = np.empty(m, np.uint8)
    _check(lib.orc_or_and_pull(m, n, _p(row_ptr), _p(col_idx), x_idx.shape[0], _p(x_idx), _p(y)),
           "or_and_pull")
    return y


def or_and_push(m, n, col_ptr, row_idx, x_idx):
    lib = _load()
    col_ptr, row_idx, x_idx = _i32(col_ptr), _i32(row_idx), _i32(x_idx)
    y = np.empty(m, np.uint8)
    _check(lib.orc_or_and_push(m, n, _p(col_ptr), _p(row_idx), x_idx.shape[0], _p(x_idx), _p(y)),
           "or_and_push")
    return y


def masked_or_and(m, n, row_ptr, col_idx, x_idx, visited):
    lib = _load()
    row_ptr, col_idx, x_idx = _i32(row_ptr), _i32(col_idx), _i32(x_idx)
    vis = np.ascontiguousarray(visited, dtype=np.uint8)
    y = np.empty(m, np.uint8)
    _check(lib.orc_masked_or_and(m, n, _p(row_ptr), _p(col_idx), x_idx.shape[0], _p(x_idx),
                                 _p(vis), _p(y)), "masked_or_and")
    return y


def bfs(n, col_ptr, row_idx, src):
    """Hop levels from src following y = A x (neighbours of j = rows of column j)."""
    lib = _load()
    col_ptr, row_idx = _i32(col_ptr), _i32(row_idx)
    lv = np.empty(n, np.int32)
    _check(lib.orc_bfs(n, _p(col_ptr), _p(row_idx), int(src), _p(lv)), "bfs")
    return lv


def spmspv_dense_x(m, n, row_ptr, col_idx, val, kind, x, xkind):
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    v = _vals(val, kind)
    xx = np.ascontiguousarray(x, dtype=np.float32 if xkind == F32 else np.uint16)
    y = np.empty(m, np.float64)
    s = np.empty(m, np.float64)
    _check(lib.orc_spmspv_dense_x(m, n, _p(row_ptr), _p(col_idx), _p(v), kind, _p(xx), xkind,
                                  _p(y), _p(s)), "spmspv_dense_x")
    return y, s


def threshold_activation(x, xkind, t):
    """x' with x'_j = x_j if |x_j| > t else 0 (magnitude thresholding of a
    dense activation, the decoding evaluation's activation sparsity); x of
    the value kind xkind (float32 array, or uint16 bf16 bits); t a float32."""
    lib = _load()
    xx = np.ascontiguousarray(x, dtype=np.float32 if xkind == F32 else np.uint16)
    out = np.empty_like(xx)
    _check(lib.orc_threshold_activation(xx.shape[0], _p(xx), xkind, float(np.float32(t)), _p(out)),
           "threshold_activation")
    return out


# ------------------------------------------------------------------ metadata
def xmeta(n, x_idx):
    lib = _load()
    x_idx = _i32(x_idx)
    nb = (n + 15) // 16
    masks = np.empty(nb, np.uint16)
    cnt = np.zeros(1, np.int32)
    _check(lib.orc_xmeta(n, x_idx.shape[0], _p(x_idx), _p(masks), _p(cnt)), "xmeta")
    return masks, int(cnt[0])


def xmeta_dense(n, x, xkind):
    lib = _load()
    xx = np.ascontiguousarray(x, dtype=np.float32 if xkind == F32 else np.uint16)
    nb = (n + 15) // 16
    masks = np.empty(nb, np.uint16)
    cnt = np.zeros(1, np.int32)
    _check(lib.orc_xmeta_dense(n, _p(xx), xkind, _p(masks), _p(cnt)), "xmeta_dense")
    return masks, int(cnt[0])


def select_push(n_nzblk, n_blk, th3=TH3) -> bool:
    return bool(_load().orc_select_push(int(n_nzblk), int(n_blk), float(th3)))


def classify(nnz, max_row, max_col, th0=TH0, th1=TH1, th2=TH2) -> int:
    return int(_load().orc_classify(int(nnz), int(max_row), int(max_col), int(th0), int(th1),
                                    float(th2)))


def tile_view(m, n, row_ptr, col_idx, th0=TH0, th1=TH1, th2=TH2):
    """Dict of the block-level views and per-tile statistics (see orc_tile_view)."""
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    mb, nb = (m + 15) // 16, (n + 15) // 16
    args0 = [m, n, _p(row_ptr), _p(col_idx), th0, th1, float(th2)]
    T = _check(lib.orc_tile_view(*args0, *([None] * 12)), "tile_view")
    out = {
        "rb_ptr": np.empty(mb + 1, np.int32), "t_cb": np.empty(T, np.int32),
        "t_rb": np.empty(T, np.int32), "t_nnz": np.empty(T, np.int32),
        "t_maxrow": np.empty(T, np.int32), "t_maxcol": np.empty(T, np.int32),
        "t_type": np.empty(T, np.int32), "t_rowmask": np.empty(T * 16, np.uint16),
        "t_colmask": np.empty(T * 16, np.uint16), "cb_ptr": np.empty(nb + 1, np.int32),
        "csc_rb": np.empty(T, np.int32), "csc2csr": np.empty(T, np.int32),
    }
    keys = ["rb_ptr", "t_cb", "t_rb", "t_nnz", "t_maxrow", "t_maxcol", "t_type", "t_rowmask",
            "t_colmask", "cb_ptr", "csc_rb", "csc2csr"]
    T2 = _check(lib.orc_tile_view(*args0, *[_p(out[k]) for k in keys]), "tile_view")
    assert T2 == T
    out["T"] = int(T)
    out["t_rowmask"] = out["t_rowmask"].reshape(T, 16)
    out["t_colmask"] = out["t_colmask"].reshape(T, 16)
    return out


def segments(rb_ptr, t_type, w_dense=W_DENSE, w_csr=W_CSR, w_coo=W_COO, cap=SEG_CAP):
    """(seg_rb, seg_t0, seg_t1) of the weighted pull segmentation."""
    lib = _load()
    rb_ptr, t_type = _i32(rb_ptr), _i32(t_type)
    mb = rb_ptr.shape[0] - 1
    ns = _check(lib.orc_segments(mb, _p(rb_ptr), _p(t_type), w_dense, w_csr, w_coo, cap,
                                 None, None, None), "segments")
    a, b, c = (np.empty(ns, np.int32) for _ in range(3))
    _check(lib.orc_segments(mb, _p(rb_ptr), _p(t_type), w_dense, w_csr, w_coo, cap,
                            _p(a), _p(b), _p(c)), "segments")
    return a, b, c


# ------------------------------------------------------------------ tolerance
def fp32_tolerance(s):
    """Per-entry bound |y_gpu - y| <= 1e-5 * sum|a*x| + 1e-6."""
    return 1e-5 * np.asarray(s, dtype=np.float64) + 1e-6


def within_tolerance(y_gpu, y_ref, s):
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    return err <= fp32_tolerance(s), err
