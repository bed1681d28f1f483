"""BFS levels (bit-exact) and the dense-activation decode path (fp32 tolerance)
through the C ABI vs the CPU oracle."""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import build, csr_of, mixed_tile_dense, up
from synth import (decode_activation, decode_weight_csr, largest_component_vertices, rmat_csr,
                   rng_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dbs():
    import spmspv_graph_traversal_amd as d

    return d


def gpu_bfs(dbs, A, n, src):
    import torch

    lv = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    dbs.dbs_bfs(A, int(src), lv)
    return lv.cpu().numpy()


@pytest.mark.parametrize("scale", [10, 14])
def test_bfs_rmat_all_paths(dbs, scale):
    rp, ci = rmat_csr(scale, 16, rng_for("test", 800, scale))
    n = 1 << scale
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    lcc = largest_component_vertices(rp, ci, n)
    rng = rng_for("test", 801, scale)
    srcs = list(rng.choice(lcc, 3, replace=False)) + [0]
    for src in srcs:
        ref = orc.bfs(n, rp, ci, src)
        for path in (0, 1, 2):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(gpu_bfs(dbs, A, n, src), ref, err_msg=f"src {src} path {path}")
        st = dbs.dbs_get_stats(A)
        assert st["bfs_levels"] == ref.max() + 1  # levels 0..max, the last one finds nothing
        assert st["bfs_reached"] == np.count_nonzero(ref >= 0)


def test_bfs_push_work_sources(dbs):
    """Push levels take their work chunks either from the frontier's block list
    (every call that could push has at most 6144 nonzero blocks) or from chunks
    the metadata kernel builds ahead (more possible): R-MAT 17 (8192 vertex
    blocks) with push forced, and with th3 raised to 10% and to 90%."""
    scale = 17
    rp, ci = rmat_csr(scale, 16, rng_for("test", 805, scale))
    n = 1 << scale
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    lcc = largest_component_vertices(rp, ci, n)
    src = int(rng_for("test", 806).choice(lcc))
    ref = orc.bfs(n, rp, ci, src)
    # forced push (any count possible): chunks built ahead; 10%: at most 819
    # blocks, from the list; 90%: up to 7372, chunks built ahead
    for path, num in ((1, 1), (0, 10), (0, 90)):
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        dbs.dbs_set_option(A, dbs.DBS_OPT_TH3_NUM, num)
        np.testing.assert_array_equal(gpu_bfs(dbs, A, n, src), ref, err_msg=f"path {path} th3 {num}%")
    dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TH3_NUM, 1)


def test_bfs_isolated_source_and_ragged(dbs):
    # 50 vertices (ragged last block), a path 0-1-...-9, vertex 20 isolated
    n = 50
    a = np.zeros((n, n), np.float32)
    for i in range(9):
        a[i, i + 1] = a[i + 1, i] = 1
    a[30, 49] = a[49, 30] = 1
    rp, ci, v = csr_of(a)
    for dt, vv in (("pattern", None), ("f32", v)):
        A = build(dbs, n, n, rp, ci, vv, dbs.DBS_PATTERN if vv is None else dbs.DBS_F32)
        for src in (0, 5, 20, 49):
            ref = orc.bfs(n, rp, ci, src)
            np.testing.assert_array_equal(gpu_bfs(dbs, A, n, src), ref, err_msg=f"{dt} {src}")
            # reached vertices, counted from the visited bitmap (an isolated
            # source, whose row holds no entry, counts itself)
            st = dbs.dbs_get_stats(A)
            assert st["bfs_reached"] == np.count_nonzero(ref >= 0), f"{dt} {src}"
            assert st["bfs_levels"] == ref.max() + 1


def test_bfs_directed_follows_y_equals_Ax(dbs):
    rng = rng_for("test", 810)
    n = 300
    a = (rng.random((n, n)) < 0.01).astype(np.float32)
    rp, ci, v = csr_of(a)
    cp, ri, _ = orc.csr_to_csc(n, n, rp, ci)
    A = build(dbs, n, n, rp, ci, v, dbs.DBS_F32)
    for src in (0, 17, 299):
        for path in (0, 1, 2):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(gpu_bfs(dbs, A, n, src), orc.bfs(n, cp, ri, src))


def test_bfs_directed_pattern_long_rows(dbs):
    # a directed pattern matrix whose row blocks span many pull segments (a
    # pull level reads each row block's first segment in one launch and the
    # rest in another), with rows that hold no entry and columns that do
    rng = rng_for("test", 811)
    n = 8192
    deg = np.where(rng.random(n) < 0.02, rng.integers(1000, 4000, n), rng.integers(0, 6, n))
    deg[rng.random(n) < 0.2] = 0
    rows = []
    for r in range(n):
        rows.append(np.unique(rng.integers(0, n, deg[r])))
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    ci = np.concatenate(rows).astype(np.int32)
    rp = rp.astype(np.int32)
    cp, ri, _ = orc.csr_to_csc(n, n, rp, ci)
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    st = dbs.dbs_get_stats(A)
    assert st["segments"] > n // 16  # some row blocks are split
    for src in (0, 1, 4097, n - 1):
        ref = orc.bfs(n, cp, ri, src)
        for path in (0, 1, 2):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(gpu_bfs(dbs, A, n, src), ref, err_msg=f"src {src} path {path}")


def test_bfs_mixed_formats_value_matrix(dbs):
    a = mixed_tile_dense(6, mb=8, nb=8, ragged=(0, 0))
    a = ((a != 0) | (a.T != 0)).astype(np.float32)
    rp, ci, v = csr_of(a)
    n = a.shape[0]
    A = build(dbs, n, n, rp, ci, v, dbs.DBS_F32)
    for src in (0, 33, 100):
        for path in (0, 1, 2):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(gpu_bfs(dbs, A, n, src), orc.bfs(n, rp, ci, src))


def run_dense(dbs, A, m, x_bits):
    import torch

    y = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
    dbs.dbs_spmspv_dense(A, up(np.asarray(x_bits, np.uint16).view(np.int16)), dbs.DBS_PLUS_TIMES, y)
    return y.cpu().numpy()


@pytest.mark.parametrize("shape", [(11008, 4096), (4096, 11008)])
@pytest.mark.parametrize("sparsity", [0.5, 0.7])
def test_decode_layers_full_size(dbs, shape, sparsity):
    """Single-token decode layer: bf16 weights with 50% / 70% random zeros, dense
    bf16 activation with 10 / 50 / 90% zeros, fp32 output."""
    rows, cols = shape
    rp, ci, bits = decode_weight_csr(rows, cols, sparsity, rng_for("decode", rows, int(sparsity * 10)))
    A = build(dbs, rows, cols, rp, ci, bits, dbs.DBS_BF16)
    for z in (0.1, 0.5, 0.9):
        x = decode_activation(cols, z, rng_for("decode", rows, int(sparsity * 10), int(z * 10)))
        yr, s = orc.spmspv_dense_x(rows, cols, rp, ci, bits, orc.BF16, x, orc.BF16)
        for path in (0, 1, 2):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            ok, err = orc.within_tolerance(run_dense(dbs, A, rows, x), yr, s)
            assert ok.all(), f"z={z} path {path}: max err {err.max():.3g}"
        masks, nz = orc.xmeta_dense(cols, x, orc.BF16)
        st = dbs.dbs_get_stats(A)
        assert st["last_n_nzblk"] == nz
        np.testing.assert_array_equal(dbs.dbs_copy_array(A, dbs.DBS_ARR_XMASK), masks)


def test_dense_x_signed_zero_and_f32(dbs):
    a = mixed_tile_dense(8)
    m, n = a.shape
    rp, ci, v = csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    import torch

    x = rng_for("test", 820).uniform(-1, 1, n).astype(np.float32)
    x[::3] = 0.0
    x[1::5] = -0.0
    y = torch.empty(m, dtype=torch.float32, device="cuda")
    dbs.dbs_spmspv_dense(A, up(x), dbs.DBS_PLUS_TIMES, y)
    yr, s = orc.spmspv_dense_x(m, n, rp, ci, v, orc.F32, x, orc.F32)
    ok, err = orc.within_tolerance(y.cpu().numpy(), yr, s)
    assert ok.all()
    masks, _ = orc.xmeta_dense(n, x, orc.F32)
    np.testing.assert_array_equal(dbs.dbs_copy_array(A, dbs.DBS_ARR_XMASK), masks)


def run_dense_threshold(dbs, A, m, x_t, t):
    import torch

    y = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
    dbs.dbs_spmspv_dense_threshold(A, x_t, t, dbs.DBS_PLUS_TIMES, y)
    return y.cpu().numpy()


@pytest.mark.parametrize("shape", [(11008, 4096), (4096, 11008)])
def test_decode_fused_threshold_full_size(dbs, shape):
    """Decode with the activation sparsified by magnitude in the metadata kernel:
    a dense bf16 activation without zeros, thresholds keeping ~10% and ~50% of
    it, against the oracle's thresholding followed by its dense-x product."""
    rows, cols = shape
    rp, ci, bits = decode_weight_csr(rows, cols, 0.5, rng_for("decode", rows, 5))
    A = build(dbs, rows, cols, rp, ci, bits, dbs.DBS_BF16)
    x = decode_activation(cols, 0.0, rng_for("decode", rows, 99))
    xf = np.abs(orc_bf16(x))
    x_t = up(x.view(np.int16))
    for keep in (0.1, 0.5):
        t = float(np.float32(np.quantile(xf, 1.0 - keep)))
        xs = orc.threshold_activation(x, orc.BF16, t)
        yr, s = orc.spmspv_dense_x(rows, cols, rp, ci, bits, orc.BF16, xs, orc.BF16)
        for path in (0, 1, 2):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            ok, err = orc.within_tolerance(run_dense_threshold(dbs, A, rows, x_t, t), yr, s)
            assert ok.all(), f"keep {keep} path {path}: max err {err.max():.3g}"
        masks, nz = orc.xmeta_dense(cols, xs, orc.BF16)
        assert dbs.dbs_get_stats(A)["last_n_nzblk"] == nz
        np.testing.assert_array_equal(dbs.dbs_copy_array(A, dbs.DBS_ARR_XMASK), masks)
    # x itself is not written
    np.testing.assert_array_equal(x_t.cpu().numpy().view(np.uint16), x)


def orc_bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def test_threshold_edge_cases(dbs):
    import torch

    a = mixed_tile_dense(9)
    m, n = a.shape
    rp, ci, v = csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    x = rng_for("test", 830).normal(0, 1, n).astype(np.float32)
    x[::4] = 0.0
    x[1::9] = -0.0
    x[5] = np.nan
    x_t = up(x)
    # t = 0: the plain dense rule except the NaN entry, which is dropped
    xs = orc.threshold_activation(x, orc.F32, 0.0)
    yr, s = orc.spmspv_dense_x(m, n, rp, ci, v, orc.F32, xs, orc.F32)
    ok, err = orc.within_tolerance(run_dense_threshold(dbs, A, m, x_t, 0.0), yr, s)
    assert ok.all(), f"max err {err.max():.3g}"
    # a threshold above every |x|: nothing active, y all zero
    y = run_dense_threshold(dbs, A, m, x_t, 1e30)
    assert np.array_equal(y, np.zeros(m, np.float32))
    assert dbs.dbs_get_stats(A)["last_n_nzblk"] == 0
    # thresholds that are not finite and non-negative are rejected on the host
    yt = torch.empty(m, dtype=torch.float32, device="cuda")
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(dbs.DBSError):
            dbs.dbs_spmspv_dense_threshold(A, x_t, bad, dbs.DBS_PLUS_TIMES, yt)
    # the plain dense call after a thresholded one sees its own x again
    xz = np.where(np.isnan(x), 0.0, x).astype(np.float32)
    dbs.dbs_spmspv_dense(A, up(xz), dbs.DBS_PLUS_TIMES, yt)
    yr, s = orc.spmspv_dense_x(m, n, rp, ci, v, orc.F32, xz, orc.F32)
    ok, _ = orc.within_tolerance(yt.cpu().numpy(), yr, s)
    assert ok.all()


def test_bfs_rmat22_full_size(dbs):
    """R-MAT scale 22 (edge factor 16, symmetrized), the BFS workload at full
    size: levels of every vertex, bit-exact against the oracle's queue BFS,
    for two of the sources the benchmark times (and every path for one)."""
    rp, ci = rmat_csr(22, 16, rng_for("rmat22"))
    n = 1 << 22
    lcc = largest_component_vertices(rp, ci, n)
    srcs = rng_for("rmat22", 1).choice(lcc, 64, replace=False)[:2]
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    for k, src in enumerate(srcs):
        ref = orc.bfs(n, rp, ci, int(src))
        for path in ((0, 1, 2) if k == 0 else (0,)):
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(gpu_bfs(dbs, A, n, int(src)), ref, err_msg=f"src {src} path {path}")
    dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
