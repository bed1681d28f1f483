"""SpMSpV through the C ABI vs the CPU oracle.

fp32 results: |y - y_ref| <= 1e-5 * sum|a*x| + 1e-6 per entry; OR-AND results,
vector metadata and the path choice: exact.
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import bf16_csr_of, build, csr_of, mixed_tile_dense, options, up
from synth import (bf16_bits_to_f32, f32_to_bf16_bits, permute_vertices, rmat_csr, rng_for, sparse_x,
                   uniform_csr)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dbs():
    import spmspv_graph_traversal_amd as d

    return d


def run_plus(dbs, A, m, xi, xv, bf16=False):
    import torch

    y = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
    xv_t = up(np.asarray(xv, np.uint16).view(np.int16)) if bf16 else up(np.asarray(xv, np.float32))
    dbs.dbs_spmspv(A, up(np.asarray(xi, np.int32)), xv_t, dbs.DBS_PLUS_TIMES, y)
    return y.cpu().numpy()


def run_or(dbs, A, m, xi):
    import torch

    y = torch.full((m,), 7, dtype=torch.uint8, device="cuda")
    dbs.dbs_spmspv(A, up(np.asarray(xi, np.int32)), None, dbs.DBS_OR_AND, y)
    return y.cpu().numpy()


def assert_close(y, yr, s, what=""):
    ok, err = orc.within_tolerance(y, yr, s)
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} entries out of tolerance, max err {err.max():.3g}"


PATHS = [0, 1, 2]  # auto, push, pull


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("density", [0.0, 0.004, 0.05, 0.3, 1.0])
def test_plus_times_mixed_formats_all_paths(dbs, seed, density):
    a = mixed_tile_dense(seed)
    m, n = a.shape
    rp, ci, v = csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    xi, xv = sparse_x(n, density, rng_for("test", 700, seed, int(density * 1000)))
    yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
    for path in PATHS:
        for cutoff in (0, 8, 17):  # patched-CSR: always row kernel (default) / mixed / always column kernel
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            dbs.dbs_set_option(A, dbs.DBS_OPT_LOCAL_PUSH_CUTOFF, cutoff)
            y = run_plus(dbs, A, m, xi, xv)
            assert_close(y, yr, s, f"path {path} cutoff {cutoff}")
            assert np.all(y[s == 0] == 0)


@pytest.mark.parametrize("density", [0.003, 0.05, 0.5])
def test_plus_times_bf16(dbs, density):
    a = mixed_tile_dense(5, mb=7, nb=9)
    m, n = a.shape
    rp, ci, bits = bf16_csr_of(a)
    A = build(dbs, m, n, rp, ci, bits, dbs.DBS_BF16)
    rng = rng_for("test", 710, int(density * 1000))
    xi, xv = sparse_x(n, density, rng)
    xb = f32_to_bf16_bits(xv)
    yr, s = orc.spmspv_pull(m, n, rp, ci, bits, orc.BF16, xi, xb, orc.BF16)
    for path in PATHS:
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        assert_close(run_plus(dbs, A, m, xi, xb, bf16=True), yr, s, f"bf16 path {path}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("cap", [64, 45, 13])
def test_plus_times_long_row_blocks(dbs, seed, cap):
    """Row blocks of 75 tiles split into pull segments of up to `cap` weight: the
    larger tiles go through the four-tiles-per-step path with partial last steps
    whose tiles sit in lanes of any quarter.  f32 and bf16, sparse and dense x."""
    a = mixed_tile_dense(seed, mb=3, nb=75)
    m, n = a.shape
    opt = options(dbs, seg_cap=cap)
    rp, ci, v = csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32, opt)
    _, _, bits = bf16_csr_of(a)
    B = build(dbs, m, n, rp, ci, bits, dbs.DBS_BF16, opt)
    for density in (0.05, 0.6, 1.0):
        xi, xv = sparse_x(n, density, rng_for("test", 720, seed, cap, int(density * 100)))
        xb = f32_to_bf16_bits(xv)
        yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
        yb, sb = orc.spmspv_pull(m, n, rp, ci, bits, orc.BF16, xi, xb, orc.BF16)
        for path in PATHS:
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            dbs.dbs_set_option(B, dbs.DBS_OPT_PATH, path)
            assert_close(run_plus(dbs, A, m, xi, xv), yr, s, f"f32 path {path} density {density}")
            assert_close(run_plus(dbs, B, m, xi, xb, bf16=True), yb, sb, f"bf16 path {path} density {density}")


def test_tiny_config_full_size(dbs):
    """4096 x 4096, 16 uniform columns per row, x with 1% entries."""
    rp, ci, v = uniform_csr(4096, 4096, 16, rng_for("tiny"))
    A = build(dbs, 4096, 4096, rp, ci, v, dbs.DBS_F32)
    xi, xv = sparse_x(4096, 0.01, rng_for("tiny", 1))
    yr, s = orc.spmspv_pull(4096, 4096, rp, ci, v, orc.F32, xi, xv, orc.F32)
    cp, ri, cv = orc.csr_to_csc(4096, 4096, rp, ci, v, orc.F32)
    yr2, _ = orc.spmspv_push(4096, 4096, cp, ri, cv, orc.F32, xi, xv, orc.F32)
    np.testing.assert_allclose(yr, yr2, rtol=1e-12, atol=1e-14)
    for path in PATHS:
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        assert_close(run_plus(dbs, A, 4096, xi, xv), yr, s, f"path {path}")
        st = dbs.dbs_get_stats(A)
        masks, nz = orc.xmeta(4096, xi)
        assert st["last_n_nzblk"] == nz
        exp_push = orc.select_push(nz, 256) if path == 0 else path == 1
        assert st["last_path"] == (0 if exp_push else 1)
        np.testing.assert_array_equal(dbs.dbs_copy_array(A, dbs.DBS_ARR_XMASK), masks)
        act = np.sort(dbs.dbs_copy_array(A, dbs.DBS_ARR_ACTIVE))
        np.testing.assert_array_equal(act, np.nonzero(masks)[0])


@pytest.mark.parametrize("density", [0.0001, 0.001, 0.01, 0.1, 0.5])
def test_or_and_rmat(dbs, density):
    rp, ci = rmat_csr(13, 16, rng_for("test", 720))
    n = 1 << 13
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    xi, _ = sparse_x(n, density, rng_for("test", 721, int(density * 1e4)), with_values=False)
    yr = orc.or_and_pull(n, n, rp, ci, xi)
    for path in PATHS:
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        np.testing.assert_array_equal(run_or(dbs, A, n, xi), yr, err_msg=f"path {path}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "pattern"])
def test_or_and_mixed_formats_counts_stored_zeros(dbs, dtype):
    a = mixed_tile_dense(2)
    m, n = a.shape
    rp, ci, v = csr_of(a)
    v = v.copy()
    v[::7] = 0.0  # explicitly stored zeros are structural entries
    if dtype == "f32":
        A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    elif dtype == "bf16":
        A = build(dbs, m, n, rp, ci, f32_to_bf16_bits(v), dbs.DBS_BF16)
    else:
        A = build(dbs, m, n, rp, ci, None, dbs.DBS_PATTERN)
    for k, density in enumerate([0.003, 0.04, 0.3, 1.0]):
        xi, _ = sparse_x(n, density, rng_for("test", 730, k), with_values=False)
        yr = orc.or_and_pull(m, n, rp, ci, xi)
        for path in PATHS:
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(run_or(dbs, A, m, xi), yr, err_msg=f"{dtype} path {path}")


def test_invalid_x_indices_contribute_nothing(dbs):
    a = mixed_tile_dense(1)
    m, n = a.shape
    rp, ci, v = csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    xi = np.array([-7, -1, 3, 17, 40, n - 1, n, n + 5], np.int32)
    xv = np.linspace(-1, 1, xi.shape[0]).astype(np.float32)
    yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
    for path in PATHS:
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        assert_close(run_plus(dbs, A, m, xi, xv), yr, s, f"path {path}")
        np.testing.assert_array_equal(run_or(dbs, A, m, xi), orc.or_and_pull(m, n, rp, ci, xi))


def test_empty_x_and_repeated_calls(dbs):
    rp, ci, v = uniform_csr(500, 700, 9, rng_for("test", 740))
    A = build(dbs, 500, 700, rp, ci, v, dbs.DBS_F32)
    y = run_plus(dbs, A, 500, np.zeros(0, np.int32), np.zeros(0, np.float32))
    assert np.all(y == 0)
    # masks of an earlier call never leak into a later one
    rng = rng_for("test", 741)
    for it in range(6):
        xi, xv = sparse_x(700, [0.3, 0.002, 0.05, 0.0, 1.0, 0.01][it], rng)
        yr, s = orc.spmspv_pull(500, 700, rp, ci, v, orc.F32, xi, xv, orc.F32)
        assert_close(run_plus(dbs, A, 500, xi, xv), yr, s, f"call {it}")
        masks, _ = orc.xmeta(700, xi)
        np.testing.assert_array_equal(dbs.dbs_copy_array(A, dbs.DBS_ARR_XMASK), masks)


def test_selector_threshold_and_option(dbs):
    # N_blk = 6400 / 16 = 400: push iff 100 * N_nzblk < 400, i.e. N_nzblk <= 3
    rp, ci, v = uniform_csr(300, 6400, 5, rng_for("test", 750))
    A = build(dbs, 300, 6400, rp, ci, v, dbs.DBS_F32)
    for nblk, exp in [(1, 0), (3, 0), (4, 1), (40, 1)]:
        xi = (np.arange(nblk) * 16 * 7 + 3).astype(np.int32)
        xv = np.ones(nblk, np.float32)
        run_plus(dbs, A, 300, xi, xv)
        st = dbs.dbs_get_stats(A)
        assert st["last_n_nzblk"] == nblk and st["last_path"] == exp
    dbs.dbs_set_option(A, dbs.DBS_OPT_TH3_NUM, 1)
    dbs.dbs_set_option(A, dbs.DBS_OPT_TH3_DEN, 10)  # th3 = 0.1
    run_plus(dbs, A, 300, (np.arange(39) * 16).astype(np.int32), np.ones(39, np.float32))
    assert dbs.dbs_get_stats(A)["last_path"] == 0


def test_check_mode_flags_unsorted_x(dbs):
    rp, ci, v = uniform_csr(100, 100, 4, rng_for("test", 760))
    A = build(dbs, 100, 100, rp, ci, v, dbs.DBS_F32)
    dbs.dbs_set_option(A, dbs.DBS_OPT_CHECK, 1)
    run_plus(dbs, A, 100, np.array([5, 3, 9], np.int32), np.ones(3, np.float32))
    st = dbs.dbs_get_stats(A, allow_bad_vector=True)
    assert st["status"] == dbs.DBS_ERR_BAD_VECTOR
    run_plus(dbs, A, 100, np.array([3, 5, 9], np.int32), np.ones(3, np.float32))
    assert dbs.dbs_get_stats(A)["status"] == dbs.DBS_OK


def test_argument_errors(dbs):
    import torch

    rp, ci, v = uniform_csr(64, 64, 3, rng_for("test", 770))
    A = build(dbs, 64, 64, rp, ci, v, dbs.DBS_F32)
    P = build(dbs, 64, 64, rp, ci, None, dbs.DBS_PATTERN)
    y = torch.zeros(64, dtype=torch.float32, device="cuda")
    xi = up(np.array([1, 2], np.int32))
    xv = up(np.ones(2, np.float32))
    lib = dbs.binding._lib
    # plus-times on a pattern matrix
    assert lib.dbs_spmspv(P.handle, 2, xi.data_ptr(), xv.data_ptr(), dbs.DBS_PLUS_TIMES, y.data_ptr(),
                          None) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_spmspv(A.handle, 65, None, None, 0, None, None) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_spmspv(A.handle, 2, xi.data_ptr(), None, 0, y.data_ptr(), None) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_spmspv(None, 0, None, None, 0, y.data_ptr(), None) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_spmspv(A.handle, 0, None, None, 5, y.data_ptr(), None) == dbs.DBS_ERR_INVALID_ARG
    rect = build(dbs, 64, 80, rp, ci, v, dbs.DBS_F32)
    lv = torch.zeros(64, dtype=torch.int32, device="cuda")
    assert lib.dbs_bfs(rect.handle, 0, lv.data_ptr(), None) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_bfs(A.handle, 64, lv.data_ptr(), None) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_set_option(A.handle, 99, 0) == dbs.DBS_ERR_INVALID_ARG
    assert lib.dbs_set_option(A.handle, dbs.DBS_OPT_PATH, 3) == dbs.DBS_ERR_INVALID_ARG
    # a pull segment holds at most one tile per lane
    for cap, dt, vals in ((-1, dbs.DBS_F32, v), (65, dbs.DBS_F32, v), (257, dbs.DBS_PATTERN, None)):
        with pytest.raises(dbs.DBSError) as e:
            build(dbs, 64, 64, rp, ci, vals, dt, options(dbs, seg_cap=cap))
        assert e.value.status == dbs.DBS_ERR_INVALID_ARG
    build(dbs, 64, 64, rp, ci, None, dbs.DBS_PATTERN, options(dbs, seg_cap=256))


def clustered_pattern_csr(n, seed):
    """Rows whose entries fall in a few 16-column windows: most tiles hold 5-30
    entries (their coordinates are payload words), short and long row blocks mixed."""
    rng = rng_for("test", 760, seed)
    rows = []
    for r in range(n):
        k = int(rng.integers(0, 5)) if r % 97 else int(rng.integers(40, 200))
        wins = rng.integers(0, n // 16, k)
        cols = (wins[:, None] * 16 + rng.integers(0, 16, (k, 12))).ravel()
        rows.append(np.unique(cols))
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    return rp.astype(np.int32), np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("cap", [256, 100, 17])
def test_or_and_pattern_coordinate_words(dbs, cap):
    n = 12000  # ragged last block
    rp, ci = clustered_pattern_csr(n, cap)
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN, options(dbs, seg_cap=cap))
    for k, density in enumerate([0.001, 0.02, 0.3]):
        xi, _ = sparse_x(n, density, rng_for("test", 761, cap, k), with_values=False)
        yr = orc.or_and_pull(n, n, rp, ci, xi)
        for path in PATHS:
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(run_or(dbs, A, n, xi), yr, err_msg=f"density {density} path {path}")


def test_rmat20_or_and_sweep_full_size(dbs):
    """R-MAT scale 20 (edge factor 16, symmetrized), OR-AND, the density sweep."""
    rp, ci = rmat_csr(20, 16, rng_for("rmat20"))
    n = 1 << 20
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    for k, density in enumerate([0.0001, 0.001, 0.01, 0.1, 0.5]):
        xi, _ = sparse_x(n, density, rng_for("rmat20", 1, k), with_values=False)
        yr = orc.or_and_pull(n, n, rp, ci, xi)
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
        np.testing.assert_array_equal(run_or(dbs, A, n, xi), yr, err_msg=f"density {density}")
        st = dbs.dbs_get_stats(A)
        _, nz = orc.xmeta(n, xi)
        assert st["last_n_nzblk"] == nz
        assert st["last_path"] == (0 if orc.select_push(nz, n // 16) else 1)
        if density <= 0.01:
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 1)
            np.testing.assert_array_equal(run_or(dbs, A, n, xi), yr, err_msg=f"push {density}")


def test_rmat20_permuted_or_and_sweep_full_size(dbs):
    """The R-MAT 20 graph with its vertices relabelled at random (about one
    entry per tile), OR-AND, the density sweep with the inputs the benchmark
    times; both paths forced at every density against the oracle."""
    rp, ci = permute_vertices(*rmat_csr(20, 16, rng_for("rmat20")), rng_for("rmat20", 2))
    n = 1 << 20
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    st = dbs.dbs_get_stats(A)
    assert st["tiles"] > 1.4 * 19_000_000  # the relabelled graph's tiles hold ~1 entry each
    for k, density in enumerate([0.0001, 0.001, 0.01, 0.1, 0.5]):
        xi, _ = sparse_x(n, density, rng_for("rmat20", 3, k), with_values=False)
        yr = orc.or_and_pull(n, n, rp, ci, xi)
        for path in PATHS:
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(run_or(dbs, A, n, xi), yr, err_msg=f"density {density} path {path}")
        _, nz = orc.xmeta(n, xi)
        assert dbs.dbs_get_stats(A)["last_n_nzblk"] == nz
    dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)


@pytest.mark.parametrize("kind", ["alternating", "permuted"])
def test_unsorted_x_is_memory_safe(dbs, kind):
    """An x_idx that is not strictly increasing registers a block once per
    leader (an entry whose predecessor is in another block): up to 16 nb
    entries for nb list slots.  Every consumer clamps the count to nb, and a
    push that enumerates its chunks from the list stays within the LDS prefix
    array.  With nb = 6144 a forced push enumerates from the list and the raw
    count reaches 16 nb = 98,304.  y is unspecified for such input: the calls
    must return, report at most nb blocks and export at most nb of them, and
    the next (sorted) call must be exact."""
    n, m = 6144 * 16, 3000
    rp, ci, v = uniform_csr(m, n, 6, rng_for("test", 780))
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    P = build(dbs, m, n, rp, ci, None, dbs.DBS_PATTERN)
    if kind == "alternating":
        bad = np.tile(np.array([0, 16], np.int32), n // 2)
    else:
        bad = rng_for("test", 781).permutation(n).astype(np.int32)
    bv = np.ones(bad.shape[0], np.float32)
    good, gv = sparse_x(n, 0.0005, rng_for("test", 782))
    yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, good, gv, orc.F32)
    yb = orc.or_and_pull(m, n, rp, ci, good)
    for path in PATHS:
        for H in (A, P):
            dbs.dbs_set_option(H, dbs.DBS_OPT_PATH, path)
        run_plus(dbs, A, m, bad, bv)
        st = dbs.dbs_get_stats(A)
        assert 0 <= st["last_n_nzblk"] <= n // 16
        assert dbs.dbs_copy_array(A, dbs.DBS_ARR_ACTIVE).shape[0] <= n // 16
        run_or(dbs, P, m, bad)
        st = dbs.dbs_get_stats(P)
        assert 0 <= st["last_n_nzblk"] <= n // 16
        assert_close(run_plus(dbs, A, m, good, gv), yr, s, f"sorted call after unsorted, path {path}")
        np.testing.assert_array_equal(run_or(dbs, P, m, good), yb, err_msg=f"path {path}")


@pytest.mark.parametrize("n,nblocks", [(1 << 16, 3000), (1 << 21, 90000)])
def test_sparse_masks_runs_across_waves(dbs, n, nblocks):
    """Block masks of a sparse x whose blocks hold 1 to 16 entries, so that a
    block's run of entries starts at every lane offset and crosses the 64-entry
    boundaries of the metadata kernel's waves; the larger case gives every
    workgroup several rounds.  Masks, N_nzblk and the OR-AND product against
    the oracle."""
    rng = rng_for("test", 790, n)
    blocks = np.sort(rng.choice(n // 16, nblocks, replace=False))
    parts = []
    for b in blocks:
        k = int(rng.integers(1, 17))
        parts.append(16 * b + np.sort(rng.choice(16, k, replace=False)))
    xi = np.concatenate(parts).astype(np.int32)
    rp, ci = rmat_csr(int(np.log2(n)), 2, rng_for("test", 791, n))
    A = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    dbs.dbs_set_option(A, dbs.DBS_OPT_CHECK, 1)
    import torch

    y = torch.empty(n, dtype=torch.uint8, device="cuda")
    dbs.dbs_spmspv(A, up(xi), None, dbs.DBS_OR_AND, y)
    st = dbs.dbs_get_stats(A)
    masks, nz = orc.xmeta(n, xi)
    assert st["last_n_nzblk"] == nz
    np.testing.assert_array_equal(dbs.dbs_copy_array(A, dbs.DBS_ARR_XMASK), masks)
    np.testing.assert_array_equal(y.cpu().numpy(), orc.or_and_pull(n, n, rp, ci, xi))


def test_widest_x_the_offsets_allow(dbs):
    """x block-padded to the last byte the 32-bit buffer offsets reach: an f32
    matrix of 1,073,741,808 columns multiplies correctly (entries in the last
    columns, so the largest offsets are used); one of 2^30 columns is refused
    for PLUS_TIMES and still takes OR-AND."""
    import gc

    import torch

    m = 40
    for n, plus_ok in ((1073741808, True), (1 << 30, False)):
        cols = np.array([0, 17, n // 2, n - 17, n - 2, n - 1], np.int64)
        rows = [3, 3, 10, 10, 39, 39]
        rp = np.zeros(m + 1, np.int32)
        for r in rows:
            rp[r + 1:] += 1
        ci = cols.astype(np.int32)
        v = rng_for("test", 795).uniform(-1, 1, ci.shape[0]).astype(np.float32)
        A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
        xi = np.array([17, n // 2, n - 2, n - 1], np.int32)
        xv = np.array([0.5, -2.0, 1.5, 3.0], np.float32)
        if plus_ok:
            for path in PATHS:
                dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
                yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
                assert_close(run_plus(dbs, A, m, xi, xv), yr, s, f"n={n} path {path}")
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 0)
        else:
            y = torch.empty(m, dtype=torch.float32, device="cuda")
            with pytest.raises(dbs.DBSError) as e:
                dbs.dbs_spmspv(A, up(xi), up(xv), dbs.DBS_PLUS_TIMES, y)
            assert e.value.status == dbs.DBS_ERR_UNSUPPORTED
        yb = torch.empty(m, dtype=torch.uint8, device="cuda")
        dbs.dbs_spmspv(A, up(xi), None, dbs.DBS_OR_AND, yb)
        np.testing.assert_array_equal(yb.cpu().numpy(), orc.or_and_pull(m, n, rp, ci, xi))
        del A
        gc.collect()
        torch.cuda.synchronize()
