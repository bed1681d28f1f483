"""Every kernel variant and every forced tile format against the CPU oracle.

* The PLUS_TIMES pull of a value matrix runs one or four segments per wave
  step, and with one segment per step two or four waves may share a segment;
  DBS_OPT_PULL_WIDTH / DBS_OPT_PULL_SHARE force each variant, so each
  instantiation of the pull kernel (f32 and bf16) meets the oracle on tiles of
  every format, including the Dense tiles the four-segment variant routes
  through the row-per-lane path.
* force_format stores every tile in one format (the format ablation of the
  DB-SpMSpV paper, Figure 10); SpMSpV (both semirings, every path) and BFS run
  on each such build.

fp32: |y - y_ref| <= 1e-5 * sum|a*x| + 1e-6 per entry; OR-AND and BFS levels:
exact.
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import bf16_csr_of, build, csr_of, mixed_tile_dense, options, up
from synth import f32_to_bf16_bits, rmat_csr, rng_for, sparse_x, uniform_csr

pytestmark = pytest.mark.gpu

PATHS = [0, 1, 2]  # auto, push, pull


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


def run_bfs(dbs, A, n, src):
    import torch

    lv = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    dbs.dbs_bfs(A, src, lv)
    return lv.cpu().numpy()


def assert_close(y, yr, s, what=""):
    ok, err = orc.within_tolerance(y, yr, s)
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} entries out of tolerance, max err {err.max():.3g}"


WIDTH_SHARE = [(1, 1), (1, 2), (1, 4), (4, 0)]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("cap", [64, 13])
def test_plus_times_pull_variants_mixed_formats(dbs, seed, cap):
    """Tiles of every format, long row blocks (split into several segments)
    and a ragged edge, through every pull variant, f32 and bf16."""
    a = mixed_tile_dense(seed, mb=4, nb=40)
    m, n = a.shape
    opt = options(dbs, seg_cap=cap)
    rp, ci, v = csr_of(a)
    _, _, bits = bf16_csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32, opt)
    B = build(dbs, m, n, rp, ci, bits, dbs.DBS_BF16, opt)
    st = dbs.dbs_get_stats(A)
    assert st["tiles_by_format"][dbs.DBS_TILE_DENSE] > 0 and st["tiles_by_format"][dbs.DBS_TILE_CSR] > 0
    for density in (0.01, 0.2, 1.0):
        xi, xv = sparse_x(n, density, rng_for("test", 900, seed, cap, int(density * 100)))
        xb = f32_to_bf16_bits(xv)
        yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
        yb, sb = orc.spmspv_pull(m, n, rp, ci, bits, orc.BF16, xi, xb, orc.BF16)
        for width, share in WIDTH_SHARE:
            for H in (A, B):
                dbs.dbs_set_option(H, dbs.DBS_OPT_PATH, 2)
                dbs.dbs_set_option(H, dbs.DBS_OPT_PULL_WIDTH, width)
                dbs.dbs_set_option(H, dbs.DBS_OPT_PULL_SHARE, share)
            what = f"density {density} width {width} share {share}"
            assert_close(run_plus(dbs, A, m, xi, xv), yr, s, "f32 " + what)
            assert_close(run_plus(dbs, B, m, xi, xb, bf16=True), yb, sb, "bf16 " + what)


def test_pull_variant_options_are_validated(dbs):
    a = mixed_tile_dense(0)
    rp, ci, v = csr_of(a)
    A = build(dbs, a.shape[0], a.shape[1], rp, ci, v, dbs.DBS_F32)
    for opt, bad in ((dbs.DBS_OPT_PULL_WIDTH, 2), (dbs.DBS_OPT_PULL_WIDTH, -1), (dbs.DBS_OPT_PULL_SHARE, 3),
                     (dbs.DBS_OPT_PULL_SHARE, 8)):
        with pytest.raises(dbs.DBSError):
            dbs.dbs_set_option(A, opt, bad)
    dbs.dbs_set_option(A, dbs.DBS_OPT_PULL_WIDTH, 4)
    assert dbs.dbs_get_option(A, dbs.DBS_OPT_PULL_WIDTH) == 4


# (rows, columns, entries per row): column-block counts 1, 5, 63, 4099,
# 65537, 196608 (the most whose active-block bits the Boolean pull stages in
# LDS) and 196609 (one more: every tile reads its mask word)
OR_SHAPES = [(40, 9, 3), (77, 80, 6), (300, 1000, 9), (700, 65584, 12), (500, (1 << 20) + 16, 20),
             (300, 196608 * 16, 12), (300, 196609 * 16, 12)]


@pytest.mark.parametrize("shape", OR_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_or_and_shapes(dbs, shape):
    """OR-AND on pattern matrices of uniform rows: equal to the oracle on
    every path, at densities that push, pull with the metadata of the active
    tiles only and pull with every tile's metadata, over consecutive calls."""
    m, n, per = shape
    rp, ci, _ = uniform_csr(m, n, per, rng_for("test", 920, m, n))
    P = build(dbs, m, n, rp, ci, None, dbs.DBS_PATTERN)
    for k, density in enumerate((0.0005, 0.02, 0.3, 0.9)):
        xi, _ = sparse_x(n, density, rng_for("test", 921, n, k), with_values=False)
        if xi.size == 0:
            xi = np.array([n // 2], np.int32)
        yo = orc.or_and_pull(m, n, rp, ci, xi)
        for path in PATHS:
            dbs.dbs_set_option(P, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(run_or(dbs, P, m, xi), yo, err_msg=f"density {density} path {path}")


def test_or_and_rmat_sweep(dbs):
    """R-MAT pattern (packed multi-row-block segments, long row blocks split
    over segments): every path equals the oracle over a density sweep."""
    rp, ci = rmat_csr(13, 16, rng_for("test", 922))[:2]
    n = rp.shape[0] - 1
    P = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    for k, density in enumerate((0.0001, 0.001, 0.01, 0.1, 0.5)):
        xi, _ = sparse_x(n, density, rng_for("test", 923, k), with_values=False)
        yo = orc.or_and_pull(n, n, rp, ci, xi)
        for path in PATHS:
            dbs.dbs_set_option(P, dbs.DBS_OPT_PATH, path)
            np.testing.assert_array_equal(run_or(dbs, P, n, xi), yo, err_msg=f"density {density} path {path}")


@pytest.mark.parametrize("force", [0, 1, 2, 3, 4])
def test_forced_format_spmspv_and_bfs(dbs, force):
    """Every tile stored in one format, value (f32, bf16) and pattern builds:
    PLUS_TIMES and OR-AND on every path, and BFS levels on every path."""
    a = mixed_tile_dense(force, mb=6, nb=6, ragged=(9, 9))
    a = np.where((a != 0) | (a.T != 0), np.where(a != 0, a, 0.25), 0).astype(np.float32)  # symmetric pattern
    n = a.shape[0]
    opt = options(dbs, force_format=force)
    rp, ci, v = csr_of(a)
    _, _, bits = bf16_csr_of(a)
    A = build(dbs, n, n, rp, ci, v, dbs.DBS_F32, opt)
    B = build(dbs, n, n, rp, ci, bits, dbs.DBS_BF16, opt)
    P = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN, opt)
    for H in (A, B, P):
        st = dbs.dbs_get_stats(H)
        assert st["tiles_by_format"][force] == st["tiles"]
    for k, density in enumerate((0.005, 0.1, 0.7)):
        xi, xv = sparse_x(n, density, rng_for("test", 910, force, k))
        xb = f32_to_bf16_bits(xv)
        yr, s = orc.spmspv_pull(n, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
        yb, sb = orc.spmspv_pull(n, n, rp, ci, bits, orc.BF16, xi, xb, orc.BF16)
        yo = orc.or_and_pull(n, n, rp, ci, xi)
        for path in PATHS:
            for H in (A, B, P):
                dbs.dbs_set_option(H, dbs.DBS_OPT_PATH, path)
            what = f"force {force} density {density} path {path}"
            assert_close(run_plus(dbs, A, n, xi, xv), yr, s, "f32 " + what)
            assert_close(run_plus(dbs, B, n, xi, xb, bf16=True), yb, sb, "bf16 " + what)
            for H in (A, B, P):
                np.testing.assert_array_equal(run_or(dbs, H, n, xi), yo, err_msg="or-and " + what)
    for src in (0, 40, n - 1):
        ref = orc.bfs(n, rp, ci, src)
        for path in PATHS:
            for H in (A, B, P):
                dbs.dbs_set_option(H, dbs.DBS_OPT_PATH, path)
                np.testing.assert_array_equal(run_bfs(dbs, H, n, src), ref, err_msg=f"bfs src {src} path {path}")


@pytest.mark.parametrize("cap", [3, 5, 9])
def test_plus_times_partial_slots_and_finalize(dbs, cap):
    """Row blocks of 150 tiles of mixed formats split into many pull segments
    (with cap 3 50 to 75 per row block, class 3; cap 5 50, class 2; cap 9 25,
    class 1): their row sums go to partial slots, summed by the finalize,
    whenever segments x sharing waves exceeds 64.  Consecutive
    calls activate different column ranges, so segments that wrote a slot in
    one call have nothing to add in the next: their slots must count as zero
    (they carry the writing call's epoch).  f32 and bf16, every pull width
    and sharing, the finalize's result against the oracle."""
    a = mixed_tile_dense(2, mb=3, nb=150, ragged=(5, 3))
    m, n = a.shape
    opt = options(dbs, seg_cap=cap)
    rp, ci, v = csr_of(a)
    _, _, bits = bf16_csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32, opt)
    B = build(dbs, m, n, rp, ci, bits, dbs.DBS_BF16, opt)
    segs = dbs.dbs_copy_array(A, dbs.DBS_ARR_SEGMENTS).reshape(-1, 4)
    per_rb = np.bincount(segs[:, 0] & 0x0FFFFFFF)
    assert per_rb.max() > (64 if cap == 3 else 16)
    rng = rng_for("test", 920, cap)
    calls = []
    for k in range(4):
        lo, hi = [(0, n), (0, n // 3), (n // 2, n), (n // 4, n // 4 + 40)][k]
        xi = np.sort(rng.choice(np.arange(lo, hi), size=max(1, (hi - lo) // 5), replace=False)).astype(np.int32)
        xv = rng.uniform(-1, 1, xi.shape[0]).astype(np.float32)
        calls.append((xi, xv))
    for width, share in WIDTH_SHARE:
        for H in (A, B):
            dbs.dbs_set_option(H, dbs.DBS_OPT_PATH, 2)
            dbs.dbs_set_option(H, dbs.DBS_OPT_PULL_WIDTH, width)
            dbs.dbs_set_option(H, dbs.DBS_OPT_PULL_SHARE, share)
        for k, (xi, xv) in enumerate(calls):
            xb = f32_to_bf16_bits(xv)
            yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
            yb, sb = orc.spmspv_pull(m, n, rp, ci, bits, orc.BF16, xi, xb, orc.BF16)
            what = f"call {k} width {width} share {share}"
            assert_close(run_plus(dbs, A, m, xi, xv), yr, s, "f32 " + what)
            assert_close(run_plus(dbs, B, m, xi, xb, bf16=True), yb, sb, "bf16 " + what)


def test_plus_times_hub_row_drained_segments(dbs):
    """A row with an entry in every column, in COO tiles: its pull segments
    hold up to 1024 of its entries (marked segments, whose LDS row sums are
    emptied after every round in the wide pull).  Every pull variant against
    the oracle, sparse and full x."""
    from test_gpu_format import hub_row_dense

    a = hub_row_dense(1)
    m, n = a.shape
    rp, ci, v = csr_of(a)
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    for k, density in enumerate((0.05, 1.0)):
        xi, xv = sparse_x(n, density, rng_for("test", 930, k))
        yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
        for width, share in WIDTH_SHARE:
            dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, 2)
            dbs.dbs_set_option(A, dbs.DBS_OPT_PULL_WIDTH, width)
            dbs.dbs_set_option(A, dbs.DBS_OPT_PULL_SHARE, share)
            assert_close(run_plus(dbs, A, m, xi, xv), yr, s, f"density {density} width {width} share {share}")
