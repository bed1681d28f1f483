"""Pins of the CPU oracle against things other than itself (CPU only).

Each check compares the oracle with an independent computation: numpy dense
products, scipy.sparse, scipy.sparse.csgraph, invariants of BFS levels, the
worked examples of the paper (tests/golden/*), or the push/pull pair.
"""
import os

import numpy as np
import pytest
import scipy.sparse as sp
from scipy.sparse.csgraph import shortest_path

import oracle as orc
from synth import (bf16_bits_to_f32, csr_from_dense, f32_to_bf16_bits, rmat_csr, rng_for,
                   uniform_csr)


def _rand_sparse_dense(rng, m, n, density, empty_rows=(), empty_cols=()):
    a = np.where(rng.random((m, n)) < density, rng.uniform(-1, 1, (m, n)), 0.0).astype(np.float32)
    for r in empty_rows:
        a[r, :] = 0
    for c in empty_cols:
        a[:, c] = 0
    return a


SHAPES = [(1, 1), (5, 7), (16, 16), (17, 33), (48, 48), (64, 40), (63, 65)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("xdens", [0.0, 0.05, 0.3, 1.0])
def test_pull_matches_dense_product(shape, xdens):
    m, n = shape
    rng = rng_for("test", m, n, int(xdens * 100))
    a = _rand_sparse_dense(rng, m, n, 0.3, empty_rows=(0,) if m > 2 else (), empty_cols=(n - 1,) if n > 2 else ())
    rp, ci, v = csr_from_dense(a)
    k = int(round(xdens * n))
    xi = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
    xv = rng.uniform(-1, 1, k).astype(np.float32)
    xd = np.zeros(n, np.float64)
    xd[xi] = xv
    y, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
    ref = a.astype(np.float64) @ xd
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, np.abs(a.astype(np.float64)) @ np.abs(xd), rtol=1e-12, atol=1e-12)


def test_pull_matches_scipy_and_push_matches_pull():
    rng = rng_for("test", 1)
    m, n = 300, 257
    rp, ci, v = uniform_csr(m, n, 9, rng)
    xi = np.sort(rng.choice(n, 40, replace=False)).astype(np.int32)
    xv = rng.uniform(-1, 1, 40).astype(np.float32)
    A = sp.csr_matrix((v.astype(np.float64), ci, rp), shape=(m, n))
    xd = np.zeros(n)
    xd[xi] = xv
    y, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
    np.testing.assert_allclose(y, A @ xd, rtol=1e-12, atol=1e-13)
    cp, ri, cv = orc.csr_to_csc(m, n, rp, ci, v, orc.F32)
    y2, s2 = orc.spmspv_push(m, n, cp, ri, cv, orc.F32, xi, xv, orc.F32)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s2, s, rtol=1e-12, atol=1e-14)


def test_csc_transpose_matches_scipy():
    rng = rng_for("test", 2)
    a = _rand_sparse_dense(rng, 40, 35, 0.2)
    rp, ci, v = csr_from_dense(a)
    cp, ri, cv = orc.csr_to_csc(40, 35, rp, ci, v, orc.F32)
    B = sp.csr_matrix(a).tocsc()
    B.sort_indices()
    np.testing.assert_array_equal(cp, B.indptr)
    np.testing.assert_array_equal(ri, B.indices)
    np.testing.assert_array_equal(cv, B.data.astype(np.float32))


def test_bf16_values_widen_exactly():
    rng = rng_for("test", 3)
    a = _rand_sparse_dense(rng, 20, 24, 0.4)
    bits = f32_to_bf16_bits(a)
    a16 = bf16_bits_to_f32(bits).reshape(a.shape)
    rp, ci, _ = csr_from_dense(a16)
    vb = bits.reshape(a.shape)[np.nonzero(a16)]
    xi = np.arange(0, 24, 3, dtype=np.int32)
    xb = f32_to_bf16_bits(rng.uniform(-1, 1, xi.shape[0]).astype(np.float32))
    y, _ = orc.spmspv_pull(20, 24, rp, ci, vb, orc.BF16, xi, xb, orc.BF16)
    xd = np.zeros(24)
    xd[xi] = bf16_bits_to_f32(xb)
    np.testing.assert_allclose(y, a16.astype(np.float64) @ xd, rtol=1e-13, atol=1e-15)


def test_bf16_rounding_is_nearest_even():
    # bf16 keeps 7 explicit mantissa bits (ulp 2**-7 at 1.0); ties go to the even mantissa
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 2**-7 + 2**-8, 1.0 + 3 * 2**-9, 1.0 + 2**-9], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, 1.0], np.float32))


def test_invalid_x_index_contributes_nothing():
    a = np.arange(1, 13, dtype=np.float32).reshape(3, 4)
    rp, ci, v = csr_from_dense(a)
    xi = np.array([-5, 1, 4, 99], np.int32)
    xv = np.array([7.0, 2.0, 7.0, 7.0], np.float32)
    y, _ = orc.spmspv_pull(3, 4, rp, ci, v, orc.F32, xi, xv, orc.F32)
    np.testing.assert_array_equal(y, a[:, 1] * 2.0)


@pytest.mark.parametrize("seed", range(4))
def test_or_and_matches_boolean_product(seed):
    rng = rng_for("test", 10, seed)
    m, n = 50 + seed, 45 + 2 * seed
    a = _rand_sparse_dense(rng, m, n, 0.08)
    a[3, 5] = 0.0
    rp, ci, _ = csr_from_dense(a)
    # an explicitly stored zero is structurally present (counts for OR-AND)
    rp2, ci2 = rp.copy(), ci.copy()
    xi = np.sort(rng.choice(n, 6, replace=False)).astype(np.int32)
    ref = ((a != 0).astype(np.int64) @ np.isin(np.arange(n), xi).astype(np.int64)) > 0
    y = orc.or_and_pull(m, n, rp2, ci2, xi)
    np.testing.assert_array_equal(y.astype(bool), ref)
    cp, ri, _ = orc.csr_to_csc(m, n, rp2, ci2)
    np.testing.assert_array_equal(orc.or_and_push(m, n, cp, ri, xi), y)
    vis = (rng.random(m) < 0.5).astype(np.uint8)
    np.testing.assert_array_equal(orc.masked_or_and(m, n, rp2, ci2, xi, vis).astype(bool), ref & (vis == 0))


def test_or_and_counts_stored_zero():
    rp = np.array([0, 1], np.int32)
    ci = np.array([2], np.int32)
    y = orc.or_and_pull(1, 4, rp, ci, np.array([2], np.int32))
    assert y[0] == 1
    y0, _ = orc.spmspv_pull(1, 4, rp, ci, np.array([0.0], np.float32), orc.F32,
                           np.array([2], np.int32), np.array([3.0], np.float32), orc.F32)
    assert y0[0] == 0.0


def _bfs_invariants(n, rp, ci, src, lv):
    assert lv[src] == 0
    rows = np.repeat(np.arange(n), np.diff(rp))
    both = (lv[rows] >= 0) & (lv[ci] >= 0)
    assert np.all(np.abs(lv[rows][both] - lv[ci][both]) <= 1)
    # nothing unreached next to something reached
    assert not np.any((lv[rows] >= 0) & (lv[ci] < 0))
    # every reached vertex other than src has a neighbour one level up
    reached = np.nonzero(lv > 0)[0]
    par = np.zeros(n, bool)
    ok = lv[ci] == lv[rows] - 1
    par[rows[ok]] = True
    assert np.all(par[reached])


@pytest.mark.parametrize("seed", range(3))
def test_bfs_matches_scipy_directed(seed):
    rng = rng_for("test", 20, seed)
    n = 70
    a = (rng.random((n, n)) < 0.03).astype(np.float32)
    rp, ci, _ = csr_from_dense(a)
    cp, ri, _ = orc.csr_to_csc(n, n, rp, ci)
    src = int(rng.integers(0, n))
    lv = orc.bfs(n, cp, ri, src)
    # y = A x expands j -> rows i with A_ij: scipy on the transposed graph
    d = shortest_path(sp.csr_matrix(a.T), directed=True, unweighted=True, indices=src)
    ref = np.where(np.isinf(d), -1, d).astype(np.int32)
    np.testing.assert_array_equal(lv, ref)


def test_bfs_rmat_invariants_and_scipy():
    rp, ci = rmat_csr(10, 8, rng_for("test", 21))
    n = 1 << 10
    lv = orc.bfs(n, rp, ci, 0)  # symmetric: CSC == CSR
    _bfs_invariants(n, rp, ci, 0, lv)
    g = sp.csr_matrix((np.ones(ci.shape[0]), ci, rp), shape=(n, n))
    d = shortest_path(g, directed=False, unweighted=True, indices=0)
    np.testing.assert_array_equal(lv, np.where(np.isinf(d), -1, d).astype(np.int32))


def test_dense_x_matches_dense_product_and_signed_zero_inactive():
    rng = rng_for("test", 30)
    a = _rand_sparse_dense(rng, 33, 48, 0.5)
    rp, ci, v = csr_from_dense(a)
    x = rng.uniform(-1, 1, 48).astype(np.float32)
    x[::3] = 0.0
    x[1::7] = -0.0
    y, s = orc.spmspv_dense_x(33, 48, rp, ci, v, orc.F32, x, orc.F32)
    np.testing.assert_allclose(y, a.astype(np.float64) @ x.astype(np.float64), rtol=1e-12, atol=1e-13)
    masks, cnt = orc.xmeta_dense(48, x, orc.F32)
    for b in range(3):
        exp = sum(1 << k for k in range(16) if x[16 * b + k] != 0)
        assert masks[b] == exp
    assert cnt == int(np.count_nonzero(masks))


def test_threshold_activation_worked_example():
    # magnitude thresholding worked by hand at t = 0.5: kept iff |x| > t
    # (0.5 itself and -0.0 drop, -0.6 and just-above -0.5 stay, NaN drops)
    x = np.array([0.4, -0.6, 0.5, 2.0, -0.0, np.nan, -0.5000001, 0.0], np.float32)
    out = orc.threshold_activation(x, orc.F32, 0.5)
    exp = np.array([0.0, -0.6, 0.0, 2.0, 0.0, 0.0, -0.5000001, 0.0], np.float32)
    assert np.array_equal(out.view(np.uint32), exp.view(np.uint32))  # dropped entries are +0
    # bf16: 0x3ED0 = 0.40625, 0xBF1A = -0.6015625, 0x3F00 = 0.5, 0x4000 = 2.0, 0x8000 = -0.0
    xb = np.array([0x3ED0, 0xBF1A, 0x3F00, 0x4000, 0x8000], np.uint16)
    assert orc.threshold_activation(xb, orc.BF16, 0.5).tolist() == [0, 0xBF1A, 0, 0x4000, 0]
    # the comparison is against the float32 threshold, exactly: t = 0.40625 drops 0.40625
    assert orc.threshold_activation(xb, orc.BF16, 0.40625).tolist() == [0, 0xBF1A, 0x3F00, 0x4000, 0]


def test_threshold_activation_special_cases_and_decode():
    rng = rng_for("test", 31)
    x = rng.normal(0.0, 1.0, 300).astype(np.float32)
    x[::17] = 0.0
    # t = 0 keeps exactly the nonzeros (the plain dense decode rule)
    assert np.array_equal(orc.threshold_activation(x, orc.F32, 0.0), np.where(x != 0, x, 0).astype(np.float32))
    # t at or above max |x| keeps nothing; counts fall as t grows
    assert not orc.threshold_activation(x, orc.F32, float(np.abs(x).max())).any()
    counts = [np.count_nonzero(orc.threshold_activation(x, orc.F32, t)) for t in (0.0, 0.3, 1.0, 2.0)]
    assert counts == sorted(counts, reverse=True) and counts[0] > counts[-1]
    # decode with the sparsified activation: the dense product over the kept entries
    a = _rand_sparse_dense(rng, 40, 300, 0.5)
    rp, ci, v = csr_from_dense(a)
    xs = orc.threshold_activation(x, orc.F32, 1.0)
    keep = np.abs(x.astype(np.float64)) > 1.0
    y, _ = orc.spmspv_dense_x(40, 300, rp, ci, v, orc.F32, xs, orc.F32)
    np.testing.assert_allclose(y, a.astype(np.float64)[:, keep] @ x.astype(np.float64)[keep], rtol=1e-12,
                               atol=1e-13)


def test_xmeta_bit_order_figure5_caption():
    # Figure 5 caption: a mask value of 10 = 0b1010 marks local positions 1 and 3
    masks, cnt = orc.xmeta(32, np.array([1, 3], np.int32))
    assert masks[0] == 10 and masks[1] == 0 and cnt == 1


def test_xmeta_brute_force():
    rng = rng_for("test", 31)
    n = 1000
    xi = np.sort(rng.choice(n, 77, replace=False)).astype(np.int32)
    masks, cnt = orc.xmeta(n, xi)
    bits = np.zeros(((n + 15) // 16) * 16, bool)
    bits[xi] = True
    exp = (bits.reshape(-1, 16) * (1 << np.arange(16))).sum(axis=1)
    np.testing.assert_array_equal(masks, exp.astype(np.uint16))
    assert cnt == len(np.unique(xi // 16))


def test_selector_threshold_is_strict():
    # section 3.3.1: push iff xb_sparsity < th3 = 0.01
    assert orc.select_push(9, 1000)
    assert not orc.select_push(10, 1000)
    assert orc.select_push(655, 65536)       # 65500 < 65536
    assert not orc.select_push(656, 65536)   # 65600 >= 65536
    assert not orc.select_push(1, 100)


def _read_classify_cases(golden_dir):
    cases, cur = [], None
    with open(os.path.join(golden_dir, "classify_tiles.txt")) as f:
        for line in f:
            line = line.rstrip("\n")
            if line.startswith("#") or not line:
                continue
            if line.startswith("case "):
                cur = {"why": line[5:], "rows": []}
            elif line.startswith("expect "):
                nz, mr, mc, ty = line.split()[1:]
                cur.update(nnz=int(nz), max_row=int(mr), max_col=int(mc), type=ty)
                cases.append(cur)
            else:
                cur["rows"].append(line)
    return cases


def test_classification_golden_tiles(golden_dir):
    cases = _read_classify_cases(golden_dir)
    assert len(cases) == 8
    names = {v: k for k, v in orc.TYPE_NAMES.items()}
    for c in cases:
        pat = np.array([[ch == "x" for ch in row] for row in c["rows"]])
        assert pat.shape == (16, 16)
        rp, ci, _ = csr_from_dense(pat.astype(np.float32))
        tv = orc.tile_view(16, 16, rp, ci)
        assert tv["T"] == 1, c["why"]
        assert tv["t_nnz"][0] == c["nnz"], c["why"]
        assert tv["t_maxrow"][0] == c["max_row"], c["why"]
        assert tv["t_maxcol"][0] == c["max_col"], c["why"]
        assert tv["t_type"][0] == names[c["type"]], c["why"]
        assert orc.classify(c["nnz"], c["max_row"], c["max_col"]) == names[c["type"]]
        # masks agree with the drawing (bit k = local column / row k)
        for r in range(16):
            assert tv["t_rowmask"][0, r] == sum(1 << k for k in range(16) if pat[r, k])
            assert tv["t_colmask"][0, r] == sum(1 << k for k in range(16) if pat[k, r])


def _kv(golden_dir, name):
    out = {}
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.split()
    return out


def test_tile_view_figure5(golden_dir):
    g = _kv(golden_dir, "fig5_block_views.txt")
    a = np.zeros((48, 48), np.float32)
    for cell in g["tiles_rb_cb"]:
        rb, cb = map(int, cell.split(","))
        a[rb * 16 + 3, cb * 16 + 5] = 1.0
    rp, ci, _ = csr_from_dense(a)
    tv = orc.tile_view(48, 48, rp, ci)
    for key, gk in [("rb_ptr", "blk_row_ptr"), ("t_cb", "blk_col_idx"), ("cb_ptr", "blk_col_ptr"),
                    ("csc_rb", "blk_row_idx"), ("csc2csr", "blk_csc2csr")]:
        np.testing.assert_array_equal(tv[key], np.array(g[gk], np.int32), err_msg=key)


@pytest.mark.parametrize("shape,dens", [((100, 90), 0.05), ((64, 64), 0.6), ((257, 31), 0.1), ((33, 500), 0.02)])
def test_tile_view_matches_scipy_block_pattern(shape, dens):
    m, n = shape
    rng = rng_for("test", 40, m, n)
    a = _rand_sparse_dense(rng, m, n, dens)
    rp, ci, _ = csr_from_dense(a)
    tv = orc.tile_view(m, n, rp, ci)
    r, c = np.nonzero(a)
    mb, nb = (m + 15) // 16, (n + 15) // 16
    B = sp.csr_matrix((np.ones(r.shape[0]), (r // 16, c // 16)), shape=(mb, nb))
    B.sum_duplicates()
    B.sort_indices()
    np.testing.assert_array_equal(tv["rb_ptr"], B.indptr)
    np.testing.assert_array_equal(tv["t_cb"], B.indices)
    np.testing.assert_array_equal(tv["t_nnz"], B.data.astype(np.int64))
    np.testing.assert_array_equal(tv["t_rb"], np.repeat(np.arange(mb), np.diff(B.indptr)))
    ids = sp.csr_matrix((np.arange(1, B.nnz + 1, dtype=np.float64), B.indices, B.indptr), shape=B.shape)
    Cc = ids.tocsc()
    Cc.sort_indices()
    np.testing.assert_array_equal(tv["cb_ptr"], Cc.indptr)
    np.testing.assert_array_equal(tv["csc_rb"], Cc.indices)
    np.testing.assert_array_equal(tv["csc2csr"], Cc.data.astype(np.int64) - 1)
    # per-tile row/column maxima from a 4-D reshape of the padded dense matrix
    pad = np.zeros((mb * 16, nb * 16), bool)
    pad[:m, :n] = a != 0
    t4 = pad.reshape(mb, 16, nb, 16).transpose(0, 2, 1, 3)
    rb, cb = tv["t_rb"], tv["t_cb"]
    np.testing.assert_array_equal(tv["t_maxrow"], t4[rb, cb].sum(axis=2).max(axis=1))
    np.testing.assert_array_equal(tv["t_maxcol"], t4[rb, cb].sum(axis=1).max(axis=1))


def test_segments_golden(golden_dir):
    codes = {"D": orc.DENSE, "R": orc.FORCE_CSR, "C": orc.FORCE_CSC, "S": orc.CSR, "O": orc.COO}
    types, rb_ptr = [], [0]
    exp = None
    with open(os.path.join(golden_dir, "segments_case.txt")) as f:
        for line in f:
            if line.startswith("rowblock"):
                toks = [t for t in line.split()[1:] if t != "-"]
                types += [codes[t] for t in toks]
                rb_ptr.append(len(types))
            elif line.startswith("expected"):
                exp = line.split("=", 1)[1].split()
    srb, s0, s1 = orc.segments(np.array(rb_ptr), np.array(types))
    got = [f"{a}:{b}-{c}" for a, b, c in zip(srb, s0, s1)]
    assert got == exp


def test_segments_cover_every_tile_once():
    rng = rng_for("test", 41)
    rb_ptr = np.concatenate([[0], np.cumsum(rng.integers(0, 40, 50))]).astype(np.int32)
    types = rng.integers(0, 5, rb_ptr[-1]).astype(np.int32)
    srb, s0, s1 = orc.segments(rb_ptr, types)
    cover = np.zeros(rb_ptr[-1], int)
    for rb, a, b in zip(srb, s0, s1):
        assert rb_ptr[rb] <= a < b <= rb_ptr[rb + 1]
        cover[a:b] += 1
    assert np.all(cover == 1)


def test_all_core_or_and_pull_equals_the_oracle():
    """The all-core CPU baseline (the oracle's Boolean pull loop with its rows
    split over OpenMP threads) gives the oracle's y exactly."""
    import oracle.oracle as o
    from synth import rmat_csr, sparse_x

    rp, ci = rmat_csr(13, 16, rng_for("test", 990))
    n = 1 << 13
    for k, d in enumerate((0.0, 0.001, 0.05, 1.0)):
        xi, _ = sparse_x(n, d, rng_for("test", 991, k), with_values=False)
        y, threads = o.or_and_pull_all_cores(n, n, rp, ci, xi)
        assert threads >= 1
        np.testing.assert_array_equal(y, orc.or_and_pull(n, n, rp, ci, xi))
