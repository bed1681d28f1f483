"""Seeded generators for the synthetic workloads.

Every generator takes a ``numpy.random.Generator`` so that callers derive all
randomness from one root seed (42, as in the paper's evaluation setup, section
5.2 of "DB-SpMSpV: Dual-View Blocked Sparse Matrix-Sparse Vector
Multiplication for Dynamic GPU Workloads").  Matrices come back as CSR with
int32 ``row_ptr``/``col_idx`` (columns sorted and unique per row) and either
float32 values, bf16 values as raw uint16 bit patterns, or no values.

Nothing here computes a product, a tile, a mask or a traversal.
"""
from __future__ import annotations

import numpy as np

ROOT_SEED = 42

# stable integer ids for the spawn keys of each workload
_CONFIG_IDS = {
    "tiny": 1,
    "rmat20": 2,
    "rmat22": 3,
    "decode": 4,
    "zipf": 5,
    "test": 9,
}


def rng_for(config: str, *item: int) -> np.random.Generator:
    """Independent generator for (workload, item...) derived from the root seed."""
    key = (_CONFIG_IDS[config],) + tuple(int(i) for i in item)
    return np.random.default_rng(np.random.SeedSequence(ROOT_SEED, spawn_key=key))


# --------------------------------------------------------------------------
# bf16 bit patterns (inputs are *stored* as bf16; rounding is round-to-nearest-even)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def _csr_from_sorted_keys(keys: np.ndarray, nrows: int, ncols: int):
    """CSR arrays from sorted unique int64 keys row*ncols+col."""
    rows = keys // ncols
    cols = (keys - rows * ncols).astype(np.int32)
    counts = np.bincount(rows, minlength=nrows)
    row_ptr = np.zeros(nrows + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    if row_ptr[-1] >= 2**31:
        raise ValueError("nnz does not fit int32")
    return row_ptr.astype(np.int32), cols


def csr_from_dense(a: np.ndarray):
    """CSR (row_ptr, col_idx, values) of the nonzero pattern of a small dense array."""
    a = np.asarray(a)
    r, c = np.nonzero(a)
    row_ptr = np.zeros(a.shape[0] + 1, dtype=np.int32)
    np.cumsum(np.bincount(r, minlength=a.shape[0]), out=row_ptr[1:])
    return row_ptr, c.astype(np.int32), a[r, c]


def _distinct_sorted_rows(m: int, n: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """(m, k) array; each row holds k distinct uniform values in [0, n), sorted."""
    if k > n:
        raise ValueError("k > n")
    cols = np.sort(rng.integers(0, n, size=(m, k), dtype=np.int64), axis=1)
    while True:
        dup = (cols[:, 1:] == cols[:, :-1]).any(axis=1) if k > 1 else np.zeros(m, bool)
        bad = np.nonzero(dup)[0]
        if bad.size == 0:
            return cols
        cols[bad] = np.sort(rng.integers(0, n, size=(bad.size, k), dtype=np.int64), axis=1)


# --------------------------------------------------------------------------
# Tiny SpMSpV: uniform random columns, fixed nnz per row
# --------------------------------------------------------------------------
def uniform_csr(m: int, n: int, per_row: int, rng: np.random.Generator):
    """m x n, ``per_row`` distinct uniform columns per row, float32 U[-1, 1]."""
    cols = _distinct_sorted_rows(m, n, per_row, rng)
    row_ptr = (np.arange(m + 1, dtype=np.int64) * per_row).astype(np.int32)
    vals = rng.uniform(-1.0, 1.0, size=m * per_row).astype(np.float32)
    return row_ptr, cols.reshape(-1).astype(np.int32), vals


# --------------------------------------------------------------------------
# R-MAT (Kronecker quadrant recursion), symmetrized, no self-loops, deduplicated
# --------------------------------------------------------------------------
def rmat_csr(scale: int, edge_factor: int, rng: np.random.Generator,
             a: float = 0.57, b: float = 0.19, c: float = 0.19):
    """Symmetric R-MAT pattern matrix with 2**scale vertices.

    edge_factor * 2**scale directed edges are drawn; at each of ``scale``
    recursion levels an edge falls in the top-left / top-right / bottom-left /
    bottom-right quadrant with probability a / b / c / 1-a-b-c (the most
    significant bit is decided first).  No vertex permutation and no noise.
    Self-loops are dropped, every edge is mirrored and duplicates are removed.
    Returns (row_ptr, col_idx) with no values.
    """
    nv = 1 << scale
    ne = edge_factor * nv
    u = np.zeros(ne, dtype=np.int64)
    v = np.zeros(ne, dtype=np.int64)
    t_ab = np.float32(a + b)
    t_a = np.float32(a)
    t_abc = np.float32(a + b + c)
    for _ in range(scale):
        r = rng.random(ne, dtype=np.float32)
        u <<= 1
        v <<= 1
        u |= r >= t_ab
        v |= ((r >= t_a) & (r < t_ab)) | (r >= t_abc)
        del r
    keep = u != v
    u = u[keep]
    v = v[keep]
    keys = np.concatenate([u * nv + v, v * nv + u])
    del u, v, keep
    keys = np.unique(keys)
    return _csr_from_sorted_keys(keys, nv, nv)


def permute_vertices(row_ptr: np.ndarray, col_idx: np.ndarray, rng: np.random.Generator):
    """The same square pattern matrix with its vertices relabelled by a seeded
    random permutation p (entry (i, j) moves to (p[i], p[j])).  On an R-MAT
    graph this scatters the hub rows and columns over the whole index range,
    so its 16x16 tiles hold about one entry each instead of ~1.6.
    Returns (row_ptr, col_idx) with sorted columns per row."""
    n = row_ptr.shape[0] - 1
    perm = rng.permutation(n).astype(np.int64)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(row_ptr.astype(np.int64)))
    keys = perm[rows] * n + perm[col_idx.astype(np.int64)]
    del rows
    keys.sort()
    return _csr_from_sorted_keys(keys, n, n)


def largest_component_vertices(row_ptr: np.ndarray, col_idx: np.ndarray, n: int) -> np.ndarray:
    """Sorted vertex ids of the largest connected component (symmetric pattern)."""
    import scipy.sparse as sp
    from scipy.sparse.csgraph import connected_components

    data = np.ones(col_idx.shape[0], dtype=np.int8)
    g = sp.csr_matrix((data, col_idx, row_ptr), shape=(n, n))
    _, labels = connected_components(g, directed=False)
    big = np.bincount(labels).argmax()
    return np.nonzero(labels == big)[0].astype(np.int32)


# --------------------------------------------------------------------------
# Single-token sparse decode: Bernoulli-pruned bf16 weights, ReLU-like activations
# --------------------------------------------------------------------------
def decode_weight_csr(rows: int, cols: int, sparsity: float, rng: np.random.Generator,
                      std: float = 0.02):
    """rows x cols weight; each entry kept with probability 1 - sparsity.

    Kept values are N(0, std) rounded to bf16; returned as uint16 bit patterns.
    """
    keep = rng.random((rows, cols), dtype=np.float32) >= np.float32(sparsity)
    counts = keep.sum(axis=1)
    _, c = np.nonzero(keep)
    del keep
    row_ptr = np.zeros(rows + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    vals = f32_to_bf16_bits(rng.normal(0.0, std, size=c.shape[0]).astype(np.float32))
    return row_ptr.astype(np.int32), c.astype(np.int32), vals


def decode_activation(k: int, zero_frac: float, rng: np.random.Generator) -> np.ndarray:
    """Dense bf16 activation of length k with exactly round(zero_frac*k) zeros.

    Nonzeros are |N(0, 1)| rounded to bf16 (uint16 bit patterns).
    """
    x = f32_to_bf16_bits(np.abs(rng.normal(0.0, 1.0, size=k)).astype(np.float32))
    nz = int(round(zero_frac * k))
    x[rng.choice(k, size=nz, replace=False)] = 0
    return x


# --------------------------------------------------------------------------
# Load-imbalance stress: Zipf row lengths, banded columns plus long-range ones
# --------------------------------------------------------------------------
def zipf_lengths(n: int, rng: np.random.Generator, alpha: float = 1.8,
                 cap: int = 1 << 20, target_nnz: int = 128 * 1000 * 1000) -> np.ndarray:
    """Row lengths min(cap, max(1, round(c*L_i))), L_i ~ Zipf(alpha), c by bisection
    so that the total is close to ``target_nnz``.  The bisection runs over the
    distinct values of L with their counts."""
    raw = rng.zipf(alpha, size=n)
    vals, inv, cnt = np.unique(raw, return_inverse=True, return_counts=True)
    vals = vals.astype(np.float64)

    def lengths(scale: float) -> np.ndarray:
        return np.minimum(cap, np.maximum(1.0, np.rint(scale * vals))).astype(np.int64)

    lo, hi = 1e-6, 1e3
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if int((lengths(mid) * cnt).sum()) < target_nnz:
            lo = mid
        else:
            hi = mid
    return lengths(lo)[inv.reshape(-1)]


def zipf_band_csr(n: int, rng: np.random.Generator, alpha: float = 1.8,
                  cap: int = 1 << 20, target_nnz: int = 128 * 1000 * 1000,
                  band_frac: float = 0.9):
    """n x n float32 U[-1, 1] matrix with Zipf row lengths.

    Row i of length L gets round(band_frac*L) columns in a band of width
    2h+1, h = max(64, L), centred at i (shifted inward at the matrix edges),
    one column drawn uniformly in each of that many equal strata of the band,
    so they are distinct; the other columns are uniform over [0, n).  The few
    duplicates a far column can make are merged.
    """
    lens = zipf_lengths(n, rng, alpha, cap, target_nnz)
    nbnd = np.rint(band_frac * lens).astype(np.int64)
    nfar = lens - nbnd
    h = np.maximum(64, lens)
    w = 2 * h + 1
    start = np.clip(np.arange(n, dtype=np.int64) - h, 0, n - w)
    # band columns: entry k of row i lies in stratum k of width w_i / nbnd_i
    rows = np.repeat(np.arange(n, dtype=np.int64), nbnd)
    k = np.arange(rows.shape[0], dtype=np.int64) - np.repeat(np.cumsum(nbnd) - nbnd, nbnd)
    width = (w / np.maximum(nbnd, 1))[rows]
    col = start[rows] + np.floor((k + rng.random(rows.shape[0])) * width).astype(np.int64)
    del k, width
    keys_b = rows * n + col
    del rows, col
    rows = np.repeat(np.arange(n, dtype=np.int64), nfar)
    keys_f = rows * n + rng.integers(0, n, size=rows.shape[0], dtype=np.int64)
    del rows
    keys = np.concatenate([keys_b, keys_f])
    del keys_b, keys_f
    keys.sort()
    keep = np.empty(keys.shape[0], dtype=bool)
    keep[0] = True
    np.not_equal(keys[1:], keys[:-1], out=keep[1:])
    keys = keys[keep]
    del keep
    row_ptr, col_idx = _csr_from_sorted_keys(keys, n, n)
    del keys
    vals = rng.uniform(-1.0, 1.0, size=col_idx.shape[0]).astype(np.float32)
    return row_ptr, col_idx, vals


# --------------------------------------------------------------------------
# sparse input vectors
# --------------------------------------------------------------------------
def sparse_x(n: int, density: float, rng: np.random.Generator, with_values: bool = True):
    """round(density*n) distinct uniform positions (sorted int32) and float32 U[-1, 1]."""
    k = int(round(density * n))
    idx = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)
    vals = rng.uniform(-1.0, 1.0, size=k).astype(np.float32) if with_values else None
    return idx, vals


def sparse_x_with_dense_blocks(n: int, density: float, rng: np.random.Generator,
                               dense_frac: float = 0.1, block: int = 16,
                               with_values: bool = True):
    """As ``sparse_x``, then a ``dense_frac`` share of the touched aligned
    ``block``-element groups is filled completely."""
    idx, _ = sparse_x(n, density, rng, with_values=False)
    groups = np.unique(idx // block)
    nfill = int(round(dense_frac * groups.shape[0]))
    if nfill:
        chosen = rng.choice(groups, size=nfill, replace=False)
        extra = (chosen[:, None] * block + np.arange(block)[None, :]).reshape(-1)
        extra = extra[extra < n]
        idx = np.union1d(idx, extra).astype(np.int32)
    vals = rng.uniform(-1.0, 1.0, size=idx.shape[0]).astype(np.float32) if with_values else None
    return idx, vals
