"""CPU checks of the seeded input generators that are not pinned through the
oracle's own tests."""
import numpy as np

from synth import permute_vertices, rmat_csr, rng_for


def test_permuted_rmat_is_a_relabelling():
    """permute_vertices keeps the graph: same entry count, symmetric, sorted
    rows, and the degree of vertex p[i] is the degree of vertex i."""
    rp, ci = rmat_csr(12, 16, rng_for("test", 1200))
    n = rp.shape[0] - 1
    prp, pci = permute_vertices(rp, ci, rng_for("test", 1201))
    assert prp[-1] == rp[-1]
    deg = np.diff(rp)
    pdeg = np.diff(prp)
    perm = rng_for("test", 1201).permutation(n)
    np.testing.assert_array_equal(pdeg[perm], deg)
    # every edge (i, j) appears as (p[i], p[j]); rows sorted and unique
    rows = np.repeat(np.arange(n), deg)
    want = np.sort(perm[rows].astype(np.int64) * n + perm[ci])
    prow = np.repeat(np.arange(n), pdeg)
    got = prow.astype(np.int64) * n + pci
    np.testing.assert_array_equal(got, want)
    # symmetric: the transpose has the same key set
    gt = np.sort(pci.astype(np.int64) * n + prow)
    np.testing.assert_array_equal(gt, got)
    # it does scatter the tiles: fewer entries per 16x16 tile than the plain graph
    def tiles(r, c):
        rr = np.repeat(np.arange(n), np.diff(r))
        return np.unique((rr // 16).astype(np.int64) * (n // 16) + c // 16).shape[0]
    assert tiles(prp, pci) > 1.2 * tiles(rp, ci)
