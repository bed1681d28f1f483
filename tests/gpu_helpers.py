"""Shared helpers of the GPU tests: upload, build, and matrices that hold every
tile format.  Inputs come from the seeded generators only."""
import numpy as np

from synth import csr_from_dense, f32_to_bf16_bits, rng_for


def up(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def build(dbs, m, n, rp, ci, v, dtype, options=None):
    val = None
    if dtype == dbs.DBS_F32:
        val = up(np.asarray(v, np.float32))
    elif dtype == dbs.DBS_BF16:
        val = up(np.asarray(v, np.uint16).view(np.int16))
    return dbs.dbs_build(m, n, up(rp), up(ci), val, dtype, options=options)


def options(dbs, **kw):
    o = dbs.default_build_options()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def mixed_tile_dense(seed, mb=5, nb=6, ragged=(7, 9)):
    """Dense float32 array whose 16x16 tiles cover every format: COO, Dense,
    ForceCSR (few full columns), ForceCSC (few full rows), patched CSR, plus
    empty tiles; the last row/column blocks are cut short (ragged edge)."""
    rng = rng_for("test", 500, seed)
    a = np.zeros((mb * 16, nb * 16), np.float32)
    kinds = ["coo", "dense", "fcsr", "fcsc", "csr", "empty"]
    for rb in range(mb):
        for cb in range(nb):
            kind = kinds[(rb + 2 * cb + seed) % len(kinds)]
            t = np.zeros((16, 16), bool)
            if kind == "coo":
                t = rng.random((16, 16)) < 0.06
            elif kind == "dense":
                t = rng.random((16, 16)) < 0.7
            elif kind == "fcsr":
                cols = rng.choice(16, 2 + (seed % 3), replace=False)
                t[:, cols] = True
                t &= rng.random((16, 16)) < 0.95
            elif kind == "fcsc":
                rows = rng.choice(16, 2 + (seed % 3), replace=False)
                t[rows, :] = True
                t &= rng.random((16, 16)) < 0.95
            elif kind == "csr":
                t = rng.random((16, 16)) < 0.3
            vals = rng.uniform(-1, 1, (16, 16)).astype(np.float32)
            vals[vals == 0] = 0.5
            a[rb * 16:(rb + 1) * 16, cb * 16:(cb + 1) * 16] = np.where(t, vals, 0)
    m = mb * 16 - ragged[0]
    n = nb * 16 - ragged[1]
    return a[:m, :n]


def csr_of(a):
    rp, ci, v = csr_from_dense(a)
    return rp, ci, v.astype(np.float32)


def bf16_csr_of(a):
    rp, ci, v = csr_from_dense(a)
    bits = f32_to_bf16_bits(v.astype(np.float32))
    # rounding can create zeros only for tiny values; keep them as stored entries
    return rp, ci, bits
