"""Host-side decoder of the library's blocked format (test code).

Reads the arrays exported by dbs_copy_array and turns every tile back into
(row, col, value-bits) triples, checking the internal consistency of each
tile format on the way (masks vs pointers vs the patched-CSR column index).
The layout decoded here is the one documented in the library's design notes.
"""
import numpy as np

COO, DENSE, FORCE_CSR, FORCE_CSC, CSR = 0, 1, 2, 3, 4


def _align(x, a):
    return (x + a - 1) // a * a


def _u16(buf, off, k=16):
    return np.frombuffer(buf[off:off + 2 * k].tobytes(), dtype=np.uint16)


def decode(arrs, vk, n_dense):
    """arrs: dict with rb_ptr, t_cb, t_meta, payload; vk: 0 f32, 1 bf16, 2 pattern.
    Returns rows, cols (int64) and value bits (uint32 for f32, uint16 for bf16, None)."""
    vs = {0: 4, 1: 2, 2: 0}[vk]
    vdt = {0: np.uint32, 1: np.uint16}.get(vk)
    meta = arrs["t_meta"].astype(np.uint64)
    pay = arrs["payload"]
    T = meta.shape[0]
    rb_of = np.repeat(np.arange(arrs["rb_ptr"].shape[0] - 1), np.diff(arrs["rb_ptr"].astype(np.int64)))
    assert rb_of.shape[0] == T
    vp = (meta & np.uint64((1 << 40) - 1)).astype(np.int64)
    nnz = ((meta >> np.uint64(40)) & np.uint64(0xFF)).astype(np.int64) + 1
    typ = ((meta >> np.uint64(48)) & np.uint64(7)).astype(np.int64)
    dense_mask_off = pay.shape[0] - 32 * n_dense if vk != 2 else None
    R, Cc, V = [], [], []

    def vals_at(off, idx):
        if vdt is None:
            return None
        raw = pay[off:off + vs * (int(idx.max()) + 1 if idx.size else 0)].tobytes()
        return np.frombuffer(raw, dtype=vdt)[idx]

    for t in range(T):
        p, k, ty = int(vp[t]), int(nnz[t]), int(typ[t])
        r0, c0 = int(rb_of[t]) * 16, int(arrs["t_cb"][t]) * 16
        if ty == COO and (int(meta[t]) >> 51) & 1:
            # up to four coordinate bytes stored in the metadata word (pattern matrices)
            assert vk == 2 and k <= 4, f"inline COO tile {t} on a value matrix or with {k} entries"
            co = np.array([(int(meta[t]) >> (8 * e)) & 0xFF for e in range(k)], np.int64)
            rr, cc = co >> 4, co & 15
            assert np.all(np.diff(rr * 16 + cc) > 0), f"COO coords not row-major at tile {t}"
            vv = None
        elif ty == COO:
            assert not (vk == 2 and k <= 4), f"small pattern COO tile {t} not inline"
            co = pay[p:p + k].astype(np.int64)
            rr, cc = co >> 4, co & 15
            assert np.all(np.diff(rr * 16 + cc) > 0), f"COO coords not row-major at tile {t}"
            vv = vals_at(p + _align(k, 4), np.arange(k)) if vs else None
        elif vk == 2:
            rm = _u16(pay, p)
            cm = _u16(pay, p + 32)
            rr, cc = np.nonzero((rm[:, None] >> np.arange(16)) & 1)
            rr2, cc2 = np.nonzero(((cm[None, :] >> np.arange(16)[:, None]) & 1))
            assert np.array_equal(np.sort(rr * 16 + cc), np.sort(rr2 * 16 + cc2)), f"pattern masks disagree at {t}"
            vv = None
        elif ty == DENSE:
            rank = p // (256 * vs)
            assert rank * 256 * vs == p and p % 128 == 0, f"Dense tile {t} misaligned"
            rm = _u16(pay, dense_mask_off + 32 * rank)
            rr, cc = np.nonzero((rm[:, None] >> np.arange(16)) & 1)
            allv = np.frombuffer(pay[p:p + 256 * vs].tobytes(), dtype=vdt)
            absent = np.ones(256, bool)
            absent[rr * 16 + cc] = False
            assert np.all(allv[absent] == 0), f"Dense tile {t} holds values outside its mask"
            vv = allv[rr * 16 + cc]
        elif ty in (FORCE_CSR, CSR):
            rm = _u16(pay, p)
            rp = pay[p + 32:p + 48].astype(np.int64)
            cnt = np.array([bin(int(x)).count("1") for x in rm])
            assert np.array_equal(rp, np.concatenate([[0], np.cumsum(cnt)[:-1]])), f"row_ptr at {t}"
            rr, cc = np.nonzero((rm[:, None] >> np.arange(16)) & 1)  # row-major order
            voff = p + 48 if ty == FORCE_CSR else p + 64 + _align(k, 16)
            vv = vals_at(voff, np.arange(k))
            if ty == CSR:
                cp = pay[p + 48:p + 64].astype(np.int64)
                rc = pay[p + 64:p + 64 + k].astype(np.int64)
                ends = np.append(cp[1:], k)
                for c in range(16):
                    for e in range(cp[c], ends[c]):
                        r, j = rc[e] >> 4, rc[e] & 15
                        cols_r = [b for b in range(16) if (int(rm[r]) >> b) & 1]
                        assert cols_r[j] == c, f"row_idx_csc2csr entry wrong at tile {t}"
                    rows_c = [r for r in range(16) if (int(rm[r]) >> c) & 1]
                    assert [rc[e] >> 4 for e in range(cp[c], ends[c])] == rows_c, f"col {c} rows at {t}"
        elif ty == FORCE_CSC:
            cm = _u16(pay, p)
            cp = pay[p + 32:p + 48].astype(np.int64)
            cnt = np.array([bin(int(x)).count("1") for x in cm])
            assert np.array_equal(cp, np.concatenate([[0], np.cumsum(cnt)[:-1]])), f"col_ptr at {t}"
            cc, rr = np.nonzero((cm[:, None] >> np.arange(16)) & 1)  # column-major order
            vv = vals_at(p + 48, np.arange(k))
        else:
            raise AssertionError(f"bad format {ty} at tile {t}")
        assert rr.shape[0] == k, f"tile {t}: {rr.shape[0]} entries, metadata says {k}"
        R.append(rr + r0)
        Cc.append(cc + c0)
        if vv is not None:
            V.append(vv)
    rows = np.concatenate(R) if R else np.zeros(0, np.int64)
    cols = np.concatenate(Cc) if Cc else np.zeros(0, np.int64)
    vals = np.concatenate(V) if V else None
    return rows, cols, vals, typ, nnz
