// Per-tile wave64 microkernels (section 3.3.3 of "DB-SpMSpV: Dual-View Blocked
// Sparse Matrix-Sparse Vector Multiplication for Dynamic GPU Workloads";
// Algorithms 2-5) and the COO lane-per-tile path.
//
// A 64-lane wave covers a whole 16x16 tile at once: lane L = q*16 + r works
// on row r and quarter q (q = L >> 4).  Where the pages split a 32-lane warp
// in two halves or pairs, the wave splits in four; row partials are merged
// across the quarters with xor-16 and xor-32 exchanges, after which lanes
// 0..15 hold the 16 row results of the tile.
//
// x values of the tile's vector block are staged in LDS (one 16-entry slot
// per wave) so that lanes with different amounts of work can read them.
#pragma once

#include "common.h"

// ---------------------------------------------------------------------------
// Raw buffer loads: a 128-bit descriptor (base, size) in SGPRs and a 32-bit
// byte offset per lane.  Reads past the size return 0 without touching
// memory, so an idle lane passes OOB_OFF instead of branching around the
// load (a branch around a load makes the compiler wait for every load in
// flight), and no 64-bit address arithmetic is spent per lane.
// ---------------------------------------------------------------------------
#define OOB_OFF 0xFFFFFFF0u
typedef __amdgpu_buffer_rsrc_t brsrc_t;

DBS_DEV brsrc_t make_rsrc(const void *p, uint64_t bytes) {
  const uint32_t n = bytes >= 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, (int)n, 0x00020000);
}
DBS_DEV uint32_t bld32(brsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
DBS_DEV uint64_t bld64(brsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return (uint64_t)v[0] | ((uint64_t)v[1] << 32);
}

extern "C" __device__ uint32_t __ockl_wfred_or_u32(uint32_t);
// OR over the 64 lanes of the wave (DPP row shifts + row mirror); uniform result
DBS_DEV uint32_t wave_or(uint32_t v) { return __ockl_wfred_or_u32(v); }
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);
DBS_DEV uint32_t wave_max(uint32_t v) { return __ockl_wfred_max_u32(v); }

// inclusive maximum over lanes 0..lane (row shifts within each 16-lane row,
// then the row broadcasts carry rows 0..2 forward; lanes a DPP step does not
// write keep 0, the identity)
DBS_DEV uint32_t wave_incl_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// inclusive prefix sum over lanes 0..lane (same DPP steps as wave_incl_max)
DBS_DEV uint32_t wave_incl_add(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// inclusive prefix sum over the 16 lanes of each quarter (DPP row shifts;
// lanes shifted in from outside the quarter read 0)
DBS_DEV uint32_t quarter_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  return v;
}

// OR-AND contribution of four coordinate bytes (row << 4 | col) under the
// x-block mask m.  Unused bytes of a tile repeat its last entry, so all four
// are decoded unconditionally (OR is idempotent).
DBS_DEV uint32_t coo_or4(uint32_t w, uint32_t m) {
  uint32_t f = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t c = (w >> (8 * k)) & 15u;
    const uint32_t r = (w >> (8 * k + 4)) & 15u;
    f |= ((m >> c) & 1u) << r;
  }
  return f;
}

template <int VK>
DBS_DEV float load_a(const uint8_t *p) {
  if (VK == VK_F32) return *(const float *)p;
  if (VK == VK_BF16) return bf16_to_f32(*(const uint16_t *)p);
  return 1.0f;
}

template <int VK>
DBS_DEV float load_x(const void *xd, int64_t j) {
  if (VK == VK_F32) return ((const float *)xd)[j];
  if (VK == VK_BF16) return bf16_to_f32(((const uint16_t *)xd)[j]);
  return 1.0f;
}

DBS_DEV float quarter_merge(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// remove the lowest k set bits
DBS_DEV uint32_t drop_low_bits(uint32_t v, int k) {
  for (int i = 0; i < k; ++i) v &= v - 1u;
  return v;
}

// ---------------------------------------------------------------------------
// PLUS_TIMES microkernels.  `m` is the tile's blk_x_mask, sx the staged x
// values (inactive entries hold 0).  Return: row r's partial in every lane
// with that r (use lanes 0..15).
// ---------------------------------------------------------------------------

// Dense, row-major (Algorithm 4): lane (q, r) loads row r, columns 4q..4q+3
// with one 16-B (fp32) or 8-B (bf16) load; the wave reads the tile with a
// single fully coalesced access.  The same kernel serves push, where the
// pages transpose through shared memory to reach columns contiguously: here
// every lane already holds its slice of each row.
template <int VK>
DBS_DEV float mk_dense(const uint8_t *base, uint32_t m, const float *sx, int q, int r) {
  float a[4];
  if (VK == VK_F32) {
    const float4 v = *(const float4 *)(base + (r * 16 + 4 * q) * 4);
    a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
  } else {
    const uint2 v = *(const uint2 *)(base + (r * 16 + 4 * q) * 2);
    a[0] = __uint_as_float(v.x << 16);
    a[1] = __uint_as_float(v.x & 0xFFFF0000u);
    a[2] = __uint_as_float(v.y << 16);
    a[3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
  float part = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 4 * q + k;
    if ((m >> c) & 1u) part += a[k] * sx[c];
  }
  return quarter_merge(part);
}

// ForceCSR pull (Algorithm 2): four interleaved lanes per row; lane q takes
// the active columns of rank q, q+4, ... ; value position = row_ptr[r] +
// popcount of the row mask below the column.
template <int VK>
DBS_DEV float mk_force_csr(const uint8_t *base, uint32_t val_off, uint32_t m, const float *sx,
                           int q, int r) {
  constexpr int VS = VK == VK_F32 ? 4 : 2;
  const uint32_t rmk = ((const uint16_t *)(base + PL_MASK))[r];
  const uint32_t rp = base[PL_PTR + r];
  uint32_t act = drop_low_bits(rmk & m, q);
  float part = 0.0f;
  while (act) {
    const uint32_t c = (uint32_t)__ffs(act) - 1u;
    const uint32_t off = rp + (uint32_t)__popc(rmk & below_mask(c));
    part += load_a<VK>(base + val_off + off * VS) * sx[c];
    act = drop_low_bits(act, 4);
  }
  return quarter_merge(part);
}

// ForceCSC push (Algorithm 3): lane (q, r) scans the active columns of
// quarter q (columns 4q..4q+3) and tests bit r of each column mask; value
// position = col_ptr[c] + popcount of the column mask below the row.
template <int VK>
DBS_DEV float mk_force_csc(const uint8_t *base, uint32_t m, const float *sx, int q, int r) {
  constexpr int VS = VK == VK_F32 ? 4 : 2;
  uint32_t act = m & (0xFu << (4 * q));
  float part = 0.0f;
  while (act) {
    const uint32_t c = (uint32_t)__ffs(act) - 1u;
    const uint32_t cm = ((const uint16_t *)(base + PL_MASK))[c];
    if ((cm >> r) & 1u) {
      const uint32_t off = base[PL_PTR + c] + (uint32_t)__popc(cm & below_mask((uint32_t)r));
      part += load_a<VK>(base + PL_FORCE_VAL + off * VS) * sx[c];
    }
    act &= act - 1u;
  }
  return quarter_merge(part);
}

// Patched CSR, column (push) variant: for each active column c the entries
// col_ptr[c] .. col_ptr[c+1] of row_idx_csc2csr give (row, index in row);
// the value sits at row_ptr[row] + index, so the row-major value array serves
// both directions.  Quarter q takes the active columns of rank q, q+4, ...;
// lane (q, e) takes entry e of that column.  Rows inside one column are
// distinct, so the per-quarter LDS partials never see two lanes on one
// address.
template <int VK>
DBS_DEV float mk_csr_push(const uint8_t *base, uint32_t nnz, uint32_t m, const float *sx,
                          float *spart /* [4][16] of this wave */, int q, int r) {
  constexpr int VS = VK == VK_F32 ? 4 : 2;
  const uint32_t voff = csr_val_off(nnz);
  spart[q * 16 + r] = 0.0f;
  __syncwarp();
  uint32_t act = drop_low_bits(m, q);
  // every lane runs the same number of rounds: that of quarter 0 (the most)
  uint32_t rounds = ((uint32_t)__popc(m) + 3u) >> 2;
  for (uint32_t it = 0; it < rounds; ++it) {
    if (act) {
      const uint32_t c = (uint32_t)__ffs(act) - 1u;
      const uint32_t start = base[PL_CSR_COLPTR + c];
      const uint32_t end = c < 15 ? base[PL_CSR_COLPTR + c + 1] : nnz;
      if (start + (uint32_t)r < end) {
        const uint32_t rc = base[PL_CSR_RC + start + r];
        const uint32_t row = rc >> 4, j = rc & 15u;
        const uint32_t off = base[PL_PTR + row] + j;
        spart[q * 16 + row] += load_a<VK>(base + voff + off * VS) * sx[c];
      }
      act = drop_low_bits(act, 4);
    }
    __syncwarp();
  }
  return quarter_merge(spart[q * 16 + r]);
}

// ---------------------------------------------------------------------------
// OR_AND microkernels: 16-bit mask of rows with a stored entry in an active
// column (wave-uniform result).
// ---------------------------------------------------------------------------
DBS_DEV uint32_t mk_bool_rows(const uint16_t *row_mask, uint32_t m, int lane) {
  uint32_t f = 0;
  if (lane < 16) f = (((uint32_t)row_mask[lane] & m) != 0u) ? (1u << lane) : 0u;
  return group_or_u32<64>(f);
}

// Algorithm 5 (Boolean ForceCSC push): OR of the masks of the active columns
DBS_DEV uint32_t mk_bool_cols(const uint16_t *col_mask, uint32_t m, int lane) {
  uint32_t f = 0;
  if (lane < 16 && ((m >> lane) & 1u)) f = col_mask[lane];
  return group_or_u32<64>(f);
}

// ---------------------------------------------------------------------------
// Tile dispatch.  `dense_mask` points at the Dense tile's row masks (value
// matrices, OR_AND only).
// ---------------------------------------------------------------------------
template <int VK>
DBS_DEV float tile_plus(const uint8_t *base, uint32_t type, uint32_t nnz, uint32_t m,
                        const float *sx, float *spart, int local_cutoff, int lane) {
  const int q = lane >> 4, r = lane & 15;
  if (type == DBS_TILE_DENSE) return mk_dense<VK>(base, m, sx, q, r);
  if (type == DBS_TILE_FORCE_CSR) return mk_force_csr<VK>(base, PL_FORCE_VAL, m, sx, q, r);
  if (type == DBS_TILE_FORCE_CSC) return mk_force_csc<VK>(base, m, sx, q, r);
  // patched CSR: local choice from the number of active x entries (section 3.3.3)
  if (__popc(m) >= local_cutoff) return mk_force_csr<VK>(base, csr_val_off(nnz), m, sx, q, r);
  return mk_csr_push<VK>(base, nnz, m, sx, spart, q, r);
}

template <int VK>
DBS_DEV uint32_t tile_or(const uint8_t *base, const uint8_t *dense_mask, uint32_t type, uint32_t m,
                         int lane) {
  if (VK == VK_PAT) {
    if (type == DBS_TILE_FORCE_CSC) return mk_bool_cols((const uint16_t *)(base + PL_PAT_COLMASK), m, lane);
    return mk_bool_rows((const uint16_t *)(base + PL_MASK), m, lane);
  }
  if (type == DBS_TILE_DENSE) return mk_bool_rows((const uint16_t *)dense_mask, m, lane);
  if (type == DBS_TILE_FORCE_CSC) return mk_bool_cols((const uint16_t *)(base + PL_MASK), m, lane);
  return mk_bool_rows((const uint16_t *)(base + PL_MASK), m, lane);  // ForceCSR, CSR
}

// ---------------------------------------------------------------------------
// COO (section 3.3.3: scan the packed coordinates), one tile per lane.
// ---------------------------------------------------------------------------
// OR-AND of a COO tile from its (4-B aligned) coordinate bytes, 32 entries
// per round of independent loads
DBS_DEV uint32_t coo_or(const uint8_t *base, uint32_t nnz, uint32_t m) {
  uint32_t f = 0;
  const uint32_t *w = (const uint32_t *)base;
  const uint32_t last = (nnz - 1) >> 2;  // last word of the tile
  for (uint32_t e0 = 0; e0 < nnz; e0 += 32) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // clamped word index: no branch around the loads
      const uint32_t wi = (e0 >> 2) + k;
      v[k] = w[wi < last ? wi : last];
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t rc = (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      if (e0 + k < nnz && ((m >> (rc & 15u)) & 1u)) f |= 1u << (rc >> 4);
    }
  }
  return f;
}

// OR-AND of a COO tile given its metadata word (coordinates inline or in the payload)
DBS_DEV uint32_t coo_or_meta(const uint8_t *payload, uint64_t meta, uint32_t m) {
  const uint32_t nnz = meta_nnz(meta);
  if (meta_inline(meta)) {
    const uint32_t w = (uint32_t)meta;
    uint32_t f = 0;
#pragma unroll
    for (uint32_t e = 0; e < COO_INLINE; ++e) {
      const uint32_t rc = (w >> (8 * e)) & 0xFFu;
      if (e < nnz && ((m >> (rc & 15u)) & 1u)) f |= 1u << (rc >> 4);
    }
    return f;
  }
  return coo_or(payload + meta_vp(meta), nnz, m);
}

// ---------------------------------------------------------------------------
// OR-AND contribution of the COO tile held by this lane (pull and push),
// given the metadata word and the first two payload words loaded ahead (pw0,
// pw1; only meaningful for COO tiles that are not inline).  Called by every
// lane of the wave.
// ---------------------------------------------------------------------------
DBS_DEV uint32_t lane_coo_or(const uint8_t *payload, uint64_t meta, uint32_t m, bool act, uint32_t pw0,
                             uint32_t pw1) {
  const bool coo = act & (meta_type(meta) == DBS_TILE_COO);
  const bool inl = meta_inline(meta);
  const uint32_t w0 = inl ? (uint32_t)meta : pw0;
  uint32_t f = coo ? coo_or4(w0, m) : 0u;
  const uint32_t nnz = meta_nnz(meta);
  const bool big = coo && !inl && nnz > 4;  // second word: entries 4..7 (values follow a
                                            // 4-entry COO tile of a value matrix)
  if (__ballot(big) != 0ull) {
    f |= big ? coo_or4(pw1, m) : 0u;
    if (__ballot(big && nnz > 8) != 0ull && big && nnz > 8) {
      const uint32_t *w = (const uint32_t *)(payload + meta_vp(meta));
      const uint32_t lastw = (nnz - 1) >> 2;
      for (uint32_t k = 2; k <= lastw; ++k) f |= coo_or4(w[k], m);
    }
  }
  return f;
}

// ---------------------------------------------------------------------------
// PLUS_TIMES over the row-major larger tiles of one pull segment (Dense,
// ForceCSR, patched CSR), four tiles per step: quarter q of the wave takes one
// tile, lane (q, r) its row r.  A lane reads its row mask (Dense: all 16),
// the x entry of column r of its tile's column block (masked by blk_x_mask),
// derives row_ptr[r] as the quarter's prefix sum of the row counts, then
// reads the row's values (contiguous, at most 16) with dword-aligned wide
// loads.  Products walk the row's stored columns in order; the x value of a
// column comes from the lane of the quarter that holds it.  Four tiles cost
// five vector memory instructions (bf16), against about ten per tile when the
// whole wave works on one tile.  `pay` must extend at least 64 bytes past
// the last value; `xr` covers the block-padded x.  Returns lane (q, r)'s
// partial for row r, to be summed over the quarters.
// ---------------------------------------------------------------------------
// One step's four tiles: this lane's tile (lane of the segment, wave-uniform
// per quarter), its metadata, and the row mask and x entry in flight.
struct RowsStep {
  uint32_t mk, c, vp, tyn;  // active columns, column block, payload offset, type | nnz << 8
  uint32_t rmk;             // row mask (Dense: loaded as 0, all 16 later)
  uint32_t xw;              // raw x entry of column r
  bool valid;
};

// first stage: take the next four tiles of `todo` and issue their row-mask
// and x loads (used only by later stages, so they stay in flight)
template <int VK>
DBS_DEV RowsStep rows_issue(brsrc_t pay, brsrc_t xr, uint64_t &todo, uint64_t meta, uint32_t m, uint32_t cb,
                            uint32_t q, uint32_t r) {
  int l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    l[k] = todo ? __ffsll((unsigned long long)todo) - 1 : -1;
    todo &= todo - 1;
  }
  const int src = q == 0 ? l[0] : q == 1 ? l[1] : q == 2 ? l[2] : l[3];
  RowsStep t;
  t.valid = src >= 0;
  const int sl = t.valid ? src : 0;
  const uint64_t mt = (uint64_t)(uint32_t)__shfl((int)(uint32_t)meta, sl) |
                      ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(meta >> 32), sl) << 32);
  // every lane takes part in each shuffle (a lane outside EXEC reads as 0
  // to the others), the mask is applied afterwards
  const uint32_t mall = (uint32_t)__shfl((int)m, sl);
  t.mk = t.valid ? mall : 0u;
  t.c = (uint32_t)__shfl((int)cb, sl);
  t.vp = (uint32_t)meta_vp(mt);
  const uint32_t ty = meta_type(mt);
  t.tyn = ty | (meta_nnz(mt) << 8);
  const bool dn = ty == DBS_TILE_DENSE;
  t.rmk = __builtin_amdgcn_raw_buffer_load_b16(pay, (t.valid & !dn) ? t.vp + 2u * r : OOB_OFF, 0, 0);
  if (VK == VK_F32) t.xw = __builtin_amdgcn_raw_buffer_load_b32(xr, t.valid ? (t.c * 16u + r) * 4u : OOB_OFF, 0, 0);
  else t.xw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(xr, t.valid ? (t.c * 16u + r) * 2u : OOB_OFF, 0, 0);
  return t;
}

// values of this lane's row, raw: 16 dwords (fp32) or 9 dwords holding the
// row's bf16 values from a dword boundary
template <int VK>
struct RowVals {
  uint32_t w[VK == VK_F32 ? 16 : 9];
};

// second stage: the row mask is in; derive the row's value offset (the
// quarter's prefix sum of row counts) and issue the value loads
template <int VK>
DBS_DEV RowVals<VK> rows_values(brsrc_t pay, RowsStep &t, uint32_t r) {
  constexpr uint32_t VS = VK == VK_F32 ? 4u : 2u;
  const uint32_t ty = t.tyn & 0xFFu;
  const bool dn = ty == DBS_TILE_DENSE;
  t.rmk = (t.valid & dn) ? 0xFFFFu : t.rmk;
  const uint32_t cnt = (uint32_t)__popc(t.rmk);
  const uint32_t rp = quarter_incl_scan(cnt) - cnt;
  const uint32_t vbase = ty == DBS_TILE_CSR ? csr_val_off(t.tyn >> 8) : (uint32_t)PL_FORCE_VAL;
  const uint32_t voff = dn ? t.vp + r * 16u * VS : t.vp + vbase + rp * VS;
  const uint32_t lo = cnt ? (voff & ~3u) : OOB_OFF;
  t.vp = voff;  // from here on: the row's value offset (its parity picks the bf16 half)
  RowVals<VK> v;
  if (VK == VK_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(pay, cnt ? lo + 16u * j : OOB_OFF, 0, 0);
      v.w[4 * j] = w[0];
      v.w[4 * j + 1] = w[1];
      v.w[4 * j + 2] = w[2];
      v.w[4 * j + 3] = w[3];
    }
  } else {
    const auto wa = __builtin_amdgcn_raw_buffer_load_b128(pay, lo, 0, 0);
    const auto wb = __builtin_amdgcn_raw_buffer_load_b128(pay, cnt ? lo + 16u : OOB_OFF, 0, 0);
    v.w[0] = wa[0];
    v.w[1] = wa[1];
    v.w[2] = wa[2];
    v.w[3] = wa[3];
    v.w[4] = wb[0];
    v.w[5] = wb[1];
    v.w[6] = wb[2];
    v.w[7] = wb[3];
    v.w[8] = __builtin_amdgcn_raw_buffer_load_b32(pay, cnt ? lo + 32u : OOB_OFF, 0, 0);
  }
  return v;
}

// last stage: products over the row's stored columns, in order; the x value
// of a column comes from the lane of the quarter that holds it.  Entries go
// four at a time with fixed register indices (their gathers batched); a
// lane's entries past its row's count add nothing.
template <int VK, int K0>
DBS_DEV void rows_chunk(const RowVals<VK> &vw, uint32_t sh, float xt, uint32_t qb, uint32_t cnt, uint32_t &rest,
                        float &part) {
  float v[4];
  if (VK == VK_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(vw.w[K0 + i]);
  } else {
    // the row's entries K0..K0+3 from a dword boundary (sh = 16: the row
    // starts in the upper half of a dword)
    const uint32_t u0 = __builtin_amdgcn_alignbit(vw.w[K0 / 2 + 1], vw.w[K0 / 2], sh);
    const uint32_t u1 = __builtin_amdgcn_alignbit(vw.w[K0 / 2 + 2], vw.w[K0 / 2 + 1], sh);
    v[0] = __uint_as_float(u0 << 16);
    v[1] = __uint_as_float(u0 & 0xFFFF0000u);
    v[2] = __uint_as_float(u1 << 16);
    v[3] = __uint_as_float(u1 & 0xFFFF0000u);
  }
  uint32_t a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (qb | ((uint32_t)(__ffs(rest) - 1) & 15u)) << 2;
    rest &= rest - 1u;
  }
  float xv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((int)a[i], __float_as_int(xt)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pv = part + v[i] * xv[i];
    part = (K0 + i < (int)cnt) ? pv : part;
  }
}

template <int VK>
DBS_DEV float rows_products(const RowsStep &t, const RowVals<VK> &vw, uint32_t q, uint32_t r, float part) {
  float xt = VK == VK_F32 ? __uint_as_float(t.xw) : __uint_as_float(t.xw << 16);
  xt = ((t.mk >> r) & 1u) ? xt : 0.0f;
  const uint32_t cnt = (uint32_t)__popc(t.rmk);
  const uint32_t kmax = wave_max(cnt);
  const uint32_t sh = (t.vp & 2u) ? 16u : 0u;
  const uint32_t qb = q << 4;
  uint32_t rest = t.rmk;
  // the tile row's dot product on its own (at most 16 products), then one add
  float tp = 0.0f;
  if (kmax > 0u) rows_chunk<VK, 0>(vw, sh, xt, qb, cnt, rest, tp);  // uniform
  if (kmax > 4u) rows_chunk<VK, 4>(vw, sh, xt, qb, cnt, rest, tp);
  if (kmax > 8u) rows_chunk<VK, 8>(vw, sh, xt, qb, cnt, rest, tp);
  if (kmax > 12u) rows_chunk<VK, 12>(vw, sh, xt, qb, cnt, rest, tp);
  return part + tp;
}

// ---------------------------------------------------------------------------
// PLUS_TIMES over Dense tiles, four per step like rows_plus: lane (q, r)
// reads row r of its quarter's tile (16 values, zeros where the tile holds
// none) and takes column k's x from lane (q, k) by a row broadcast (DPP
// row_newbcast); bf16 values go in pairs through the bf16 dot product, x
// pairs held by lanes (q, 0..7).  No row mask and no prefix sum: a step is
// one round of loads.
// ---------------------------------------------------------------------------
template <int VK>
struct DenseStep {
  uint32_t mk;   // active columns of the lane's tile (0: no tile)
  uint32_t xw;   // bf16: x pair of columns 2(r&7), 2(r&7)+1; fp32: x of column r
  uint32_t w[VK == VK_F32 ? 16 : 8];
};

template <int VK>
DBS_DEV DenseStep<VK> dense_issue(brsrc_t pay, brsrc_t xr, uint64_t &todo, uint64_t meta, uint32_t m, uint32_t cb,
                                  uint32_t q, uint32_t r) {
  int l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    l[k] = todo ? __ffsll((unsigned long long)todo) - 1 : -1;
    todo &= todo - 1;
  }
  const int src = q == 0 ? l[0] : q == 1 ? l[1] : q == 2 ? l[2] : l[3];
  const bool valid = src >= 0;
  const int sl = valid ? src : 0;
  const uint64_t mt = (uint64_t)(uint32_t)__shfl((int)(uint32_t)meta, sl) |
                      ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(meta >> 32), sl) << 32);
  const uint32_t mall = (uint32_t)__shfl((int)m, sl);
  const uint32_t c = (uint32_t)__shfl((int)cb, sl);
  DenseStep<VK> t;
  t.mk = valid ? mall : 0u;
  const uint32_t vp = (uint32_t)meta_vp(mt);
  if (VK == VK_F32) {
    t.xw = __builtin_amdgcn_raw_buffer_load_b32(xr, valid ? (c * 16u + r) * 4u : OOB_OFF, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(pay, valid ? vp + r * 64u + 16u * j : OOB_OFF, 0, 0);
      t.w[4 * j] = w[0];
      t.w[4 * j + 1] = w[1];
      t.w[4 * j + 2] = w[2];
      t.w[4 * j + 3] = w[3];
    }
  } else {
    t.xw = __builtin_amdgcn_raw_buffer_load_b32(xr, valid ? (c * 16u + 2u * (r & 7u)) * 2u : OOB_OFF, 0, 0);
    const auto wa = __builtin_amdgcn_raw_buffer_load_b128(pay, valid ? vp + r * 32u : OOB_OFF, 0, 0);
    const auto wb = __builtin_amdgcn_raw_buffer_load_b128(pay, valid ? vp + r * 32u + 16u : OOB_OFF, 0, 0);
    t.w[0] = wa[0];
    t.w[1] = wa[1];
    t.w[2] = wa[2];
    t.w[3] = wa[3];
    t.w[4] = wb[0];
    t.w[5] = wb[1];
    t.w[6] = wb[2];
    t.w[7] = wb[3];
  }
  return t;
}

// lane (q, K)'s value to every lane of quarter q
template <int K>
DBS_DEV uint32_t quarter_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + K, 0xF, 0xF, true);
}

typedef __bf16 dbs_bf16x2 __attribute__((ext_vector_type(2)));

template <int VK, int K = 0>
DBS_DEV float dense_dot(const uint32_t (&w)[VK == VK_F32 ? 16 : 8], uint32_t xm, float part) {
  if constexpr (K < (VK == VK_F32 ? 16 : 8)) {
    const uint32_t xb = quarter_bcast<K>(xm);
    if constexpr (VK == VK_F32) {
      part = fmaf(__uint_as_float(w[K]), __uint_as_float(xb), part);
    } else {
      part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dbs_bf16x2, w[K]), __builtin_bit_cast(dbs_bf16x2, xb),
                                             part, false);
    }
    return dense_dot<VK, K + 1>(w, xm, part);
  } else {
    return part;
  }
}

template <int VK>
DBS_DEV float dense_products(const DenseStep<VK> &t, uint32_t r, float part) {
  uint32_t xm;
  if (VK == VK_F32) {
    xm = ((t.mk >> r) & 1u) ? t.xw : 0u;
  } else {
    const uint32_t m2 = t.mk >> (2u * (r & 7u));
    xm = t.xw & (((m2 & 1u) ? 0x0000FFFFu : 0u) | ((m2 & 2u) ? 0xFFFF0000u : 0u));
  }
  // the tile row's dot product on its own (at most 16 products), then one add
  return part + dense_dot<VK>(t.w, xm, 0.0f);
}

template <int VK>
DBS_DEV float dense_plus(brsrc_t pay, brsrc_t xr, uint64_t todo, uint64_t meta, uint32_t m, uint32_t cb, int lane) {
  const uint32_t q = (uint32_t)lane >> 4, r = (uint32_t)lane & 15u;
  float part = 0.0f;
  // step b's loads are in flight while step a's products run (a and b
  // alternate; the next step is issued even when no tile remains, so that
  // the wait for a step does not wait for the one after it)
  DenseStep<VK> a = dense_issue<VK>(pay, xr, todo, meta, m, cb, q, r);
  while (true) {
    const bool more_b = todo != 0ull;  // uniform
    const DenseStep<VK> b = dense_issue<VK>(pay, xr, todo, meta, m, cb, q, r);
    part = dense_products<VK>(a, r, part);
    if (!more_b) break;
    const bool more_a = todo != 0ull;
    a = dense_issue<VK>(pay, xr, todo, meta, m, cb, q, r);
    part = dense_products<VK>(b, r, part);
    if (!more_a) break;
  }
  return part;
}

template <int VK>
DBS_DEV float rows_plus(brsrc_t pay, brsrc_t xr, uint64_t todo, uint64_t meta, uint32_t m, uint32_t cb, int lane) {
  const uint32_t q = (uint32_t)lane >> 4, r = (uint32_t)lane & 15u;
  float part = 0.0f;
  // two steps in flight: while step a's values load and its products run,
  // step b's row masks and x entries are on their way (a and b alternate,
  // so that no in-flight register is copied).  The next step is issued
  // whether or not tiles remain (then with every lane out of range), so
  // that the waits for a step's values do not also wait for it.
  RowsStep a = rows_issue<VK>(pay, xr, todo, meta, m, cb, q, r);
  while (true) {
    const RowVals<VK> va = rows_values<VK>(pay, a, r);
    const bool more_b = todo != 0ull;  // uniform
    RowsStep b = rows_issue<VK>(pay, xr, todo, meta, m, cb, q, r);
    part = rows_products<VK>(a, va, q, r, part);
    if (!more_b) break;
    const RowVals<VK> vb = rows_values<VK>(pay, b, r);
    const bool more_a = todo != 0ull;
    a = rows_issue<VK>(pay, xr, todo, meta, m, cb, q, r);
    part = rows_products<VK>(b, vb, q, r, part);
    if (!more_a) break;
  }
  return part;
}
