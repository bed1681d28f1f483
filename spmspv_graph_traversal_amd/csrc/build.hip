// Format builder: CSR -> dual-view blocked format (section 3.2.1 and Figure
// 5(b) of "DB-SpMSpV: Dual-View Blocked Sparse Matrix-Sparse Vector
// Multiplication for Dynamic GPU Workloads"), entirely on the GPU.
//
// Tiles are found by a 16-way merge: one aligned group of 16 lanes (a DPP
// row of the wave) owns one row block, one lane per row; each step takes the
// smallest column block over the 16 row cursors, which yields the tiles of
// the row block in ascending column-block order (the primary block-CSR order)
// together with each row's slice of the tile.  The merge runs three times
// (count, classify, fill) so that nothing per-nonzero has to be stored.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "common.h"

namespace {

constexpr int BT = 256;               // threads per block
constexpr int RB_PER_BLOCK = BT / 16;  // row blocks per block (4 per wave)

// flags of the CSR validation
enum { BAD_FIRST = 1, BAD_LAST = 2, BAD_PTR = 4, BAD_COL = 8, BAD_ORDER = 16 };

// Rows with more entries than this are checked by a whole workgroup
// (k_validate_long): a thread walking a row of a million entries alone would
// set the time of the whole check.
constexpr int64_t VAL_LONG = 1024;

// flag[0]: the flags; flag[1]: number of long rows listed in long_rows
// (room for nnz / (VAL_LONG + 1) + 1 of them)
__global__ __launch_bounds__(BT) void k_validate(int32_t m, int32_t n, int64_t nnz,
                                                 const int32_t *row_ptr, const int32_t *col_idx,
                                                 uint32_t *flag, uint32_t *long_rows) {
  const int64_t i = (int64_t)blockIdx.x * BT + threadIdx.x;
  if (i >= m) return;
  const int64_t a = row_ptr[i], b = row_ptr[i + 1];
  uint32_t f = 0;
  if (i == 0 && a != 0) f |= BAD_FIRST;
  if (i == m - 1 && b != nnz) f |= BAD_LAST;
  if (a < 0 || b < a || b > nnz) {
    atomicOr(flag, f | BAD_PTR);
    return;
  }
  if (b - a > VAL_LONG) {
    // when every row passes the pointer check the pointers never decrease,
    // the rows do not overlap and at most nnz / (VAL_LONG + 1) of them are
    // this long; otherwise BAD_PTR is set for some row and the list stops at
    // its room
    const uint32_t p = atomicAdd(flag + 1, 1u);
    if ((int64_t)p <= nnz / (VAL_LONG + 1)) long_rows[p] = (uint32_t)i;
    if (f) atomicOr(flag, f);
    return;
  }
  int64_t prev = -1;
  for (int64_t k = a; k < b; ++k) {
    const int64_t c = col_idx[k];
    if (c < 0 || c >= n) f |= BAD_COL;
    if (c <= prev) f |= BAD_ORDER;
    prev = c;
  }
  if (f) atomicOr(flag, f);
}

// the listed long rows, a workgroup per row: every entry is compared with the
// one before it in the same row
__global__ __launch_bounds__(BT) void k_validate_long(int32_t n, int64_t nnz, const int32_t *row_ptr,
                                                      const int32_t *col_idx, uint32_t *flag,
                                                      const uint32_t *long_rows) {
  const uint32_t room = (uint32_t)(nnz / (VAL_LONG + 1) + 1);
  const uint32_t cnt = flag[1] < room ? flag[1] : room;
  for (uint32_t j = blockIdx.x; j < cnt; j += gridDim.x) {
    const int64_t r = long_rows[j];
    const int64_t a = row_ptr[r], b = row_ptr[r + 1];  // checked by k_validate: 0 <= a <= b <= nnz
    uint32_t f = 0;
    for (int64_t k = a + threadIdx.x; k < b; k += BT) {
      const int64_t c = col_idx[k];
      if (c < 0 || c >= n) f |= BAD_COL;
      if (k > a && c <= (int64_t)col_idx[k - 1]) f |= BAD_ORDER;
    }
    if (f) atomicOr(flag, f);
  }
}

// Rows that hold an entry, 16 bits per row block (two row blocks a word).
// BFS starts with the empty rows marked visited: nothing can reach them.
__global__ __launch_bounds__(BT) void k_rows_nz(int32_t m, int64_t words, const int32_t *row_ptr, uint32_t *out) {
  const int64_t k = (int64_t)blockIdx.x * BT + threadIdx.x;
  if (k >= words) return;
  uint32_t w = 0;
  for (int i = 0; i < 32; ++i) {
    const int64_t r = k * 32 + i;
    if (r < m && row_ptr[r + 1] > row_ptr[r]) w |= 1u << i;
  }
  out[k] = w;
}

// Per-lane row cursor of the merge.
struct RowCursor {
  int64_t p, e;
};

// Merge items: a row block whose rows hold more than LONG_RB_NNZ entries is
// merged in pieces of CHUNK_CB column blocks, one 16-lane group each (the
// merge walks a row block's tiles one after another, so a hub row block's
// walk set the build time); the others are one item each.  Item i covers
// row block item_rb[i], column blocks [item_lo[i], item_hi[i]), and its tiles
// start at item_off[i] in block-CSR order.
constexpr int64_t LONG_RB_NNZ = 4096;
constexpr uint32_t CHUNK_CB = 64;

struct Items {
  const uint32_t *rb, *lo, *hi;
  int64_t n;
};

// first position in [p, e) whose column is >= col (entries sorted)
DBS_DEV int64_t lower_col(const int32_t *col_idx, int64_t p, int64_t e, int64_t col) {
  while (p < e) {
    const int64_t mid = p + ((e - p) >> 1);
    if ((int64_t)col_idx[mid] < col) p = mid + 1;
    else e = mid;
  }
  return p;
}

// lane r's cursor over its row's entries in the item's column-block range
DBS_DEV RowCursor item_cursor(int32_t m, const int32_t *row_ptr, const int32_t *col_idx, uint32_t rb,
                              uint32_t lo, uint32_t hi, int r) {
  RowCursor c{0, 0};
  const int64_t row = (int64_t)rb * DBS_TILE + r;
  if (row < m) {
    c.p = row_ptr[row];
    c.e = row_ptr[row + 1];
    if (lo != 0u) c.p = lower_col(col_idx, c.p, c.e, (int64_t)lo * DBS_TILE);
    if (hi != 0xFFFFFFFFu) c.e = lower_col(col_idx, c.p, c.e, (int64_t)hi * DBS_TILE);
  }
  return c;
}

DBS_DEV uint32_t cursor_cb(const RowCursor &c, const int32_t *col_idx) {
  return c.p < c.e ? ((uint32_t)col_idx[c.p] >> 4) : 0xFFFFFFFFu;
}

// advance the cursor over the entries of column block `cb`; returns the row's
// 16-bit mask of local columns in this tile
DBS_DEV uint32_t cursor_take(RowCursor &c, const int32_t *col_idx, uint32_t cb) {
  uint32_t rm = 0;
  while (c.p < c.e) {
    const uint32_t col = (uint32_t)col_idx[c.p];
    if ((col >> 4) != cb) break;
    rm |= 1u << (col & 15u);
    ++c.p;
  }
  return rm;
}

// column masks of the tile: lane r (of the 16-lane group) returns the mask of
// local rows holding an entry in local column r
DBS_DEV uint32_t transpose_masks16(uint32_t rm, int r) {
  uint32_t cm = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t v = (uint32_t)__shfl((int)rm, k, 16);
    cm |= ((v >> r) & 1u) << k;
  }
  return cm;
}

// Tile format from nnz and the largest row / column counts (section 3.2.1).
// skew_r / skew_c = max_row / max_col because both skews divide by
// nnz / 16 + eps, so the th2 tests are exact integer comparisons.
DBS_DEV uint32_t classify_tile(uint32_t nnz, uint32_t maxr, uint32_t maxc,
                               const dbs_build_options &o) {
  if (o.force_format >= 0) return (uint32_t)o.force_format;
  if ((int)nnz < o.th0) return DBS_TILE_COO;
  if ((int)nnz > o.th1) return DBS_TILE_DENSE;
  if ((uint64_t)maxr * (uint64_t)o.th2_den > (uint64_t)maxc * (uint64_t)o.th2_num)
    return DBS_TILE_FORCE_CSC;
  if ((uint64_t)maxc * (uint64_t)o.th2_den > (uint64_t)maxr * (uint64_t)o.th2_num)
    return DBS_TILE_FORCE_CSR;
  return DBS_TILE_CSR;
}

// Items: the number of merge items of each row block and the first column
// block's chunk of a long one.  One thread per row block.
__global__ void k_rb_items(int32_t m, int32_t mb, const int32_t *row_ptr, const int32_t *col_idx, uint32_t *nitem,
                           uint32_t *chunk0) {
  const int64_t rb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rb >= mb) return;
  const int64_t r0 = rb * DBS_TILE, r1 = r0 + DBS_TILE < m ? r0 + DBS_TILE : m;
  uint32_t n = 1, c0 = 0;
  if ((int64_t)row_ptr[r1] - row_ptr[r0] > LONG_RB_NNZ) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
    for (int64_t row = r0; row < r1; ++row) {
      const int64_t a = row_ptr[row], b = row_ptr[row + 1];
      if (a < b) {
        const uint32_t f = (uint32_t)col_idx[a] >> 4, l = (uint32_t)col_idx[b - 1] >> 4;
        lo = f < lo ? f : lo;
        hi = l > hi ? l : hi;
      }
    }
    c0 = lo / CHUNK_CB;
    n = hi / CHUNK_CB - c0 + 1;
  }
  nitem[rb] = n;
  chunk0[rb] = c0;
}

// the items themselves: (row block, column-block range); one thread per row block
__global__ void k_fill_items(int32_t mb, const uint32_t *nitem, const uint32_t *item_start, const uint32_t *chunk0,
                             uint32_t *item_rb, uint32_t *item_lo, uint32_t *item_hi) {
  const int64_t rb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rb >= mb) return;
  const uint32_t n = nitem[rb], s0 = item_start[rb];
  if (n == 1u) {
    item_rb[s0] = (uint32_t)rb;
    item_lo[s0] = 0u;
    item_hi[s0] = 0xFFFFFFFFu;
    return;
  }
  for (uint32_t j = 0; j < n; ++j) {
    item_rb[s0 + j] = (uint32_t)rb;
    item_lo[s0 + j] = (chunk0[rb] + j) * CHUNK_CB;
    item_hi[s0 + j] = (chunk0[rb] + j + 1) * CHUNK_CB;
  }
}

// block-CSR row pointer: the first tile of each row block's first item
__global__ void k_rb_ptr_from_items(int32_t mb, const uint32_t *item_start, const uint32_t *item_off, int64_t ni,
                                    uint32_t *rb_ptr) {
  const int64_t rb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rb > mb) return;
  rb_ptr[rb] = rb < mb ? item_off[item_start[rb]] : item_off[ni];
}

// pass 1: tiles per item
__global__ __launch_bounds__(BT) void k_tile_count(int32_t m, const int32_t *row_ptr, const int32_t *col_idx,
                                                   Items it, uint32_t *item_cnt) {
  const int r = threadIdx.x & 15;
  const int64_t i = (int64_t)blockIdx.x * RB_PER_BLOCK + (int64_t)(threadIdx.x >> 4);
  RowCursor c{0, 0};
  if (i < it.n) c = item_cursor(m, row_ptr, col_idx, it.rb[i], it.lo[i], it.hi[i], r);
  uint32_t cnt = 0;
  while (true) {
    const uint32_t cb = group_min_u32<16>(cursor_cb(c, col_idx));
    if (cb == 0xFFFFFFFFu) break;
    ++cnt;
    (void)cursor_take(c, col_idx, cb);
  }
  if (r == 0 && i < it.n) item_cnt[i] = cnt;
}

// pass 2: per tile column block, row block, nnz, format and payload size
__global__ __launch_bounds__(BT) void k_tile_classify(int32_t m, const int32_t *row_ptr, const int32_t *col_idx,
                                                      Items it, const uint32_t *item_off,
                                                      dbs_build_options o, int vk, int64_t T,
                                                      uint32_t *t_cb, uint32_t *t_rb, uint32_t *t_nt,
                                                      uint64_t *sizes) {
  const int r = threadIdx.x & 15;
  const int64_t i = (int64_t)blockIdx.x * RB_PER_BLOCK + (int64_t)(threadIdx.x >> 4);
  RowCursor c{0, 0};
  uint32_t rb = 0;
  if (i < it.n) {
    rb = it.rb[i];
    c = item_cursor(m, row_ptr, col_idx, rb, it.lo[i], it.hi[i], r);
  }
  int64_t t = i < it.n ? (int64_t)item_off[i] : 0;
  while (true) {
    const uint32_t cb = group_min_u32<16>(cursor_cb(c, col_idx));
    if (cb == 0xFFFFFFFFu) break;
    const uint32_t rm = cursor_take(c, col_idx, cb);
    const uint32_t cm = transpose_masks16(rm, r);
    const uint32_t nnz = group_sum_u32<16>((uint32_t)__popc(rm));
    const uint32_t maxr = group_max_u32<16>((uint32_t)__popc(rm));
    const uint32_t maxc = group_max_u32<16>((uint32_t)__popc(cm));
    const uint32_t type = classify_tile(nnz, maxr, maxc, o);
    if (r == 0) {
      t_cb[t] = cb;
      t_rb[t] = (uint32_t)rb;
      t_nt[t] = (nnz - 1) | (type << 16);
      const int sec = tile_section((int)type, vk);
      const uint64_t bytes = tile_payload_bytes((int)type, nnz, vk);
      sizes[t] = sec == 0 ? bytes : 0;
      sizes[T + t] = sec == 1 ? bytes : 0;
      sizes[2 * T + t] = sec == 2 ? bytes : 0;
    }
    ++t;
  }
}

__global__ void k_pack_meta(int64_t T, int vk, const uint32_t *t_nt, const uint64_t *off,
                            uint64_t *t_meta) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const uint32_t nt = t_nt[t];
  const uint32_t nnz = (nt & 0xFFFFu) + 1, type = nt >> 16;
  const int sec = tile_section((int)type, vk);
  t_meta[t] = meta_pack(off[(int64_t)sec * T + t], nnz, type);
}

template <int VK>
DBS_DEV void store_val(uint8_t *dst, const void *val, int64_t k) {
  if (VK == VK_F32) {
    *(float *)dst = ((const float *)val)[k];
  } else if (VK == VK_BF16) {
    *(uint16_t *)dst = ((const uint16_t *)val)[k];
  }
}
template <int VK>
DBS_DEV void store_zero(uint8_t *dst) {
  if (VK == VK_F32) *(float *)dst = 0.0f;
  else if (VK == VK_BF16) *(uint16_t *)dst = 0;
}

// pass 3: write every tile's payload in its format
template <int VK>
__global__ __launch_bounds__(BT) void k_tile_fill(int32_t m, const int32_t *row_ptr, const int32_t *col_idx,
                                                  const void *val, Items it, const uint32_t *item_off,
                                                  const uint64_t *t_meta, uint64_t *t_meta_w, uint8_t *payload,
                                                  uint64_t dense_mask_off, uint16_t *t_cm) {
  constexpr int VS = VK == VK_F32 ? 4 : VK == VK_BF16 ? 2 : 0;
  const int r = threadIdx.x & 15;
  const int64_t i = (int64_t)blockIdx.x * RB_PER_BLOCK + (int64_t)(threadIdx.x >> 4);
  RowCursor c{0, 0};
  if (i < it.n) c = item_cursor(m, row_ptr, col_idx, it.rb[i], it.lo[i], it.hi[i], r);
  int64_t t = i < it.n ? (int64_t)item_off[i] : 0;
  while (true) {
    const uint32_t cb = group_min_u32<16>(cursor_cb(c, col_idx));
    if (cb == 0xFFFFFFFFu) break;
    const int64_t p0 = c.p;
    const uint32_t rm = cursor_take(c, col_idx, cb);
    const uint32_t tcm = group_or_u32<16>(rm);  // the tile's columns with entries
    if (r == 0) t_cm[t] = (uint16_t)tcm;
    const uint32_t cnt = (uint32_t)__popc(rm);
    const uint32_t rp = group_incl_scan_u32<16>(cnt) - cnt;  // row start inside the tile
    const uint32_t cm = transpose_masks16(rm, r);            // lane r: column r
    const uint32_t ccnt = (uint32_t)__popc(cm);
    const uint32_t cp = group_incl_scan_u32<16>(ccnt) - ccnt;  // column start
    const uint64_t meta = t_meta[t];
    const uint32_t type = meta_type(meta), nnz = meta_nnz(meta);
    uint8_t *base = payload + meta_vp(meta);
    if (type == DBS_TILE_COO && coo_is_inline(VK, nnz)) {
      // coordinate bytes in row-major order; the unused bytes repeat the last
      // entry, so OR-AND readers may decode all four without a count check
      uint32_t word = 0;
      for (uint32_t j = 0; j < cnt; ++j)
        word |= ((r << 4) | ((uint32_t)col_idx[p0 + j] & 15u)) << (8 * (rp + j));
      if (cnt > 0 && rp + cnt == nnz) {
        const uint32_t last = (r << 4) | ((uint32_t)col_idx[p0 + cnt - 1] & 15u);
        for (uint32_t e = nnz; e < 4; ++e) word |= last << (8 * e);
      }
      word = group_or_u32<16>(word);
      if (r == 0) ((uint64_t *)t_meta_w)[t] = meta_pack(0, nnz, type) | META_INLINE | word;
    } else if (type == DBS_TILE_COO) {
      for (uint32_t j = 0; j < cnt; ++j) {
        const uint32_t col = (uint32_t)col_idx[p0 + j] & 15u;
        base[rp + j] = (uint8_t)((r << 4) | col);
        if (VS) store_val<VK>(base + coo_val_off(nnz) + (rp + j) * VS, val, p0 + j);
      }
      // padding to the 4-B boundary repeats the last entry (see above)
      if (cnt > 0 && rp + cnt == nnz) {
        const uint8_t last = (uint8_t)((r << 4) | ((uint32_t)col_idx[p0 + cnt - 1] & 15u));
        for (uint32_t e = nnz; e < align_up(nnz, 4); ++e) base[e] = last;
      }
    } else if (VK == VK_PAT) {
      ((uint16_t *)(base + PL_MASK))[r] = (uint16_t)rm;
      ((uint16_t *)(base + PL_PAT_COLMASK))[r] = (uint16_t)cm;
    } else if (type == DBS_TILE_DENSE) {
      ((uint16_t *)(payload + dense_mask_off + 32 * (meta_vp(meta) / (256 * VS))))[r] = (uint16_t)rm;
      uint32_t j = 0;
      for (int cc = 0; cc < 16; ++cc) {
        uint8_t *dst = base + (r * 16 + cc) * VS;
        if ((rm >> cc) & 1u) store_val<VK>(dst, val, p0 + (j++));
        else store_zero<VK>(dst);
      }
    } else if (type == DBS_TILE_FORCE_CSR) {
      ((uint16_t *)(base + PL_MASK))[r] = (uint16_t)rm;
      base[PL_PTR + r] = (uint8_t)rp;
      for (uint32_t j = 0; j < cnt; ++j) store_val<VK>(base + PL_FORCE_VAL + (rp + j) * VS, val, p0 + j);
    } else {
      // ForceCSC and patched CSR need every column's mask and start
      if (type == DBS_TILE_FORCE_CSC) {
        ((uint16_t *)(base + PL_MASK))[r] = (uint16_t)cm;
        base[PL_PTR + r] = (uint8_t)cp;
      } else {
        ((uint16_t *)(base + PL_MASK))[r] = (uint16_t)rm;
        base[PL_PTR + r] = (uint8_t)rp;
        base[PL_CSR_COLPTR + r] = (uint8_t)cp;
      }
      uint32_t j = 0;
#pragma unroll 1
      for (int cc = 0; cc < 16; ++cc) {
        const uint32_t cmc = (uint32_t)__shfl((int)cm, cc, 16);
        const uint32_t cpc = (uint32_t)__shfl((int)cp, cc, 16);
        if ((rm >> cc) & 1u) {
          const uint32_t pos = cpc + (uint32_t)__popc(cmc & below_mask((uint32_t)r));
          if (type == DBS_TILE_FORCE_CSC) {
            store_val<VK>(base + PL_FORCE_VAL + pos * VS, val, p0 + j);
          } else {
            base[PL_CSR_RC + pos] = (uint8_t)((r << 4) | j);
            store_val<VK>(base + csr_val_off(nnz) + (rp + j) * VS, val, p0 + j);
          }
          ++j;
        }
      }
    }
    ++t;
  }
}

__global__ void k_iota(uint32_t *v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) v[i] = (uint32_t)i;
}

__global__ void k_hist_cb(const uint32_t *t_cb, int64_t T, uint32_t *cnt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) atomicAdd(&cnt[t_cb[i]], 1u);
}

__global__ void k_gather_rb(const uint32_t *csc2csr, const uint32_t *t_rb, int64_t T,
                            uint32_t *csc_rb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) csc_rb[i] = t_rb[csc2csr[i]];
}

__global__ void k_gather_cm(const uint32_t *csc2csr, const uint16_t *t_cm, int64_t T, uint16_t *csc_cm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) csc_cm[i] = t_cm[csc2csr[i]];
}

DBS_DEV uint32_t seg_weight(uint32_t type, const dbs_build_options &o) {
  return type == DBS_TILE_DENSE ? (uint32_t)o.seg_w_dense
                                : type == DBS_TILE_COO ? (uint32_t)o.seg_w_coo : (uint32_t)o.seg_w_csr;
}

// Row blocks of more tiles than this are segmented by a workgroup each
// (k_segments_long): one thread walking a hub row block's tiles alone would
// set the time of the whole pass.
constexpr uint32_t SEG_LONG = 512;

// Pull load balance (section 3.3.2): greedy weighted segments inside each row
// block.  mode 0 counts, mode 1 writes.
__global__ void k_segments(int32_t mb, const uint32_t *rb_ptr, const uint32_t *t_nt,
                           dbs_build_options o, uint32_t *seg_cnt, const uint32_t *seg_off,
                           uint32_t *segs, int mode) {
  const int32_t rb = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
  if (rb >= mb) return;
  const uint32_t t0 = rb_ptr[rb], t1 = rb_ptr[rb + 1];
  if (t1 - t0 > SEG_LONG) return;  // k_segments_long
  uint32_t nseg = 0, acc = 0, start = t0;
  uint32_t out = mode ? seg_off[rb] : 0;
  const uint32_t split = (mode && seg_cnt[rb] > 1) ? SEG_SPLIT : 0u;
  for (uint32_t t = t0; t < t1; ++t) {
    acc += seg_weight(t_nt[t] >> 16, o);
    if (acc >= (uint32_t)o.seg_cap) {
      if (mode) {
        uint32_t *s = segs + 4 * (uint64_t)(out + nseg);
        s[0] = (uint32_t)rb | split;
        s[1] = start;
        s[2] = t + 1;
        s[3] = 0;
      }
      ++nseg;
      start = t + 1;
      acc = 0;
    }
  }
  if (start < t1) {
    if (mode) {
      uint32_t *s = segs + 4 * (uint64_t)(out + nseg);
      s[0] = (uint32_t)rb | split;
      s[1] = start;
      s[2] = t1;
      s[3] = 0;
    }
    ++nseg;
  }
  if (!mode) seg_cnt[rb] = nseg;
}

// The same rule for the row blocks of more than SEG_LONG tiles, a workgroup
// per row block, 256 tiles at a time: an inclusive prefix of the chunk's
// weights, then each close is the first tile after the previous one whose
// running weight reaches the cap (one ballot per close).
__global__ __launch_bounds__(BT) void k_segments_long(int32_t mb, const uint32_t *rb_ptr, const uint32_t *t_nt,
                                                      dbs_build_options o, uint32_t *seg_cnt,
                                                      const uint32_t *seg_off, uint32_t *segs, int mode) {
  __shared__ uint32_t s_pre[BT];
  __shared__ uint32_t s_min[BT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t cap = (uint32_t)o.seg_cap;
  for (int32_t rb = (int32_t)blockIdx.x; rb < mb; rb += (int32_t)gridDim.x) {
    const uint32_t t0 = rb_ptr[rb], t1 = rb_ptr[rb + 1];
    if (t1 - t0 <= SEG_LONG) continue;  // uniform
    const uint32_t out = mode ? seg_off[rb] : 0u;
    const uint32_t split = (mode && seg_cnt[rb] > 1) ? SEG_SPLIT : 0u;
    uint32_t nseg = 0, start = t0, acc = 0;  // uniform: running weight since the last close
    for (uint32_t c0 = t0; c0 < t1; c0 += BT) {
      const uint32_t t = c0 + (uint32_t)tid;
      const bool in = t < t1;
      __syncthreads();  // the previous chunk's reads of s_pre are done
      s_pre[tid] = in ? seg_weight(t_nt[t] >> 16, o) : 0u;
      __syncthreads();
      for (int d = 1; d < BT; d <<= 1) {
        const uint32_t add = tid >= d ? s_pre[tid - d] : 0u;
        __syncthreads();
        s_pre[tid] += add;
        __syncthreads();
      }
      const uint32_t pre = s_pre[tid];
      uint32_t off = 0;  // prefix at the last close inside this chunk
      int jlast = -1;    // that close's position in the chunk
      while (true) {     // uniform
        const bool hit = in && tid > jlast && acc + (pre - off) >= cap;
        const uint64_t b = __ballot(hit);
        if (lane == 0) s_min[wv] = b ? (uint32_t)(wv * 64 + __ffsll((unsigned long long)b) - 1) : (uint32_t)BT;
        __syncthreads();
        uint32_t j = s_min[0];
#pragma unroll
        for (int k = 1; k < BT / 64; ++k) j = s_min[k] < j ? s_min[k] : j;
        __syncthreads();
        if (j >= (uint32_t)BT) break;
        if (mode && tid == 0) {
          uint32_t *sg = segs + 4 * (uint64_t)(out + nseg);
          sg[0] = (uint32_t)rb | split;
          sg[1] = start;
          sg[2] = c0 + j + 1;
          sg[3] = 0;
        }
        ++nseg;
        start = c0 + j + 1;
        off = s_pre[j];
        acc = 0;
        jlast = (int)j;
      }
      acc += s_pre[BT - 1] - off;
    }
    if (start < t1) {
      if (mode && tid == 0) {
        uint32_t *sg = segs + 4 * (uint64_t)(out + nseg);
        sg[0] = (uint32_t)rb | split;
        sg[1] = start;
        sg[2] = t1;
        sg[3] = 0;
      }
      ++nseg;
    }
    if (!mode && tid == 0) seg_cnt[rb] = nseg;
  }
}

// Partial slots (value matrices): per row block, the slots its segments
// need (its segment count when above SEG_SLOT_MIN, else 0) and whether it
// is listed for the finalize.
__global__ void k_slot_counts(int32_t mb, const uint32_t *seg_cnt, uint32_t *nslot, uint32_t *isfin) {
  const int32_t rb = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
  if (rb >= mb) return;
  const uint32_t c = seg_cnt[rb];
  nslot[rb] = c > SEG_SLOT_MIN ? c : 0u;
  isfin[rb] = c > SEG_SLOT_MIN ? 1u : 0u;
}

// Class bits and slot of every segment of such a row block (segment j of
// row block rb takes slot slot_off[rb] + j), and the finalize list entry
// {row block, first slot, segments, class} of each; the largest class goes
// to *maxcls (one atomic per wave).
__global__ void k_slots(int64_t nseg, uint32_t *segs, const uint32_t *seg_cnt, const uint32_t *seg_off,
                        const uint32_t *slot_off, const uint32_t *fin_off, uint32_t *fin, uint32_t *maxcls) {
  const int64_t sg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t cls = 0;
  if (sg < nseg) {
    const uint32_t rb = segs[4 * sg] & SEG_RB_MASK;
    const uint32_t c = seg_cnt[rb];
    cls = seg_class(c);
    if (cls) {
      const uint32_t j = (uint32_t)sg - seg_off[rb];
      segs[4 * sg] |= cls << SEG_CLS_SHIFT;
      segs[4 * sg + 3] = slot_off[rb] + j + 1u;
      if (j == 0) {
        uint32_t *f = fin + 4 * (uint64_t)fin_off[rb];
        f[0] = rb;
        f[1] = slot_off[rb];
        f[2] = c;
        f[3] = cls;
      }
    }
  }
  cls = group_max_u32<64>(cls);
  if ((threadIdx.x & 63) == 0 && cls) atomicMax(maxcls, cls);
}

// Marks (SEG_DRAIN) the pull segments of a value matrix in which some row
// holds more than SEG_DRAIN_ROW entries of COO tiles: the wide PLUS_TIMES
// pull then empties its LDS row sums after every round of those segments.
// One thread per segment, counting its COO tiles' coordinate bytes per row.
__global__ void k_seg_drain(int64_t nseg, uint32_t *segs, const uint64_t *t_meta, const uint8_t *payload) {
  const int64_t sg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sg >= nseg) return;
  const uint32_t t0 = segs[4 * sg + 1], t1 = segs[4 * sg + 2];
  uint32_t cnt[16];
  for (int r = 0; r < 16; ++r) cnt[r] = 0;
  for (uint32_t t = t0; t < t1; ++t) {
    const uint64_t mt = t_meta[t];
    if (meta_type(mt) != DBS_TILE_COO) continue;
    const uint8_t *c = payload + meta_vp(mt);
    const uint32_t nz = meta_nnz(mt);
    for (uint32_t e = 0; e < nz; ++e) cnt[c[e] >> 4] += 1;
  }
  uint32_t mx = 0;
  for (int r = 0; r < 16; ++r) mx = cnt[r] > mx ? cnt[r] : mx;
  if (mx > SEG_DRAIN_ROW) segs[4 * sg] |= SEG_DRAIN;
}

__global__ void k_type_stats(const uint32_t *t_nt, int64_t T, unsigned long long *st) {
  __shared__ unsigned long long s[10];
  if (threadIdx.x < 10) s[threadIdx.x] = 0;
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t nt = t_nt[i];
    atomicAdd(&s[nt >> 16], 1ull);
    atomicAdd(&s[5 + (nt >> 16)], (unsigned long long)((nt & 0xFFFFu) + 1));
  }
  __syncthreads();
  if (threadIdx.x < 10) atomicAdd(&st[threadIdx.x], s[threadIdx.x]);
}

inline unsigned nblocks(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

// Work of a Boolean-pull segment, for ordering: its tiles, plus two per
// coordinate word and eight per tile read as row masks.  One thread per
// segment.
__global__ void k_seg_cost(const uint32_t *psegs, int64_t npseg, const uint64_t *t_meta, uint32_t *cost) {
  const int64_t sg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sg >= npseg) return;
  const uint32_t t0 = psegs[4 * sg + 1], t1 = psegs[4 * sg + 2];
  uint32_t c = 0;
  for (uint32_t t = t0; t < t1; ++t) {
    const uint64_t meta = t_meta[t];
    const uint32_t type = meta_type(meta);
    c += 1u + (type != DBS_TILE_COO ? 8u : meta_inline(meta) ? 0u : 2u * ((meta_nnz(meta) + 3u) / 4u));
  }
  cost[sg] = c;
}

// A pattern tile of one entry (held inline): with at most CBX_MAX_NB column
// blocks, the Boolean pull decodes it from its column-block word alone.
__host__ __device__ inline bool single_entry_tile(uint64_t meta) {
  return meta_type(meta) == DBS_TILE_COO && meta_nnz(meta) == 1u && meta_inline(meta);
}

// Owner of every coordinate word of a pattern COO tile held in the payload:
// the tile's rank in its Boolean-pull segment (< 256): its index among the
// segment's tiles not marked single (m2idx: the exclusive count of such tiles
// before each tile; null: every tile counts).  The pull spreads a segment's
// words over the lanes; with the owner stored, a lane finds the mask of its
// word's tile with one LDS read.  Also the tile's row block within its
// segment (0 .. PAT_MAX_RB-1), in bits 52..55 of its metadata word: a
// segment that packs several row blocks sends each found row to its row
// block by it.  And every tile's column-block word for the pull (t_cbx): the
// column block and that row block, and (m2idx given, at most CBX_MAX_NB
// column blocks) for a tile of one entry that entry, for the others their
// rank.  One thread per segment.
__global__ void k_word_owner(const uint32_t *psegs, int64_t npseg, const uint32_t *rb_ptr, uint64_t *t_meta,
                             uint8_t *wown, const uint32_t *m2idx, const uint32_t *t_cb, uint32_t *t_cbx) {
  const int64_t sg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sg >= npseg) return;
  const bool compact = m2idx != nullptr;
  const uint32_t rb = psegs[4 * sg], t0 = psegs[4 * sg + 1], t1 = psegs[4 * sg + 2], nrb = psegs[4 * sg + 3];
  uint32_t ri = 0, next = nrb > 1u ? rb_ptr[rb + 1] : t1;  // first tile of row block rb + ri + 1
  for (uint32_t t = t0; t < t1; ++t) {
    while (t >= next && ri + 1u < nrb) {
      ++ri;
      next = ri + 1u < nrb ? rb_ptr[rb + ri + 1u] : t1;
    }
    const uint64_t meta = (t_meta[t] & ~META_SEG_RB) | ((uint64_t)ri << META_SEG_RB_SHIFT);
    t_meta[t] = meta;
    const uint32_t rank = compact ? m2idx[t] - m2idx[t0] : t - t0;
    // the pull's column-block word
    uint32_t cw = t_cb[t] | (ri << (compact ? CBX_RI_SHIFT : CBX_RI_SHIFT_WIDE));
    if (compact)
      cw |= single_entry_tile(meta) ? CBX_SINGLE | (((uint32_t)meta & 0xFFu) << CBX_RC_SHIFT) : rank << CBX_RC_SHIFT;
    t_cbx[t] = cw;
    if (meta_type(meta) != DBS_TILE_COO || meta_inline(meta)) continue;
    const uint64_t w0 = meta_vp(meta) / 4, nw = (meta_nnz(meta) + 3u) / 4u;
    for (uint64_t w = 0; w < nw; ++w) wown[w0 + w] = (uint8_t)rank;
  }
}

// 1 for a tile whose metadata the Boolean pull reads (not single), else 0
__global__ void k_ranked_flags(const uint64_t *t_meta, int64_t T, uint32_t *flag) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) flag[t] = single_entry_tile(t_meta[t]) ? 0u : 1u;
}

// metadata of the tiles not marked single, in tile order.  One thread per tile.
__global__ void k_meta2(const uint64_t *t_meta, const uint32_t *m2idx, int64_t T, uint64_t *meta2) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  if (m2idx[t + 1] != m2idx[t]) meta2[m2idx[t]] = t_meta[t];
}

// per Boolean-pull segment: its first entry in meta2 and its entries (m2idx
// null: every tile has one, meta2 being t_meta).  One thread per segment.
__global__ void k_m2seg(const uint32_t *psegs, int64_t npseg, const uint32_t *m2idx, uint32_t *m2seg) {
  const int64_t sg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sg >= npseg) return;
  const uint32_t t0 = psegs[4 * sg + 1], t1 = psegs[4 * sg + 2];
  const uint32_t b = m2idx ? m2idx[t0] : t0, e = m2idx ? m2idx[t1] : t1;
  m2seg[2 * sg] = b;
  m2seg[2 * sg + 1] = e - b;
}

// Segments of the Boolean pull (pattern matrices), in the order it runs
// them: first, one segment per run of consecutive short row blocks (a
// single segment each above; at most PAT_MAX_RB row blocks and seg_cap tiles
// per run) and the first segment of every long row block; then the other
// segments of the long row blocks.  A BFS pull level runs the two parts as
// two launches: most rows of a long row block are found by its first
// segment, and the second launch skips the row blocks with nothing left to
// find.  Packing short row blocks keeps a wave's 256 lanes busy, and the
// pull's cost per segment is what bounds it.  Built on the host: one
// sequential pass over the row blocks.
hipError_t build_pull_order(dbs_matrix *A, const uint32_t *seg_cnt, hipStream_t s) {
  const int32_t mb = A->mb;
  const int64_t nseg = A->nseg;
  std::vector<uint32_t> cnt(mb), rbp(mb + 1), sg(4 * (size_t)nseg);
  hipError_t e = hipMemcpyAsync(cnt.data(), seg_cnt, (size_t)mb * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(rbp.data(), A->rb_ptr, (size_t)(mb + 1) * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && nseg > 0) e = hipMemcpyAsync(sg.data(), A->segs, (size_t)nseg * 16, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  const uint32_t cap = (uint32_t)A->bopt.seg_cap;
  std::vector<uint32_t> first, rest;
  first.reserve(4 * (size_t)mb);
  rest.reserve(4 * (size_t)nseg);
  auto put = [](std::vector<uint32_t> &v, uint32_t rb, uint32_t t0, uint32_t t1, uint32_t nrb) {
    v.push_back(rb);
    v.push_back(t0);
    v.push_back(t1);
    v.push_back(nrb);
  };
  int64_t run = -1;  // first row block of the open run of short row blocks
  auto close_run = [&](int32_t end_rb) {  // the run covers row blocks [run, end_rb]
    if (run >= 0) put(first, (uint32_t)run, rbp[run], rbp[end_rb + 1], (uint32_t)(end_rb - run + 1));
    run = -1;
  };
  int32_t last_short = -1;
  uint64_t o = 0;  // first segment of the row block in sg
  for (int32_t rb = 0; rb < mb; ++rb) {
    const uint32_t c = cnt[rb];
    if (c == 1u) {
      if (run >= 0 && (rbp[rb + 1] - rbp[run] > cap || rb - run + 1 > DBS_PAT_MAX_RB)) close_run(last_short);
      if (run < 0) run = rb;
      last_short = rb;
    } else if (c > 1u) {
      close_run(last_short);
      for (uint32_t j = 0; j < c; ++j) {
        const uint32_t *d = &sg[4 * (o + j)];
        put(j == 0 ? first : rest, d[0] & ~SEG_SPLIT, d[1], d[2], 1u);
      }
    }
    o += c;
  }
  close_run(last_short);
  A->nseg0 = (int64_t)first.size() / 4;
  A->npseg = A->nseg0 + (int64_t)rest.size() / 4;
  first.insert(first.end(), rest.begin(), rest.end());
  first.resize(first.size() + 4 * 16, 0u);  // 16 zeroed descriptors of padding
  e = dbs_dev_alloc(A, (void **)&A->psegs, first.size() * 4);
  if (e == hipSuccess) e = hipMemcpyAsync(A->psegs, first.data(), first.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e;
}

// Each launch's segments sorted by decreasing work: a wave takes every
// (number of waves)-th segment, so every wave gets one segment of each
// size class and the waves finish together (in list order, the waves that
// drew the long row blocks' segments ran up to a third longer than the
// median).  Row-block order does not matter to the pull.
template <class Tmp>
hipError_t order_by_cost(dbs_matrix *A, Tmp &tmp, hipStream_t s) {
  const int64_t np = A->npseg;
  uint32_t *dcost;
  hipError_t e = tmp.get((void **)&dcost, (size_t)np * 4);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_seg_cost, dim3(nblocks(np, 256)), dim3(256), 0, s, (const uint32_t *)A->psegs, np,
                     (const uint64_t *)A->t_meta, dcost);
  e = hipGetLastError();
  std::vector<uint32_t> cost(np), sg(4 * (size_t)np);
  if (e == hipSuccess) e = hipMemcpyAsync(cost.data(), dcost, (size_t)np * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sg.data(), A->psegs, (size_t)np * 16, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  std::vector<uint32_t> idx(np), out(4 * (size_t)np);
  for (int64_t i = 0; i < np; ++i) idx[i] = (uint32_t)i;
  auto by_cost = [&](uint32_t a, uint32_t b) { return cost[a] > cost[b]; };
  std::stable_sort(idx.begin(), idx.begin() + A->nseg0, by_cost);
  std::stable_sort(idx.begin() + A->nseg0, idx.end(), by_cost);
  for (int64_t i = 0; i < np; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = sg[4 * (size_t)idx[i] + j];
  e = hipMemcpyAsync(A->psegs, out.data(), (size_t)np * 16, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e;
}

// First column block of each segment (for ordering).  One thread per segment.
__global__ void k_seg_first_cb(const uint32_t *segs, int64_t nseg, const uint32_t *t_cb, uint32_t *key) {
  const int64_t sg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sg >= nseg) return;
  key[sg] = t_cb[segs[4 * sg + 1]];
}

// Order of the PLUS_TIMES pull's segments: the segments of the row blocks
// split into more than 64 segments (class 3) first, sorted by their first
// column block, then the others in row-block order.  The pull's waves take
// consecutive segments together, so the segments in flight of the long row
// blocks cover one window of columns: the x lines of that window are read
// into L2 once and used by every long row block whose band covers it,
// instead of once per row block.  (A long row block's segments already
// write their sums to slots or with atomics, in any order.)
template <class Tmp>
hipError_t order_long_by_column(dbs_matrix *A, Tmp &tmp, hipStream_t s) {
  const int64_t ns = A->nseg;
  uint32_t *dkey;
  hipError_t e = tmp.get((void **)&dkey, (size_t)ns * 4);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_seg_first_cb, dim3(nblocks(ns, 256)), dim3(256), 0, s, (const uint32_t *)A->segs, ns,
                     (const uint32_t *)A->t_cb, dkey);
  e = hipGetLastError();
  std::vector<uint32_t> key(ns), sg(4 * (size_t)ns), out(4 * (size_t)ns);
  if (e == hipSuccess) e = hipMemcpyAsync(key.data(), dkey, (size_t)ns * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sg.data(), A->segs, (size_t)ns * 16, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  std::vector<uint32_t> idx;
  idx.reserve(ns);
  for (int64_t i = 0; i < ns; ++i)
    if (((sg[4 * (size_t)i] >> SEG_CLS_SHIFT) & 3u) == 3u) idx.push_back((uint32_t)i);
  if (idx.empty()) return hipSuccess;
  std::stable_sort(idx.begin(), idx.end(), [&](uint32_t a, uint32_t b) { return key[a] < key[b]; });
  for (int64_t i = 0; i < ns; ++i)
    if (((sg[4 * (size_t)i] >> SEG_CLS_SHIFT) & 3u) != 3u) idx.push_back((uint32_t)i);
  for (int64_t i = 0; i < ns; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = sg[4 * (size_t)idx[i] + j];
  e = hipMemcpyAsync(A->segs, out.data(), (size_t)ns * 16, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e;
}

int bits_for(uint32_t maxval) {
  int b = 0;
  while (b < 32 && (maxval >> b) != 0) ++b;
  return b;
}

}  // namespace

// temporaries of the build, freed on every exit path
struct BuildTmp {
  static constexpr int kMax = 48;
  dbs_matrix *A;
  void *p[kMax] = {nullptr};
  size_t sz[kMax] = {0};
  int k = 0;
  explicit BuildTmp(dbs_matrix *a) : A(a) {}
  hipError_t get(void **out, size_t bytes) {
    if (k >= kMax) return hipErrorInvalidValue;
    void *q = nullptr;
    hipError_t e = dbs_dev_alloc(A, &q, bytes ? bytes : 1);
    if (e != hipSuccess) return e;
    p[k] = q;
    sz[k] = bytes ? bytes : 1;
    ++k;
    *out = q;
    return hipSuccess;
  }
  ~BuildTmp() {
    for (int i = 0; i < k; ++i) dbs_dev_free(A, p[i], sz[i]);
  }
};

#define BUILD_TRY(expr)                                                                     \
  do {                                                                                      \
    hipError_t e_ = DBS_NOTE(expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return (e_ == hipErrorOutOfMemory || e_ == hipErrorMemoryAllocation) ? DBS_ERR_OUT_OF_MEMORY \
                                                                        : DBS_ERR_DEVICE;  \
  } while (0)

dbs_status dbs_build_impl(dbs_matrix *A, const int32_t *row_ptr, const int32_t *col_idx,
                          const void *val, hipStream_t s) {
  BuildTmp tmp(A);
  const int32_t m = A->m, mb = A->mb, nb = A->nb;
  const int64_t nnz = A->nnz;
  const int vk = A->vk;

  // --- validate the CSR on the device
  uint32_t *flag, *long_rows;
  BUILD_TRY(tmp.get((void **)&flag, 8));
  BUILD_TRY(tmp.get((void **)&long_rows, (size_t)(nnz / (VAL_LONG + 1) + 1) * 4));
  BUILD_TRY(hipMemsetAsync(flag, 0, 8, s));
  hipLaunchKernelGGL(k_validate, dim3(nblocks(m, BT)), dim3(BT), 0, s, m, A->n, nnz, row_ptr,
                     col_idx, flag, long_rows);
  BUILD_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_validate_long, dim3(1024), dim3(BT), 0, s, A->n, nnz, row_ptr, col_idx, flag,
                     (const uint32_t *)long_rows);
  BUILD_TRY(hipGetLastError());
  uint32_t hflag = 0;
  BUILD_TRY(hipMemcpyAsync(&hflag, flag, 4, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipStreamSynchronize(s));
  if (hflag) return DBS_ERR_BAD_CSR;

  // --- rows holding an entry
  const int64_t rwords = ((int64_t)mb + 1) / 2;
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->rows_nz, (size_t)rwords * 4));
  hipLaunchKernelGGL(k_rows_nz, dim3(nblocks(rwords, BT)), dim3(BT), 0, s, m, rwords, row_ptr, A->rows_nz);
  BUILD_TRY(hipGetLastError());

  // --- merge items: one per row block, long row blocks in column-block pieces
  uint32_t *nitem, *chunk0, *item_start;
  BUILD_TRY(tmp.get((void **)&nitem, (size_t)mb * 4));
  BUILD_TRY(tmp.get((void **)&chunk0, (size_t)mb * 4));
  BUILD_TRY(tmp.get((void **)&item_start, (size_t)(mb + 1) * 4));
  void *stmp;
  BUILD_TRY(tmp.get(&stmp, dbs_scan_tmp_bytes((int64_t)mb + 1)));
  hipLaunchKernelGGL(k_rb_items, dim3(nblocks(mb, BT)), dim3(BT), 0, s, m, mb, row_ptr, col_idx, nitem, chunk0);
  BUILD_TRY(hipGetLastError());
  BUILD_TRY(dbs_scan_u32(nitem, item_start, mb, stmp, s));
  uint32_t hNI = 0;
  BUILD_TRY(hipMemcpyAsync(&hNI, item_start + mb, 4, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipStreamSynchronize(s));
  const int64_t NI = hNI;
  uint32_t *item_rb, *item_lo, *item_hi, *item_cnt, *item_off;
  BUILD_TRY(tmp.get((void **)&item_rb, (size_t)NI * 4 + 4));
  BUILD_TRY(tmp.get((void **)&item_lo, (size_t)NI * 4 + 4));
  BUILD_TRY(tmp.get((void **)&item_hi, (size_t)NI * 4 + 4));
  BUILD_TRY(tmp.get((void **)&item_cnt, (size_t)NI * 4 + 4));
  BUILD_TRY(tmp.get((void **)&item_off, (size_t)(NI + 1) * 4));
  void *stmpi;
  BUILD_TRY(tmp.get(&stmpi, dbs_scan_tmp_bytes(NI + 1)));
  hipLaunchKernelGGL(k_fill_items, dim3(nblocks(mb, BT)), dim3(BT), 0, s, mb, (const uint32_t *)nitem,
                     (const uint32_t *)item_start, (const uint32_t *)chunk0, item_rb, item_lo, item_hi);
  BUILD_TRY(hipGetLastError());
  const Items items{item_rb, item_lo, item_hi, NI};
  const unsigned gblocks = nblocks(NI, RB_PER_BLOCK);

  // --- pass 1: tiles per item, block-CSR row pointer
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->rb_ptr, (size_t)(mb + 1) * 4));
  hipLaunchKernelGGL(k_tile_count, dim3(gblocks), dim3(BT), 0, s, m, row_ptr, col_idx, items, item_cnt);
  BUILD_TRY(hipGetLastError());
  BUILD_TRY(dbs_scan_u32(item_cnt, item_off, NI, stmpi, s));
  hipLaunchKernelGGL(k_rb_ptr_from_items, dim3(nblocks((int64_t)mb + 1, BT)), dim3(BT), 0, s, mb,
                     (const uint32_t *)item_start, (const uint32_t *)item_off, NI, A->rb_ptr);
  BUILD_TRY(hipGetLastError());
  uint32_t hT = 0;
  BUILD_TRY(hipMemcpyAsync(&hT, A->rb_ptr + mb, 4, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipStreamSynchronize(s));
  const int64_t T = hT;
  A->T = T;

  // --- pass 2: classify tiles, payload sizes per section
  uint32_t *t_rb, *t_nt;
  uint64_t *sizes, *offs;
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->t_cb, (size_t)T * 4 + 4));
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->t_meta, (size_t)T * 8 + 8));
  BUILD_TRY(tmp.get((void **)&t_rb, (size_t)T * 4 + 4));
  BUILD_TRY(tmp.get((void **)&t_nt, (size_t)T * 4 + 4));
  BUILD_TRY(tmp.get((void **)&sizes, (size_t)3 * T * 8 + 8));
  BUILD_TRY(tmp.get((void **)&offs, (size_t)(3 * T + 1) * 8));
  void *stmp3;
  BUILD_TRY(tmp.get(&stmp3, dbs_scan_tmp_bytes(3 * T + 1)));
  hipLaunchKernelGGL(k_tile_classify, dim3(gblocks), dim3(BT), 0, s, m, row_ptr, col_idx, items,
                     (const uint32_t *)item_off, A->bopt, vk, T, A->t_cb, t_rb, t_nt, sizes);
  BUILD_TRY(hipGetLastError());
  BUILD_TRY(dbs_scan_u64(sizes, offs, 3 * T, stmp3, s));
  uint64_t total = 0, dense_bytes = 0;
  BUILD_TRY(hipMemcpyAsync(&total, offs + 3 * T, 8, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipMemcpyAsync(&dense_bytes, offs + T, 8, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipStreamSynchronize(s));
  // Dense row masks after the three value sections (value matrices only)
  A->dense_mask_off = (total + 127) & ~127ull;
  if (vk != VK_PAT) total = A->dense_mask_off + 32ull * (dense_bytes / (256ull * (uint64_t)vk_size(vk)));
  // (the 40-bit offsets of the metadata word are looser than this)
  if (!dbs_format_fits_offsets(total, (uint64_t)T)) return DBS_ERR_UNSUPPORTED;
  A->payload_bytes = (int64_t)total;
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->payload, (size_t)total + DBS_PAYLOAD_SLACK));
  BUILD_TRY(hipMemsetAsync(A->payload + total, 0, DBS_PAYLOAD_SLACK, s));
  if (T > 0) {
    hipLaunchKernelGGL(k_pack_meta, dim3(nblocks(T, BT)), dim3(BT), 0, s, T, vk, t_nt, offs, A->t_meta);
    BUILD_TRY(hipGetLastError());
  }

  // --- pass 3: payloads, and each tile's column set (CSR order)
  uint16_t *t_cm;
  BUILD_TRY(tmp.get((void **)&t_cm, (size_t)T * 2 + 2));
  if (vk == VK_F32)
    hipLaunchKernelGGL(k_tile_fill<VK_F32>, dim3(gblocks), dim3(BT), 0, s, m, row_ptr, col_idx, val, items,
                       (const uint32_t *)item_off, (const uint64_t *)A->t_meta, A->t_meta, A->payload,
                       A->dense_mask_off, t_cm);
  else if (vk == VK_BF16)
    hipLaunchKernelGGL(k_tile_fill<VK_BF16>, dim3(gblocks), dim3(BT), 0, s, m, row_ptr, col_idx, val, items,
                       (const uint32_t *)item_off, (const uint64_t *)A->t_meta, A->t_meta, A->payload,
                       A->dense_mask_off, t_cm);
  else
    hipLaunchKernelGGL(k_tile_fill<VK_PAT>, dim3(gblocks), dim3(BT), 0, s, m, row_ptr, col_idx, val, items,
                       (const uint32_t *)item_off, (const uint64_t *)A->t_meta, A->t_meta, A->payload,
                       A->dense_mask_off, t_cm);
  BUILD_TRY(hipGetLastError());

  // --- block-level CSC view: stable sort of the tiles by column block
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->cb_ptr, (size_t)(nb + 1) * 4));
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->csc_rb, (size_t)T * 4 + 4));
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->csc2csr, (size_t)T * 4 + 4));
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->csc_cm, (size_t)T * 2 + 2));
  uint32_t *keys, *keys_tmp, *vals_tmp, *cb_cnt;
  void *rtmp;
  BUILD_TRY(tmp.get((void **)&keys, (size_t)T * 4 + 4));
  BUILD_TRY(tmp.get((void **)&keys_tmp, (size_t)T * 4 + 4));
  BUILD_TRY(tmp.get((void **)&vals_tmp, (size_t)T * 4 + 4));
  BUILD_TRY(tmp.get((void **)&cb_cnt, (size_t)nb * 4));
  BUILD_TRY(tmp.get(&rtmp, dbs_radix_tmp_bytes(T)));
  void *stmpn;
  BUILD_TRY(tmp.get(&stmpn, dbs_scan_tmp_bytes((int64_t)nb + 1)));
  BUILD_TRY(hipMemsetAsync(cb_cnt, 0, (size_t)nb * 4, s));
  if (T > 0) {
    BUILD_TRY(hipMemcpyAsync(keys, A->t_cb, (size_t)T * 4, hipMemcpyDeviceToDevice, s));
    hipLaunchKernelGGL(k_iota, dim3(nblocks(T, BT)), dim3(BT), 0, s, A->csc2csr, T);
    hipLaunchKernelGGL(k_hist_cb, dim3(nblocks(T, BT)), dim3(BT), 0, s, (const uint32_t *)A->t_cb, T, cb_cnt);
    BUILD_TRY(hipGetLastError());
    BUILD_TRY(dbs_radix_sort_pairs(keys, A->csc2csr, keys_tmp, vals_tmp, T, bits_for((uint32_t)(nb - 1)),
                                   rtmp, s));
    hipLaunchKernelGGL(k_gather_rb, dim3(nblocks(T, BT)), dim3(BT), 0, s, (const uint32_t *)A->csc2csr,
                       (const uint32_t *)t_rb, T, A->csc_rb);
    BUILD_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_gather_cm, dim3(nblocks(T, BT)), dim3(BT), 0, s, (const uint32_t *)A->csc2csr,
                       (const uint16_t *)t_cm, T, A->csc_cm);
    BUILD_TRY(hipGetLastError());
  }
  BUILD_TRY(dbs_scan_u32(cb_cnt, A->cb_ptr, nb, stmpn, s));

  // --- pull segments
  uint32_t *seg_cnt, *seg_off;
  BUILD_TRY(tmp.get((void **)&seg_cnt, (size_t)mb * 4));
  BUILD_TRY(tmp.get((void **)&seg_off, (size_t)(mb + 1) * 4));
  hipLaunchKernelGGL(k_segments, dim3(nblocks(mb, BT)), dim3(BT), 0, s, mb, (const uint32_t *)A->rb_ptr,
                     (const uint32_t *)t_nt, A->bopt, seg_cnt, (const uint32_t *)nullptr,
                     (uint32_t *)nullptr, 0);
  BUILD_TRY(hipGetLastError());
  const unsigned lgrid = mb < 2048 ? (unsigned)mb : 2048u;
  hipLaunchKernelGGL(k_segments_long, dim3(lgrid), dim3(BT), 0, s, mb, (const uint32_t *)A->rb_ptr,
                     (const uint32_t *)t_nt, A->bopt, seg_cnt, (const uint32_t *)nullptr, (uint32_t *)nullptr, 0);
  BUILD_TRY(hipGetLastError());
  BUILD_TRY(dbs_scan_u32(seg_cnt, seg_off, mb, stmp, s));
  uint32_t hS = 0;
  BUILD_TRY(hipMemcpyAsync(&hS, seg_off + mb, 4, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipStreamSynchronize(s));
  A->nseg = hS;
  // padded with zeroed descriptors: the pull reads them in groups of up to 16
  BUILD_TRY(dbs_dev_alloc(A, (void **)&A->segs, ((size_t)hS + 16) * 16));
  BUILD_TRY(hipMemsetAsync(A->segs + 4 * (size_t)hS, 0, 16 * 16, s));
  hipLaunchKernelGGL(k_segments, dim3(nblocks(mb, BT)), dim3(BT), 0, s, mb, (const uint32_t *)A->rb_ptr,
                     (const uint32_t *)t_nt, A->bopt, seg_cnt, (const uint32_t *)seg_off, A->segs, 1);
  BUILD_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_segments_long, dim3(lgrid), dim3(BT), 0, s, mb, (const uint32_t *)A->rb_ptr,
                     (const uint32_t *)t_nt, A->bopt, seg_cnt, (const uint32_t *)seg_off, A->segs, 1);
  BUILD_TRY(hipGetLastError());
  if (vk != VK_PAT && hS > 0) {
    hipLaunchKernelGGL(k_seg_drain, dim3(nblocks(hS, BT)), dim3(BT), 0, s, (int64_t)hS, A->segs,
                       (const uint64_t *)A->t_meta, (const uint8_t *)A->payload);
    BUILD_TRY(hipGetLastError());
    // partial slots of the row blocks with more than SEG_SLOT_MIN segments
    uint32_t *nslot, *slot_off, *isfin, *fin_off, *maxcls;
    BUILD_TRY(tmp.get((void **)&nslot, (size_t)mb * 4));
    BUILD_TRY(tmp.get((void **)&slot_off, (size_t)(mb + 1) * 4));
    BUILD_TRY(tmp.get((void **)&isfin, (size_t)mb * 4));
    BUILD_TRY(tmp.get((void **)&fin_off, (size_t)(mb + 1) * 4 + 4));
    maxcls = fin_off + mb + 1;
    BUILD_TRY(hipMemsetAsync(maxcls, 0, 4, s));
    hipLaunchKernelGGL(k_slot_counts, dim3(nblocks(mb, BT)), dim3(BT), 0, s, mb, (const uint32_t *)seg_cnt, nslot,
                       isfin);
    BUILD_TRY(hipGetLastError());
    BUILD_TRY(dbs_scan_u32(nslot, slot_off, mb, stmp, s));
    BUILD_TRY(dbs_scan_u32(isfin, fin_off, mb, stmp, s));
    uint32_t hn[2] = {0, 0};
    BUILD_TRY(hipMemcpyAsync(&hn[0], slot_off + mb, 4, hipMemcpyDeviceToHost, s));
    BUILD_TRY(hipMemcpyAsync(&hn[1], fin_off + mb, 4, hipMemcpyDeviceToHost, s));
    BUILD_TRY(hipStreamSynchronize(s));
    A->nslots = hn[0];
    A->nfin = hn[1];
    // the pull addresses the slots with 32-bit byte offsets
    if ((uint64_t)A->nslots * DBS_MAX_SHARE * SLOT_WORDS * 4 >= 0xFFFFFFF0ull) return DBS_ERR_UNSUPPORTED;
    if (A->nfin > 0) {
      BUILD_TRY(dbs_dev_alloc(A, (void **)&A->fin, (size_t)A->nfin * 16));
      const size_t pbytes = (size_t)A->nslots * DBS_MAX_SHARE * SLOT_WORDS * 4;
      BUILD_TRY(dbs_dev_alloc(A, (void **)&A->partial, pbytes));
      BUILD_TRY(hipMemsetAsync(A->partial, 0, pbytes, s));  // no slot holds a valid epoch
      hipLaunchKernelGGL(k_slots, dim3(nblocks(hS, BT)), dim3(BT), 0, s, (int64_t)hS, A->segs,
                         (const uint32_t *)seg_cnt, (const uint32_t *)seg_off, (const uint32_t *)slot_off,
                         (const uint32_t *)fin_off, A->fin, maxcls);
      BUILD_TRY(hipGetLastError());
      uint32_t hm = 0;
      BUILD_TRY(hipMemcpyAsync(&hm, maxcls, 4, hipMemcpyDeviceToHost, s));
      // the finalize takes the list in order: longest row blocks first, so
      // that they do not start last
      std::vector<uint32_t> fl(4 * (size_t)A->nfin), fo(4 * (size_t)A->nfin);
      BUILD_TRY(hipMemcpyAsync(fl.data(), A->fin, (size_t)A->nfin * 16, hipMemcpyDeviceToHost, s));
      BUILD_TRY(hipStreamSynchronize(s));
      std::vector<uint32_t> ix((size_t)A->nfin);
      for (size_t i = 0; i < ix.size(); ++i) ix[i] = (uint32_t)i;
      std::stable_sort(ix.begin(), ix.end(), [&](uint32_t a, uint32_t b) { return fl[4 * (size_t)a + 2] > fl[4 * (size_t)b + 2]; });
      for (size_t i = 0; i < ix.size(); ++i)
        for (int j = 0; j < 4; ++j) fo[4 * i + j] = fl[4 * (size_t)ix[i] + j];
      BUILD_TRY(hipMemcpyAsync(A->fin, fo.data(), (size_t)A->nfin * 16, hipMemcpyHostToDevice, s));
      BUILD_TRY(hipStreamSynchronize(s));
      // sorted by segment count, the entries of class >= c come first
      for (int c = 0; c < 4; ++c) {
        int64_t k = 0;
        while (k < A->nfin && fo[4 * (size_t)k + 3] >= (uint32_t)c) ++k;
        A->fin_cls[c] = k;
      }
      for (int p = 0; p < 3; ++p) {
        int64_t k = 0;
        while (k < A->nfin && (uint64_t)fo[4 * (size_t)k + 2] * (1u << p) > 256u) ++k;
        A->fin_big[p] = k;
      }
      (void)hm;
      BUILD_TRY(order_long_by_column(A, tmp, s));
    }
  }
  if (vk == VK_PAT) {
    BUILD_TRY(build_pull_order(A, seg_cnt, s));
    const size_t ow = (size_t)(A->payload_bytes + DBS_PAYLOAD_SLACK) / 4;
    BUILD_TRY(dbs_dev_alloc(A, (void **)&A->wown, ow));
    BUILD_TRY(hipMemsetAsync(A->wown, 0, ow, s));
    // tiles of one entry are marked single (their metadata is not read by
    // the pull) when the column block leaves room for them in the word
    const bool compact = A->nb <= CBX_MAX_NB;
    uint32_t *m2idx = nullptr;
    A->nmeta2 = T;
    if (compact) {
      uint32_t *flag;
      void *stmpm;
      BUILD_TRY(tmp.get((void **)&flag, (size_t)T * 4 + 4));
      BUILD_TRY(tmp.get((void **)&m2idx, (size_t)T * 4 + 4));
      BUILD_TRY(tmp.get(&stmpm, dbs_scan_tmp_bytes(T + 1)));
      if (T > 0) {
        hipLaunchKernelGGL(k_ranked_flags, dim3(nblocks(T, BT)), dim3(BT), 0, s, (const uint64_t *)A->t_meta, T,
                           flag);
        BUILD_TRY(hipGetLastError());
      }
      BUILD_TRY(dbs_scan_u32(flag, m2idx, T, stmpm, s));
      uint32_t hn2 = 0;
      BUILD_TRY(hipMemcpyAsync(&hn2, m2idx + T, 4, hipMemcpyDeviceToHost, s));
      BUILD_TRY(hipStreamSynchronize(s));
      A->nmeta2 = hn2;
    }
    BUILD_TRY(dbs_dev_alloc(A, (void **)&A->t_cbx, (size_t)T * 4 + 4));
    if (A->npseg > 0) {
      hipLaunchKernelGGL(k_word_owner, dim3(nblocks(A->npseg, BT)), dim3(BT), 0, s, (const uint32_t *)A->psegs,
                         A->npseg, (const uint32_t *)A->rb_ptr, (uint64_t *)A->t_meta, A->wown,
                         (const uint32_t *)m2idx, (const uint32_t *)A->t_cb, A->t_cbx);
      BUILD_TRY(hipGetLastError());
      BUILD_TRY(order_by_cost(A, tmp, s));
    }
    if (compact) {
      BUILD_TRY(dbs_dev_alloc(A, (void **)&A->meta2, (size_t)(A->nmeta2 + 1) * 8));
      BUILD_TRY(hipMemsetAsync(A->meta2, 0, (size_t)(A->nmeta2 + 1) * 8, s));
      if (T > 0) {
        hipLaunchKernelGGL(k_meta2, dim3(nblocks(T, BT)), dim3(BT), 0, s, (const uint64_t *)A->t_meta,
                           (const uint32_t *)m2idx, T, A->meta2);
        BUILD_TRY(hipGetLastError());
      }
    } else {
      A->meta2 = A->t_meta;
    }
    const size_t m2b = (size_t)(A->npseg + 16) * 8;
    BUILD_TRY(dbs_dev_alloc(A, (void **)&A->m2seg, m2b));
    BUILD_TRY(hipMemsetAsync(A->m2seg, 0, m2b, s));
    if (A->npseg > 0) {
      hipLaunchKernelGGL(k_m2seg, dim3(nblocks(A->npseg, BT)), dim3(BT), 0, s, (const uint32_t *)A->psegs,
                         A->npseg, (const uint32_t *)m2idx, A->m2seg);
      BUILD_TRY(hipGetLastError());
    }
  }

  // --- statistics per format
  unsigned long long *st;
  BUILD_TRY(tmp.get((void **)&st, 10 * 8));
  BUILD_TRY(hipMemsetAsync(st, 0, 80, s));
  if (T > 0) {
    hipLaunchKernelGGL(k_type_stats, dim3(nblocks(T, BT) < 1024u ? nblocks(T, BT) : 1024u), dim3(BT), 0, s,
                       (const uint32_t *)t_nt, T, st);
    BUILD_TRY(hipGetLastError());
  }
  unsigned long long hst[10];
  BUILD_TRY(hipMemcpyAsync(hst, st, 80, hipMemcpyDeviceToHost, s));
  BUILD_TRY(hipStreamSynchronize(s));
  for (int i = 0; i < 5; ++i) {
    A->st.tiles_by_format[i] = (int64_t)hst[i];
    A->st.nnz_by_format[i] = (int64_t)hst[5 + i];
  }
  return DBS_OK;
}
