/*
 * CPU oracle for dual-view blocked SpMSpV, BFS and sparse decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library, and the HIP library never calls it.
 *
 * Every function is the plain definition, single-threaded, with fp64
 * accumulation.  Citations refer to the paper "DB-SpMSpV: Dual-View Blocked
 * Sparse Matrix-Sparse Vector Multiplication for Dynamic GPU Workloads"
 * (arXiv 2608.16308) by section / algorithm / figure.
 *
 * Conventions shared by all entry points
 *   CSR: row_ptr[m+1], col_idx[nnz] (int32, columns sorted and unique per row)
 *   value kinds: 0 = float32, 1 = bf16 (uint16 bit pattern), 2 = pattern (no values)
 *   sparse x: x_idx[nnz_x] (listed positions are the active set J; indices
 *             outside [0, n) contribute nothing), x_val[nnz_x] of a value kind.
 *   y[i] of the PLUS_TIMES semiring is returned in double together with
 *   s[i] = sum |a_ij * x_j| over the same terms (the scale of the error bound).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_PATTERN = 2 };
enum { ORC_COO = 0, ORC_DENSE = 1, ORC_FORCE_CSR = 2, ORC_FORCE_CSC = 3, ORC_CSR = 4 };

#define ORC_TILE 16 /* section 3.2.1: uniform 16x16 blocks */

static double orc_load(const void *v, int kind, int64_t k) {
  if (kind == ORC_F32) return (double)((const float *)v)[k];
  if (kind == ORC_BF16) {
    uint32_t b = (uint32_t)((const uint16_t *)v)[k] << 16; /* exact widening */
    float f;
    memcpy(&f, &b, sizeof f);
    return (double)f;
  }
  return 1.0;
}

static size_t orc_vsize(int kind) { return kind == ORC_F32 ? 4 : kind == ORC_BF16 ? 2 : 0; }

/* Dense view of the active set J and of x over J (section 2.1: only part of x is active). */
static int orc_scatter_x(int32_t n, int32_t nnz_x, const int32_t *x_idx, const void *x_val,
                         int xkind, unsigned char **act, double **xv) {
  *act = (unsigned char *)calloc((size_t)n + 1, 1);
  *xv = (double *)calloc((size_t)n + 1, sizeof(double));
  if (!*act || !*xv) return -1;
  for (int64_t i = 0; i < nnz_x; ++i) {
    int32_t j = x_idx[i];
    if (j < 0 || j >= n) continue; /* invalid index: contributes nothing */
    (*act)[j] = 1;
    (*xv)[j] = x_val ? orc_load(x_val, xkind, i) : 1.0;
  }
  return 0;
}

/* Plain transpose CSR -> CSC by counting; rows stay ascending within a column. */
int orc_csr_to_csc(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                   const void *val, int vkind, int32_t *col_ptr, int32_t *row_idx, void *csc_val) {
  int64_t nnz = row_ptr[m];
  int64_t *cnt = (int64_t *)calloc((size_t)n + 1, sizeof(int64_t));
  if (!cnt) return -1;
  for (int64_t k = 0; k < nnz; ++k) cnt[col_idx[k] + 1]++;
  for (int32_t j = 0; j < n; ++j) cnt[j + 1] += cnt[j];
  for (int32_t j = 0; j <= n; ++j) col_ptr[j] = (int32_t)cnt[j];
  size_t vs = orc_vsize(vkind);
  for (int32_t i = 0; i < m; ++i) {
    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
      int64_t p = cnt[col_idx[k]]++;
      row_idx[p] = i;
      if (vs && val && csc_val) memcpy((char *)csc_val + p * vs, (const char *)val + k * vs, vs);
    }
  }
  free(cnt);
  return 0;
}

/*
 * Pull SpMSpV over CSR (Algorithm 1, bottom half; section 2.1):
 *   y_i = sum over k in row i with col_k in J of val_k * x_{col_k}.
 */
int orc_spmspv_pull(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                    const void *val, int vkind, int32_t nnz_x, const int32_t *x_idx,
                    const void *x_val, int xkind, double *y, double *s) {
  unsigned char *act;
  double *xv;
  if (orc_scatter_x(n, nnz_x, x_idx, x_val, xkind, &act, &xv)) return -1;
  for (int32_t i = 0; i < m; ++i) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
      int32_t j = col_idx[k];
      if (!act[j]) continue;
      double t = orc_load(val, vkind, k) * xv[j];
      acc += t;
      mag += fabs(t);
    }
    y[i] = acc;
    if (s) s[i] = mag;
  }
  free(act);
  free(xv);
  return 0;
}

/*
 * Push SpMSpV over CSC (Algorithm 1, top half; section 2.1): for each listed
 * active entry j, walk column j and add val * x_j into y[row].
 */
int orc_spmspv_push(int32_t m, int32_t n, const int32_t *col_ptr, const int32_t *row_idx,
                    const void *csc_val, int vkind, int32_t nnz_x, const int32_t *x_idx,
                    const void *x_val, int xkind, double *y, double *s) {
  for (int32_t i = 0; i < m; ++i) {
    y[i] = 0.0;
    if (s) s[i] = 0.0;
  }
  for (int64_t q = 0; q < nnz_x; ++q) {
    int32_t j = x_idx[q];
    if (j < 0 || j >= n) continue;
    double xj = x_val ? orc_load(x_val, xkind, q) : 1.0;
    for (int64_t k = col_ptr[j]; k < col_ptr[j + 1]; ++k) {
      double t = orc_load(csc_val, vkind, k) * xj;
      y[row_idx[k]] += t;
      if (s) s[row_idx[k]] += fabs(t);
    }
  }
  return 0;
}

/* Boolean (OR-AND) pull: y_i = 1 iff some stored entry of row i lies in an active column. */
int orc_or_and_pull(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                    int32_t nnz_x, const int32_t *x_idx, uint8_t *y) {
  unsigned char *act;
  double *xv;
  if (orc_scatter_x(n, nnz_x, x_idx, NULL, ORC_PATTERN, &act, &xv)) return -1;
  for (int32_t i = 0; i < m; ++i) {
    uint8_t f = 0;
    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1] && !f; ++k) f = act[col_idx[k]];
    y[i] = f;
  }
  free(act);
  free(xv);
  return 0;
}

/* Boolean (OR-AND) push over CSC: every row stored in an active column becomes 1. */
int orc_or_and_push(int32_t m, int32_t n, const int32_t *col_ptr, const int32_t *row_idx,
                    int32_t nnz_x, const int32_t *x_idx, uint8_t *y) {
  memset(y, 0, (size_t)m);
  for (int64_t q = 0; q < nnz_x; ++q) {
    int32_t j = x_idx[q];
    if (j < 0 || j >= n) continue;
    for (int64_t k = col_ptr[j]; k < col_ptr[j + 1]; ++k) y[row_idx[k]] = 1;
  }
  return 0;
}

/*
 * Masked Boolean step used by BFS (section 4.2; Algorithm 5 drops visited rows
 * from the found set): y_i = (not visited_i) and OR_{j in F} A_ij.
 */
int orc_masked_or_and(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                      int32_t nnz_x, const int32_t *x_idx, const uint8_t *visited, uint8_t *y) {
  if (orc_or_and_pull(m, n, row_ptr, col_idx, nnz_x, x_idx, y)) return -1;
  for (int32_t i = 0; i < m; ++i)
    if (visited[i]) y[i] = 0;
  return 0;
}

/*
 * Textbook FIFO-queue BFS.  The frontier is the sparse vector x and the next
 * frontier is A x (section 4.2), so the neighbours of j are the rows i with a
 * stored A_ij, i.e. column j of A: pass the CSC arrays.  levels[src] = 0, hop
 * distance elsewhere, -1 if unreachable.  Returns the number of levels.
 */
int orc_bfs(int32_t n, const int32_t *col_ptr, const int32_t *row_idx, int32_t src,
            int32_t *levels) {
  if (src < 0 || src >= n) return -1;
  int32_t *queue = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  if (!queue) return -1;
  for (int32_t i = 0; i < n; ++i) levels[i] = -1;
  int64_t head = 0, tail = 0;
  levels[src] = 0;
  queue[tail++] = src;
  int32_t depth = 0;
  while (head < tail) {
    int32_t j = queue[head++];
    if (levels[j] > depth) depth = levels[j];
    for (int64_t k = col_ptr[j]; k < col_ptr[j + 1]; ++k) {
      int32_t i = row_idx[k];
      if (levels[i] < 0) {
        levels[i] = levels[j] + 1;
        queue[tail++] = i;
      }
    }
  }
  free(queue);
  return depth + 1;
}

/* Dense-activation SpMSpV (section 4.3): x_j is active iff x_j != 0 (+0 and -0 inactive). */
int orc_spmspv_dense_x(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                       const void *val, int vkind, const void *x, int xkind, double *y, double *s) {
  for (int32_t i = 0; i < m; ++i) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
      double xj = orc_load(x, xkind, col_idx[k]);
      if (xj == 0.0) continue;
      double t = orc_load(val, vkind, k) * xj;
      acc += t;
      mag += fabs(t);
    }
    y[i] = acc;
    if (s) s[i] = mag;
  }
  (void)n;
  return 0;
}

/*
 * Activation sparsification by magnitude thresholding (the decoding
 * evaluation of section 5.4: activation sparsity from magnitude-based
 * thresholding, after the training-free activation-sparsity reference):
 * x'_j = x_j when |x_j| > t, else +0.  The comparison is exact (|x_j| and t
 * are both exactly representable in double); a NaN entry compares false and
 * becomes 0.  x and out are of the same value kind (float32 or bf16 bits).
 */
int orc_threshold_activation(int32_t n, const void *x, int xkind, float t, void *out) {
  if (xkind != ORC_F32 && xkind != ORC_BF16) return 1;
  for (int32_t j = 0; j < n; ++j) {
    const double a = fabs(orc_load(x, xkind, j));
    const int keep = a > (double)t;
    if (xkind == ORC_F32) ((float *)out)[j] = keep ? ((const float *)x)[j] : 0.0f;
    else ((uint16_t *)out)[j] = keep ? ((const uint16_t *)x)[j] : (uint16_t)0;
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Vector-block metadata (section 3.2.2, section 4.1): blk_x_mask[b] has bit k
 * set iff element 16b+k is active; N_nzblk counts the blocks with a nonzero
 * mask.  Bit k stands for local position k, least significant bit first (the
 * Figure 5 caption: a row mask of 10 = 0b1010 marks columns 1 and 3).
 * ------------------------------------------------------------------------ */
int orc_xmeta(int32_t n, int32_t nnz_x, const int32_t *x_idx, uint16_t *masks, int32_t *n_nzblk) {
  int32_t nb = (n + ORC_TILE - 1) / ORC_TILE;
  memset(masks, 0, sizeof(uint16_t) * (size_t)nb);
  for (int64_t q = 0; q < nnz_x; ++q) {
    int32_t j = x_idx[q];
    if (j < 0 || j >= n) continue;
    masks[j / ORC_TILE] |= (uint16_t)(1u << (j % ORC_TILE));
  }
  int32_t c = 0;
  for (int32_t b = 0; b < nb; ++b) c += masks[b] != 0;
  *n_nzblk = c;
  return 0;
}

int orc_xmeta_dense(int32_t n, const void *x, int xkind, uint16_t *masks, int32_t *n_nzblk) {
  int32_t nb = (n + ORC_TILE - 1) / ORC_TILE;
  memset(masks, 0, sizeof(uint16_t) * (size_t)nb);
  for (int32_t j = 0; j < n; ++j)
    if (orc_load(x, xkind, j) != 0.0) masks[j / ORC_TILE] |= (uint16_t)(1u << (j % ORC_TILE));
  int32_t c = 0;
  for (int32_t b = 0; b < nb; ++b) c += masks[b] != 0;
  *n_nzblk = c;
  return 0;
}

/*
 * High-level selector (section 3.3.1): xb_sparsity = N_nzblk / N_blk; push
 * when it is below th3, pull otherwise.  Returns 1 for push.
 */
int orc_select_push(int32_t n_nzblk, int32_t n_blk, double th3) {
  double xb = (double)n_nzblk / (double)n_blk;
  return xb < th3 ? 1 : 0;
}

/*
 * Low-level block format choice (section 3.2.1; the decision flow of Figure 6):
 *   nnz < th0 -> COO; nnz > th1 -> Dense; otherwise, with the axis skew
 *   skew_a = max_l n_l^(a) / (nnz / B_a + eps), B_r = B_c = 16:
 *   skew_r / skew_c > th2 -> ForceCSC; skew_c / skew_r > th2 -> ForceCSR;
 *   else patched CSR.
 */
int orc_classify(int32_t nnz, int32_t max_row, int32_t max_col, int32_t th0, int32_t th1,
                 double th2) {
  const double eps = 1e-6;
  if (nnz < th0) return ORC_COO;
  if (nnz > th1) return ORC_DENSE;
  double skew_r = (double)max_row / ((double)nnz / ORC_TILE + eps);
  double skew_c = (double)max_col / ((double)nnz / ORC_TILE + eps);
  if (skew_r / skew_c > th2) return ORC_FORCE_CSC;
  if (skew_c / skew_r > th2) return ORC_FORCE_CSR;
  return ORC_CSR;
}

/* qsort key: (column block, local row, local column) */
static int orc_cmp_i64(const void *a, const void *b) {
  int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
  return (x > y) - (x < y);
}

/*
 * Block-level views of the 16x16 tiling (section 3.2.1, Figure 5(b)).
 * Tiles are numbered in the primary block-CSR order (row block major, column
 * block ascending).  Outputs (any may be NULL; call once with all NULL to get T):
 *   rb_ptr[mb+1]                global_block_csr_row_ptr
 *   t_cb[T], t_rb[T]            column / row block of each tile
 *   t_nnz, t_maxrow, t_maxcol   nonzeros, largest row count, largest column count
 *   t_type[T]                   format code from orc_classify
 *   t_rowmask[T*16]             per local row, 16-bit mask of its local columns
 *   t_colmask[T*16]             per local column, 16-bit mask of its local rows
 *   cb_ptr[nb+1], csc_rb[T]     global_block_csc_col_ptr / _row_idx
 *   csc2csr[T]                  primary tile id of each CSC position
 * Returns T, or -1 on allocation failure.
 */
int64_t orc_tile_view(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                      int32_t th0, int32_t th1, double th2, int32_t *rb_ptr, int32_t *t_cb,
                      int32_t *t_rb, int32_t *t_nnz, int32_t *t_maxrow, int32_t *t_maxcol,
                      int32_t *t_type, uint16_t *t_rowmask, uint16_t *t_colmask, int32_t *cb_ptr,
                      int32_t *csc_rb, int32_t *csc2csr) {
  int32_t mb = (m + ORC_TILE - 1) / ORC_TILE;
  int32_t nb = (n + ORC_TILE - 1) / ORC_TILE;
  int64_t T = 0;
  int64_t cap = 0;
  int64_t *keys = NULL;
  if (rb_ptr) rb_ptr[0] = 0;
  for (int32_t rb = 0; rb < mb; ++rb) {
    int32_t r0 = rb * ORC_TILE;
    int32_t r1 = r0 + ORC_TILE < m ? r0 + ORC_TILE : m;
    int64_t cnt = (int64_t)row_ptr[r1] - row_ptr[r0];
    if (cnt > cap) {
      free(keys);
      cap = cnt;
      keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
      if (!keys) return -1;
    }
    int64_t q = 0;
    for (int32_t r = r0; r < r1; ++r)
      for (int64_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
        int64_t c = col_idx[k];
        keys[q++] = ((c / ORC_TILE) << 8) | ((int64_t)(r - r0) << 4) | (c % ORC_TILE);
      }
    qsort(keys, (size_t)cnt, sizeof(int64_t), orc_cmp_i64);
    for (int64_t a = 0; a < cnt;) {
      int64_t cb = keys[a] >> 8, e = a;
      int32_t rows[ORC_TILE] = {0}, cols[ORC_TILE] = {0};
      uint16_t rmask[ORC_TILE] = {0}, cmask[ORC_TILE] = {0};
      while (e < cnt && (keys[e] >> 8) == cb) {
        int lr = (int)((keys[e] >> 4) & 15), lc = (int)(keys[e] & 15);
        rows[lr]++;
        cols[lc]++;
        rmask[lr] |= (uint16_t)(1u << lc);
        cmask[lc] |= (uint16_t)(1u << lr);
        ++e;
      }
      int32_t nz = (int32_t)(e - a), mr = 0, mc = 0;
      for (int l = 0; l < ORC_TILE; ++l) {
        if (rows[l] > mr) mr = rows[l];
        if (cols[l] > mc) mc = cols[l];
      }
      if (t_cb) t_cb[T] = (int32_t)cb;
      if (t_rb) t_rb[T] = rb;
      if (t_nnz) t_nnz[T] = nz;
      if (t_maxrow) t_maxrow[T] = mr;
      if (t_maxcol) t_maxcol[T] = mc;
      if (t_type) t_type[T] = orc_classify(nz, mr, mc, th0, th1, th2);
      if (t_rowmask) memcpy(t_rowmask + T * ORC_TILE, rmask, sizeof rmask);
      if (t_colmask) memcpy(t_colmask + T * ORC_TILE, cmask, sizeof cmask);
      ++T;
      a = e;
    }
    if (rb_ptr) rb_ptr[rb + 1] = (int32_t)T;
  }
  free(keys);
  if (cb_ptr && t_cb) {
    /* block-level CSC: counting sort of the tiles by column block, taking tiles
       in primary order so that row blocks ascend within each column block */
    int64_t *cur = (int64_t *)calloc((size_t)nb + 1, sizeof(int64_t));
    if (!cur) return -1;
    for (int64_t t = 0; t < T; ++t) cur[t_cb[t] + 1]++;
    for (int32_t b = 0; b < nb; ++b) cur[b + 1] += cur[b];
    for (int32_t b = 0; b <= nb; ++b) cb_ptr[b] = (int32_t)cur[b];
    for (int64_t t = 0; t < T; ++t) {
      int64_t p = cur[t_cb[t]]++;
      if (csc2csr) csc2csr[p] = (int32_t)t;
      if (csc_rb) {
        /* row block of tile t: position of t inside rb_ptr */
        int32_t lo = 0, hi = mb;
        while (hi - lo > 1) {
          int32_t mid = (lo + hi) / 2;
          if (rb_ptr[mid] <= t) lo = mid; else hi = mid;
        }
        csc_rb[p] = lo;
      }
    }
    free(cur);
  }
  return T;
}

/*
 * Pull load balance (section 3.3.2): walk the tiles of each row block in
 * primary order, adding the format weight (Dense w_dense; ForceCSR, ForceCSC
 * and CSR w_csr; COO w_coo); the tile that brings the running weight to at
 * least `cap` closes the segment.  Segments never cross row blocks; row blocks
 * without tiles get no segment.  Outputs (may be NULL to count): seg_rb, seg_t0,
 * seg_t1 (tile range [t0, t1)).  Returns the segment count.
 */
int64_t orc_segments(int32_t mb, const int32_t *rb_ptr, const int32_t *t_type, int32_t w_dense,
                     int32_t w_csr, int32_t w_coo, int32_t cap, int32_t *seg_rb, int32_t *seg_t0,
                     int32_t *seg_t1) {
  int64_t ns = 0;
  for (int32_t rb = 0; rb < mb; ++rb) {
    int32_t start = rb_ptr[rb], acc = 0;
    for (int32_t t = rb_ptr[rb]; t < rb_ptr[rb + 1]; ++t) {
      int ty = t_type[t];
      acc += ty == ORC_DENSE ? w_dense : ty == ORC_COO ? w_coo : w_csr;
      if (acc >= cap) {
        if (seg_rb) { seg_rb[ns] = rb; seg_t0[ns] = start; seg_t1[ns] = t + 1; }
        ++ns;
        start = t + 1;
        acc = 0;
      }
    }
    if (start < rb_ptr[rb + 1]) {
      if (seg_rb) { seg_rb[ns] = rb; seg_t0[ns] = start; seg_t1[ns] = rb_ptr[rb + 1]; }
      ++ns;
    }
  }
  return ns;
}
