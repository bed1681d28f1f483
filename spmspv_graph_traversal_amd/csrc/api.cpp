// C-ABI entry points of the library (declared in include/dbs.h): argument
// validation, handle lifetime, options, statistics and array export.  All
// compute is in the HIP kernels of build.hip, spmspv.hip and bfs.hip.
#include <float.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "common.h"
#include "meta.h"

hipError_t dbs_note(hipError_t e, const char *file, int line) {
  static const int verbose = getenv("DBS_VERBOSE") != nullptr;
  if (e != hipSuccess && verbose) fprintf(stderr, "[dbs] %s:%d: %s\n", file, line, hipGetErrorString(e));
  return e;
}

hipError_t dbs_dev_alloc(dbs_matrix *A, void **p, size_t bytes) {
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();  // clear the sticky error of a failed allocation
    return e;
  }
  A->mem_now += (int64_t)bytes;
  if (A->mem_now > A->mem_peak) A->mem_peak = A->mem_now;
  return hipSuccess;
}

void dbs_dev_free(dbs_matrix *A, void *p, size_t bytes) {
  if (!p) return;
  (void)hipFree(p);
  A->mem_now -= (int64_t)bytes;
}

namespace {

// fold the timing slot `i` into the sums (waits for its last event)
hipError_t fold_slot(dbs_matrix *A, int i) {
  float a = 0.0f, b = 0.0f;
  hipError_t e = hipEventSynchronize(A->tev[i][3]);
  if (e == hipSuccess) e = hipEventElapsedTime(&a, A->tev[i][0], A->tev[i][1]);
  if (e == hipSuccess) e = hipEventElapsedTime(&b, A->tev[i][2], A->tev[i][3]);
  if (e != hipSuccess) return e;
  A->st.timed_calls += 1;
  A->st.sum_meta_ms += a;
  A->st.sum_compute_ms += b;
  A->st.last_meta_ms = a;
  A->st.last_compute_ms = b;
  return hipSuccess;
}

// fold every recorded slot, oldest first
hipError_t fold_all(dbs_matrix *A) {
  const int R = dbs_matrix::kTimingRing;
  while (A->tev_used > 0) {
    const int i = (A->tev_head - A->tev_used + R) % R;
    hipError_t e = fold_slot(A, i);
    if (e != hipSuccess) return e;
    A->tev_used -= 1;
  }
  return hipSuccess;
}

void free_all(dbs_matrix *A) {
  void *bufs[] = {A->rb_ptr, A->t_cb,     A->t_meta,   A->cb_ptr,     A->csc_rb,  A->csc2csr, A->csc_cm,
                  A->payload, A->segs,    A->psegs,    A->t_cbx,   A->m2seg,   A->wown,
                  A->meta2 != A->t_meta ? A->meta2 : nullptr,    A->rows_nz,  A->xmask,    A->xbits,      A->xd,
                  A->act_list, A->chunks,
                  A->ctr,    A->bfs_bm,   A->bfs_vis,  A->bfs_fbits, A->bfs_list,   A->bfs_chunks, A->bfs_ctr,
                  A->fin,    A->partial};
  for (void *b : bufs)
    if (b) (void)hipFree(b);
  if (A->bfs_host) (void)hipHostFree(A->bfs_host);
  for (hipEvent_t e : A->ev)
    if (e) (void)hipEventDestroy(e);
  if (A->tev_ready)
    for (int i = 0; i < dbs_matrix::kTimingRing; ++i)
      for (int j = 0; j < 4; ++j) (void)hipEventDestroy(A->tev[i][j]);
}

dbs_status map_err(hipError_t e) {
  if (e == hipSuccess) return DBS_OK;
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return DBS_ERR_OUT_OF_MEMORY;
  return DBS_ERR_DEVICE;
}

#define API_TRY(expr)                       \
  do {                                      \
    dbs_status st_ = map_err(DBS_NOTE(expr));         \
    if (st_ != DBS_OK) return st_;          \
  } while (0)

bool valid_options(const dbs_build_options &o) {
  if (o.th0 < 0 || o.th1 < 0 || o.th2_num <= 0 || o.th2_den <= 0) return false;
  if (o.force_format < -1 || o.force_format > DBS_TILE_CSR) return false;
  if (o.seg_w_dense < 1 || o.seg_w_csr < 1 || o.seg_w_coo < 1 || o.seg_cap < 0) return false;
  return true;
}

dbs_status alloc_call_scratch(dbs_matrix *A) {
  const int vs = A->vk == VK_F32 ? 4 : 2;  // a dense f32 x on a pattern matrix needs no staging
  API_TRY(dbs_dev_alloc(A, (void **)&A->xmask, (size_t)A->nb * 4));
  API_TRY(hipMemset(A->xmask, 0, (size_t)A->nb * 4));
  A->nbw = (A->nb + 31) / 32;
  if (A->vk == VK_PAT) {
    API_TRY(dbs_dev_alloc(A, (void **)&A->xbits, (size_t)A->nbw * 8 + 4));
    API_TRY(hipMemset(A->xbits, 0, (size_t)A->nbw * 8 + 4));
  }
  API_TRY(dbs_dev_alloc(A, &A->xd, (size_t)A->nb * 16 * vs));
  API_TRY(dbs_dev_alloc(A, (void **)&A->act_list, (size_t)A->nb * 4));
  A->max_chunks = A->T / 64 + A->nb + 1;
  API_TRY(dbs_dev_alloc(A, (void **)&A->chunks, (size_t)A->max_chunks * 8));
  API_TRY(dbs_dev_alloc(A, (void **)&A->ctr, 16 * 4));
  API_TRY(hipMemset(A->ctr, 0, 16 * 4));
  return DBS_OK;
}

}  // namespace

hipEvent_t *dbs_timing_slot(dbs_matrix *A) {
  const int R = dbs_matrix::kTimingRing;
  if (!A->tev_ready) {
    for (int i = 0; i < R; ++i)
      for (int j = 0; j < 4; ++j)
        if (DBS_NOTE(hipEventCreate(&A->tev[i][j])) != hipSuccess) return nullptr;
    A->tev_ready = 1;
  }
  if (A->tev_used == R) {  // ring full: fold the oldest (long finished) call
    const int i = (A->tev_head - A->tev_used + R) % R;
    if (DBS_NOTE(fold_slot(A, i)) != hipSuccess) return nullptr;
    A->tev_used -= 1;
  }
  hipEvent_t *slot = A->tev[A->tev_head];
  A->tev_head = (A->tev_head + 1) % R;
  A->tev_used += 1;
  return slot;
}

extern "C" {

dbs_status dbs_build_options_default(dbs_build_options *o) {
  if (!o) return DBS_ERR_INVALID_ARG;
  o->th0 = 32;
  o->th1 = 128;
  o->th2_num = 2;
  o->th2_den = 1;
  o->force_format = -1;
  o->seg_w_dense = 4;
  o->seg_w_csr = 2;
  o->seg_w_coo = 1;
  o->seg_cap = 0;  // by value type
  return DBS_OK;
}

dbs_status dbs_build(int32_t m, int32_t n, int64_t nnz, const int32_t *row_ptr, const int32_t *col_idx,
                     const void *val, dbs_dtype dtype, const dbs_build_options *opt, void *stream,
                     dbs_handle *out) {
  if (!out || !row_ptr || m < 1 || n < 1 || nnz < 0 || nnz >= (int64_t)1 << 31) return DBS_ERR_INVALID_ARG;
  if (dtype != DBS_F32 && dtype != DBS_BF16 && dtype != DBS_PATTERN) return DBS_ERR_INVALID_ARG;
  if (nnz > 0 && !col_idx) return DBS_ERR_INVALID_ARG;
  if (dtype != DBS_PATTERN && nnz > 0 && !val) return DBS_ERR_INVALID_ARG;
  dbs_build_options o;
  if (opt) o = *opt;
  else dbs_build_options_default(&o);
  if (!valid_options(o)) return DBS_ERR_INVALID_ARG;
  // a pull segment holds at most one tile per lane for value matrices and
  // PAT_SEG_CAP tiles (four per lane) for pattern matrices
  const int cap_max = dtype == DBS_PATTERN ? DBS_PAT_SEG_CAP : DBS_WAVE;
  if (o.seg_cap == 0) o.seg_cap = cap_max;
  if (o.seg_cap > cap_max) return DBS_ERR_INVALID_ARG;

  dbs_matrix *A = new (std::nothrow) dbs_matrix;
  if (!A) return DBS_ERR_OUT_OF_MEMORY;
  memset((void *)A, 0, sizeof(*A));
  hipStream_t s = (hipStream_t)stream;
  if (DBS_NOTE(hipGetDevice(&A->device)) != hipSuccess) {
    delete A;
    return DBS_ERR_DEVICE;
  }
  A->m = m;
  A->n = n;
  A->mb = (m + 15) / 16;
  A->nb = (n + 15) / 16;
  A->nnz = nnz;
  A->dtype = dtype;
  A->vk = dtype == DBS_F32 ? VK_F32 : dtype == DBS_BF16 ? VK_BF16 : VK_PAT;
  A->bopt = o;
  A->opt[DBS_OPT_PATH] = 0;
  A->opt[DBS_OPT_TH3_NUM] = 1;
  A->opt[DBS_OPT_TH3_DEN] = 100;
  A->opt[DBS_OPT_LOCAL_PUSH_CUTOFF] = 0;
  A->opt[DBS_OPT_TIMING] = 0;
  A->opt[DBS_OPT_CHECK] = 0;
  A->opt[DBS_OPT_PULL_WIDTH] = 0;
  A->opt[DBS_OPT_PULL_SHARE] = 0;
  A->st.last_path = -1;
  A->st.last_meta_ms = -1.0f;
  A->st.last_compute_ms = -1.0f;
  A->st.bfs_ms = -1.0f;
  A->st.bfs_kernel_ms = -1.0f;
  A->last_stream = s;

  dbs_status st = dbs_build_impl(A, row_ptr, col_idx, val, s);
  if (st != DBS_OK && getenv("DBS_VERBOSE")) fprintf(stderr, "[dbs] build stage failed: %d\n", (int)st);
  if (st == DBS_OK) {
    A->st.build_peak_bytes = A->mem_peak;
    st = alloc_call_scratch(A);
  }
  for (hipEvent_t &e : A->ev)
    if (st == DBS_OK) st = map_err(DBS_NOTE(hipEventCreate(&e)));
  if (st == DBS_OK) st = map_err(DBS_NOTE(hipStreamSynchronize(s)));
  if (st != DBS_OK) {
    (void)hipStreamSynchronize(s);
    free_all(A);
    delete A;
    return st;
  }
  A->st.m = m;
  A->st.n = n;
  A->st.mb = A->mb;
  A->st.nb = A->nb;
  A->st.nnz = nnz;
  A->st.tiles = A->T;
  A->st.segments = A->nseg;
  A->st.payload_bytes = A->payload_bytes;
  // views: block-CSR (rb_ptr, column blocks, metadata), block-CSC (cb_ptr,
  // row blocks, primary ids, column sets)
  A->st.index_bytes = (int64_t)(A->mb + 1) * 4 + A->T * (4 + 8 + 4 + 4 + 2) + (int64_t)(A->nb + 1) * 4;
  // pattern matrices: the Boolean pull's segments, column-block words,
  // metadata of the tiles not marked single, per-segment entries and word owners
  int64_t pull_bytes = 0;
  if (A->vk == VK_PAT)
    pull_bytes = A->npseg * (16 + 8) + A->T * 4 + (A->meta2 != A->t_meta ? A->nmeta2 * 8 : 0) +
                 (A->payload_bytes + DBS_PAYLOAD_SLACK) / 4;
  A->st.format_bytes = A->st.payload_bytes + A->st.index_bytes + A->nseg * 16 + pull_bytes;
  *out = A;
  return DBS_OK;
}

static dbs_status check_semiring(const dbs_matrix *A, dbs_semiring sr) {
  if (sr != DBS_PLUS_TIMES && sr != DBS_OR_AND) return DBS_ERR_INVALID_ARG;
  if (sr == DBS_PLUS_TIMES && A->dtype == DBS_PATTERN) return DBS_ERR_INVALID_ARG;
  // PLUS_TIMES stages x block-padded and reads it with 32-bit byte offsets
  if (sr == DBS_PLUS_TIMES && !dbs_x_fits_offsets((uint64_t)A->nb, A->vk == VK_F32 ? 4u : 2u))
    return DBS_ERR_UNSUPPORTED;
  return DBS_OK;
}

dbs_status dbs_spmspv(dbs_handle A, int32_t nnz_x, const int32_t *x_idx, const void *x_val, dbs_semiring sr,
                      void *y, void *stream) {
  if (!A || !y || nnz_x < 0 || nnz_x > A->n) return DBS_ERR_INVALID_ARG;
  if (nnz_x > 0 && !x_idx) return DBS_ERR_INVALID_ARG;
  dbs_status st = check_semiring(A, sr);
  if (st != DBS_OK) return st;
  if (sr == DBS_PLUS_TIMES && nnz_x > 0 && !x_val) return DBS_ERR_INVALID_ARG;
  return dbs_spmspv_impl(A, nnz_x, x_idx, x_val, nullptr, sr, y, (hipStream_t)stream);
}

dbs_status dbs_spmspv_dense(dbs_handle A, const void *x, dbs_semiring sr, void *y, void *stream) {
  if (!A || !x || !y) return DBS_ERR_INVALID_ARG;
  dbs_status st = check_semiring(A, sr);
  if (st != DBS_OK) return st;
  return dbs_spmspv_impl(A, 0, nullptr, nullptr, x, sr, y, (hipStream_t)stream);
}

dbs_status dbs_spmspv_dense_threshold(dbs_handle A, const void *x, float threshold, dbs_semiring sr, void *y,
                                      void *stream) {
  if (!A || !x || !y) return DBS_ERR_INVALID_ARG;
  if (!(threshold >= 0.0f) || threshold > FLT_MAX) return DBS_ERR_INVALID_ARG;  // NaN, negative, inf
  dbs_status st = check_semiring(A, sr);
  if (st != DBS_OK) return st;
  return dbs_spmspv_impl(A, 0, nullptr, nullptr, x, sr, y, (hipStream_t)stream, threshold);
}

dbs_status dbs_bfs(dbs_handle A, int32_t src, int32_t *levels, void *stream) {
  if (!A || !levels || A->m != A->n || src < 0 || src >= A->m) return DBS_ERR_INVALID_ARG;
  return dbs_bfs_impl(A, src, levels, (hipStream_t)stream);
}

dbs_status dbs_bfs_noalloc(dbs_handle A, int32_t src, int32_t *levels, void *stream) {
  if (!A || !levels || A->m != A->n || src < 0 || src >= A->m) return DBS_ERR_INVALID_ARG;
  return dbs_bfs_noalloc_impl(A, src, levels, (hipStream_t)stream);
}

dbs_status dbs_set_option(dbs_handle A, int32_t option, int64_t value) {
  if (!A) return DBS_ERR_INVALID_ARG;
  switch (option) {
    case DBS_OPT_PATH:
      if (value < 0 || value > 2) return DBS_ERR_INVALID_ARG;
      break;
    case DBS_OPT_TH3_NUM:
      if (value < 0 || value > ((int64_t)1 << 31)) return DBS_ERR_INVALID_ARG;
      break;
    case DBS_OPT_TH3_DEN:
      if (value < 1 || value > ((int64_t)1 << 31)) return DBS_ERR_INVALID_ARG;
      break;
    case DBS_OPT_LOCAL_PUSH_CUTOFF:
      if (value < 0 || value > 17) return DBS_ERR_INVALID_ARG;
      break;
    case DBS_OPT_TIMING:
      if (value != 0 && value != 1) return DBS_ERR_INVALID_ARG;
      API_TRY(fold_all(A));
      A->st.timed_calls = 0;
      A->st.sum_meta_ms = 0.0;
      A->st.sum_compute_ms = 0.0;
      break;
    case DBS_OPT_CHECK:
      if (value != 0 && value != 1) return DBS_ERR_INVALID_ARG;
      break;
    case DBS_OPT_PULL_WIDTH:
      if (value != 0 && value != 1 && value != 4) return DBS_ERR_INVALID_ARG;
      break;
    case DBS_OPT_PULL_SHARE:
      if (value != 0 && value != 1 && value != 2 && value != 4) return DBS_ERR_INVALID_ARG;
      break;
    default:
      return DBS_ERR_INVALID_ARG;
  }
  A->opt[option] = value;
  return DBS_OK;
}

dbs_status dbs_get_option(dbs_handle A, int32_t option, int64_t *value) {
  if (!A || !value || option < 0 || option > DBS_OPT_PULL_SHARE) return DBS_ERR_INVALID_ARG;
  *value = A->opt[option];
  return DBS_OK;
}

dbs_status dbs_get_stats(dbs_handle A, dbs_stats *out) {
  if (!A || !out) return DBS_ERR_INVALID_ARG;
  dbs_status ret = DBS_OK;
  if (A->st.last_path == -2) {
    // counters of the last call live in the buffer before the current one
    const uint32_t *c = A->ctr + 8 * (1 - A->cbuf);
    uint32_t h[8];
    API_TRY(hipMemcpyAsync(h, c, sizeof h, hipMemcpyDeviceToHost, A->last_stream));
    API_TRY(hipStreamSynchronize(A->last_stream));
    const uint32_t nz = dbs_meta::nzblk_clamped(h[0], A->nb);
    A->st.last_n_nzblk = (int32_t)nz;
    A->st.last_push_chunks = h[1];
    const bool push = dbs_meta::selector_push(nz, A->nb, (int32_t)A->opt[DBS_OPT_PATH], A->opt[DBS_OPT_TH3_NUM],
                                              A->opt[DBS_OPT_TH3_DEN]);
    A->st.last_path = push ? 0 : 1;
    if (h[2]) ret = DBS_ERR_BAD_VECTOR;
  } else {
    API_TRY(hipStreamSynchronize(A->last_stream));
  }
  API_TRY(fold_all(A));
  const dbs_status sr = dbs_bfs_count_reached(A);
  if (sr != DBS_OK) return sr;
  *out = A->st;
  return ret;
}

dbs_status dbs_copy_array(dbs_handle A, int32_t which, void *dst, int64_t capacity, int64_t *bytes_out) {
  if (!A) return DBS_ERR_INVALID_ARG;
  const void *src = nullptr;
  int64_t bytes = 0;
  switch (which) {
    case DBS_ARR_RB_PTR: src = A->rb_ptr; bytes = (int64_t)(A->mb + 1) * 4; break;
    case DBS_ARR_T_CB: src = A->t_cb; bytes = A->T * 4; break;
    case DBS_ARR_T_META: src = A->t_meta; bytes = A->T * 8; break;
    case DBS_ARR_CB_PTR: src = A->cb_ptr; bytes = (int64_t)(A->nb + 1) * 4; break;
    case DBS_ARR_CSC_RB: src = A->csc_rb; bytes = A->T * 4; break;
    case DBS_ARR_CSC2CSR: src = A->csc2csr; bytes = A->T * 4; break;
    case DBS_ARR_CSC_CM: src = A->csc_cm; bytes = A->T * 2; break;
    case DBS_ARR_PAYLOAD: src = A->payload; bytes = A->payload_bytes; break;
    case DBS_ARR_SEGMENTS: src = A->segs; bytes = A->nseg * 16; break;
    case DBS_ARR_PAT_SEGS: src = A->psegs; bytes = A->psegs ? A->npseg * 16 : 0; break;
    case DBS_ARR_T_CBX: src = A->t_cbx; bytes = A->t_cbx ? A->T * 4 : 0; break;
    case DBS_ARR_META2: src = A->meta2; bytes = A->meta2 ? A->nmeta2 * 8 : 0; break;
    case DBS_ARR_PAT_M2: src = A->m2seg; bytes = A->m2seg ? A->npseg * 8 : 0; break;
    case DBS_ARR_XMASK: src = A->xmask; bytes = (int64_t)A->nb * 2; break;
    case DBS_ARR_ACTIVE: {
      dbs_stats tmp;
      dbs_status s2 = dbs_get_stats(A, &tmp);
      if (s2 != DBS_OK && s2 != DBS_ERR_BAD_VECTOR) return s2;
      src = A->act_list;
      bytes = A->st.last_path >= 0 ? (int64_t)A->st.last_n_nzblk * 4 : 0;
      break;
    }
    default: return DBS_ERR_INVALID_ARG;
  }
  if (bytes_out) *bytes_out = bytes;
  if (!dst) return DBS_OK;
  if (capacity < bytes) return DBS_ERR_INVALID_ARG;
  API_TRY(hipStreamSynchronize(A->last_stream));
  if (which == DBS_ARR_XMASK) {
    // untag: entries of an older epoch are zero masks
    uint32_t *tmp = (uint32_t *)malloc((size_t)A->nb * 4 + 4);
    if (!tmp) return DBS_ERR_OUT_OF_MEMORY;
    hipError_t e = hipMemcpy(tmp, A->xmask, (size_t)A->nb * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      free(tmp);
      return map_err(e);
    }
    uint16_t *d = (uint16_t *)dst;
    for (int32_t b = 0; b < A->nb; ++b) d[b] = (tmp[b] >> 16) == A->epoch ? (uint16_t)(tmp[b] & 0xFFFFu) : 0;
    free(tmp);
    return DBS_OK;
  }
  if (bytes > 0) API_TRY(hipMemcpy(dst, src, (size_t)bytes, hipMemcpyDeviceToHost));
  return DBS_OK;
}

dbs_status dbs_free(dbs_handle A) {
  if (!A) return DBS_OK;
  (void)hipStreamSynchronize(A->last_stream);
  free_all(A);
  delete A;
  return DBS_OK;
}

const char *dbs_status_string(dbs_status s) {
  switch (s) {
    case DBS_OK: return "ok";
    case DBS_ERR_INVALID_ARG: return "invalid argument";
    case DBS_ERR_BAD_CSR: return "invalid CSR input";
    case DBS_ERR_OUT_OF_MEMORY: return "device out of memory";
    case DBS_ERR_DEVICE: return "HIP runtime error";
    case DBS_ERR_UNSUPPORTED: return "unsupported";
    case DBS_ERR_BAD_VECTOR: return "x_idx not strictly increasing";
    case DBS_ERR_TOO_LARGE: return "problem larger than the fixed scratch of an allocation-free call";
  }
  return "unknown status";
}

}  // extern "C"
