/*
 * dbs.h — dual-view blocked sparse matrix x sparse vector multiplication
 * (DB-SpMSpV) with BFS and sparse-decode drivers, for AMD Instinct MI355X
 * (gfx950).
 *
 * The method is the one of "DB-SpMSpV: Dual-View Blocked Sparse Matrix-Sparse
 * Vector Multiplication for Dynamic GPU Workloads" (arXiv 2608.16308):
 *   section 2.1      the product y = A x with push (column-driven) and pull
 *                    (row-driven) formulations, Algorithm 1;
 *   section 3.2      the dual-view blocked format: 16x16 tiles, block-level
 *                    CSR and CSC index views over one shared tile payload,
 *                    five tile formats, 16-element vector blocks with masks;
 *   section 3.3      the two-level adaptive engine: push/pull selection from
 *                    the nonzero-block ratio, per-tile microkernels, load
 *                    balancing and hierarchical writeback;
 *   section 4.1      on-GPU construction of the vector-block metadata;
 *   section 4.2      DB-BFS (frontier = sparse x, visited mask);
 *   section 4.3      DB-Decoding (dense activation -> activation masks).
 *
 * Conventions for every entry point
 *   - Matrix and vector pointers are DEVICE pointers (memory from hipMalloc or
 *     any allocator of the current device), unless stated otherwise.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are stream-ordered and asynchronous unless stated otherwise.
 *   - The caller owns all input and output buffers.  The handle owns the
 *     blocked format and the transient scratch it uses.  Inputs are never
 *     written.  Outputs are overwritten completely on every call.
 *   - Errors are reported by the return code only; nothing is thrown across
 *     the ABI.  On an error return no output has been written, except where
 *     a device-side check is documented.
 *   - A handle may be used by one stream at a time: calls on one handle that
 *     overlap in time race on its scratch.
 */
#ifndef DBS_H
#define DBS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dbs_matrix *dbs_handle; /* opaque */

typedef enum {
  DBS_OK = 0,
  DBS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad enum, dtype/semiring mismatch */
  DBS_ERR_BAD_CSR = 2,       /* row_ptr not monotone / not starting at 0 / not ending at nnz,
                                column out of range, columns not strictly increasing in a row */
  DBS_ERR_OUT_OF_MEMORY = 3, /* a device allocation failed; nothing is leaked */
  DBS_ERR_DEVICE = 4,        /* a HIP runtime call failed */
  DBS_ERR_UNSUPPORTED = 5,   /* valid request this library does not implement */
  DBS_ERR_BAD_VECTOR = 6,    /* check mode found x_idx not strictly increasing */
  DBS_ERR_TOO_LARGE = 7      /* the problem needs more than the fixed scratch of an
                                allocation-free call (DBS_NOALLOC_SCRATCH_BYTES) */
} dbs_status;

/* value type of the matrix (and of x for DBS_PLUS_TIMES) */
typedef enum { DBS_F32 = 0, DBS_BF16 = 1, DBS_PATTERN = 2 } dbs_dtype;

/* PLUS_TIMES: y_i = sum_j a_ij x_j over active j, fp32 output, fp32 accumulation.
 * OR_AND:     y_i = 1 iff row i has a stored entry in an active column (values
 *             ignored, explicitly stored zeros count), uint8 0/1 output. */
typedef enum { DBS_PLUS_TIMES = 0, DBS_OR_AND = 1 } dbs_semiring;

/* Tile formats of section 3.2.1 (Figure 5(b)). */
typedef enum {
  DBS_TILE_COO = 0,       /* nnz < th0: packed (row<<4 | col) bytes + values */
  DBS_TILE_DENSE = 1,     /* nnz > th1: 256 values, row-major */
  DBS_TILE_FORCE_CSR = 2, /* column skew > th2 x row skew: row masks + row pointers */
  DBS_TILE_FORCE_CSC = 3, /* row skew > th2 x column skew: column masks + column pointers */
  DBS_TILE_CSR = 4        /* otherwise: patched CSR (row view + col_ptr + row_idx_csc2csr) */
} dbs_tile_format;

/* ------------------------------------------------------------------------
 * Build-time options (section 3.2.1 thresholds, section 3.3.2 segment weights).
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t th0;            /* COO below this nnz (default 32) */
  int32_t th1;            /* Dense above this nnz (default 128) */
  int32_t th2_num;        /* skew ratio threshold th2 = th2_num / th2_den (default 2/1) */
  int32_t th2_den;
  int32_t force_format;   /* -1 = adaptive (default); a dbs_tile_format value stores every
                             tile in that format (the format ablation of Figure 10) */
  int32_t seg_w_dense;    /* pull segment weights: Dense (default 4) */
  int32_t seg_w_csr;      /*   ForceCSR / ForceCSC / CSR (default 2) */
  int32_t seg_w_coo;      /*   COO (default 1) */
  int32_t seg_cap;        /* a segment closes at the tile bringing its weight to >= cap.
                             0 (default): 64 for value matrices, 256 for pattern matrices
                             (one 64-lane wave works on a segment, one tile per lane for
                             value matrices, four for pattern matrices; the pages'
                             32-lane warps use 16).  Explicit range 1..64 (value) or
                             1..256 (pattern): a segment holds at most seg_cap tiles;
                             other values give DBS_ERR_INVALID_ARG. */
} dbs_build_options;

/* Fills `opt` with the defaults above.  Never fails for a non-NULL pointer. */
dbs_status dbs_build_options_default(dbs_build_options *opt);

/*
 * dbs_build — convert a CSR matrix into the dual-view blocked format
 * (section 3.2.1, Figure 5(b)); the conversion runs on the GPU.
 *
 *   m, n      rows and columns, 1 <= m, n < 2^31
 *   nnz       stored entries, 0 <= nnz < 2^31
 *   row_ptr   device int32[m+1], row_ptr[0] = 0, non-decreasing, row_ptr[m] = nnz
 *   col_idx   device int32[nnz], strictly increasing within each row, in [0, n)
 *   val       device values: float[nnz] (DBS_F32), bf16 bit patterns uint16[nnz]
 *             (DBS_BF16) or NULL (DBS_PATTERN: structure only)
 *   opt       build options, or NULL for the defaults
 *   stream    hipStream_t; the call is SYNCHRONOUS on it (it reads sizes back)
 *   out       receives the new handle; untouched on error
 *
 * The CSR arrays may be freed once the call returns.  Returns DBS_ERR_BAD_CSR
 * for an invalid CSR (checked on the device before any other work), and
 * DBS_ERR_UNSUPPORTED for a format the kernels cannot address with their
 * 32-bit byte offsets: a tile payload of more than 4,294,967,024 bytes (4 GiB -
 * 272), or more than 536,870,910 tiles.
 */
dbs_status dbs_build(int32_t m, int32_t n, int64_t nnz, const int32_t *row_ptr,
                     const int32_t *col_idx, const void *val, dbs_dtype dtype,
                     const dbs_build_options *opt, void *stream, dbs_handle *out);

/*
 * dbs_spmspv — y = A x for a sparse x (sections 3.3, 4.1).
 *
 *   nnz_x     number of listed entries, 0 <= nnz_x <= n
 *   x_idx     device int32[nnz_x], strictly increasing.  Listed positions form
 *             the active set; an index outside [0, n) contributes nothing.
 *   x_val     device values of the matrix dtype (float or bf16 bits), required
 *             for DBS_PLUS_TIMES, ignored (may be NULL) for DBS_OR_AND.
 *   sr        DBS_PLUS_TIMES (not allowed on a DBS_PATTERN matrix) or DBS_OR_AND
 *   y         device float[m] (PLUS_TIMES) or uint8[m] holding 0/1 (OR_AND)
 *
 * One call launches the vector-metadata kernel and the SpMSpV kernel; the
 * push/pull choice (push iff N_nzblk / N_blk < th3) is taken on the device.
 * DBS_PLUS_TIMES on a DBS_F32 matrix of more than 1,073,741,808 columns, or a
 * DBS_BF16 one of more than 2,147,483,632 (x block-padded past 4 GiB - 16
 * bytes), returns DBS_ERR_UNSUPPORTED; so do the dense calls below.
 * In check mode (DBS_OPT_CHECK) a non-increasing x_idx is flagged on the
 * device and reported by the next dbs_get_stats as DBS_ERR_BAD_VECTOR;
 * without check mode such input gives unspecified (but memory-safe) y.
 */
dbs_status dbs_spmspv(dbs_handle A, int32_t nnz_x, const int32_t *x_idx, const void *x_val,
                      dbs_semiring sr, void *y, void *stream);

/*
 * dbs_spmspv_dense — y = A x for a dense x whose zeros are inactive, the
 * single-token decode case (section 4.3).  The activation masks are built on
 * the GPU from x (section 4.1): x_j is active iff x_j != 0 (+0 and -0 are
 * inactive).
 *
 *   x   device float[n] (DBS_F32) or bf16 bits uint16[n] (DBS_BF16); for
 *       DBS_OR_AND on a DBS_PATTERN matrix, float[n]
 *   y   as for dbs_spmspv
 */
dbs_status dbs_spmspv_dense(dbs_handle A, const void *x, dbs_semiring sr, void *y,
                            void *stream);

/*
 * dbs_spmspv_dense_threshold — decode with the activation sparsified in the
 * metadata kernel: y = A x' with x'_j = x_j when |x_j| > threshold, else 0
 * (magnitude thresholding, the activation sparsity of the decoding
 * evaluation, section 5.4).  The masks (section 4.1) come from x' and the
 * multiply reads x' only; x itself is not written.  threshold = 0 gives
 * dbs_spmspv_dense, except that a NaN entry of x is dropped here (every
 * comparison with NaN is false).
 *
 *   x          as for dbs_spmspv_dense
 *   threshold  finite and >= 0, else DBS_ERR_INVALID_ARG
 *   y          as for dbs_spmspv
 */
dbs_status dbs_spmspv_dense_threshold(dbs_handle A, const void *x, float threshold, dbs_semiring sr,
                                      void *y, void *stream);

/*
 * dbs_bfs — single-source BFS levels (section 4.2, Algorithm 5).  Each level
 * is one masked OR_AND SpMSpV y = A f with the frontier f as the sparse
 * vector; push or pull is chosen per level from the frontier's nonzero-block
 * ratio with the same rule as dbs_spmspv.  Vertex i is reached from j when
 * A_ij is stored (for a symmetric A this is the usual undirected BFS).
 *
 *   A        square (m == n) matrix of any dtype (values are ignored)
 *   src      source vertex, 0 <= src < m
 *   levels   device int32[m]: hop distance from src, -1 if unreachable
 *
 * SYNCHRONOUS on `stream`: the levels are launched in batches of eight and
 * the host reads the frontier sizes of a batch once (one stream
 * synchronization per eight levels); the levels of the last batch that come
 * after the first empty frontier return at once.  Uses device scratch that
 * the handle allocates on the first call (bitmaps, block lists, counters).
 */
dbs_status dbs_bfs(dbs_handle A, int32_t src, int32_t *levels, void *stream);

/*
 * dbs_bfs_noalloc — dbs_bfs for callers that cannot allocate memory (code
 * that must not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, same levels, same kernels; the run's device
 * scratch comes from a fixed array of DBS_NOALLOC_SCRATCH_BYTES that each
 * device holds for the life of the process (set up on the first call on a
 * device), and the frontier sizes go to a host buffer on the call's stack.
 * The call makes no allocation of its own (no hipMalloc, hipHostMalloc,
 * hipFree).
 *
 *   Scratch needed: the 256-B-aligned sum of 4 (3 ceil(nb/2) + 1) (frontier
 *   bitmaps), 4 (ceil(nb/2) + 1) (visited), 4 (3 nb + 1) (block lists) and
 *   4 (25 + 8) (counters) bytes, about 20 nb bytes (nb = ceil(n/16)): up to
 *   about 26 million vertices.  When a push level could need chunk lists cut
 *   ahead (a forced push with nb > 6144, or th3 above 6144 / nb), 8 (3
 *   (T/64 + nb + 1) + 1) bytes more.  A larger problem returns
 *   DBS_ERR_TOO_LARGE before any work.
 *
 *   The array is shared by every call on the device and keeps the last
 *   call's contents (each call clears what it needs at its start): calls that
 *   overlap in time on one device race.  The current device must be the
 *   handle's (else DBS_ERR_INVALID_ARG).  dbs_stats.bfs_reached is not
 *   counted for this call (it stays -1): the visited bitmap it would be
 *   counted from lives in the shared array.
 */
#define DBS_NOALLOC_SCRATCH_BYTES (32u << 20)
dbs_status dbs_bfs_noalloc(dbs_handle A, int32_t src, int32_t *levels, void *stream);

/* Per-handle run-time options (dbs_set_option / dbs_get_option). */
enum {
  DBS_OPT_PATH = 0,              /* 0 auto (default), 1 force push, 2 force pull */
  DBS_OPT_TH3_NUM = 1,           /* th3 = num / den (default 1 / 100): push iff */
  DBS_OPT_TH3_DEN = 2,           /*   N_nzblk * den < N_blk * num              */
  DBS_OPT_LOCAL_PUSH_CUTOFF = 3, /* patched-CSR tiles use the column (push) microkernel
                                    when popcount(blk_x_mask) < cutoff (default 0: always
                                    the row microkernel, the faster one on this GPU) */
  DBS_OPT_TIMING = 4,            /* 1: time the kernels of each call with HIP events (setting
                                    it, to 0 or 1, also clears the sums in dbs_stats) */
  DBS_OPT_CHECK = 5,             /* 1: validate x_idx ordering on the device */
  DBS_OPT_PULL_WIDTH = 6,        /* PLUS_TIMES pull of a value matrix, segments per wave
                                    step: 0 auto (default: four when every resident wave
                                    gets several steps, else one), 1 or 4 forced */
  DBS_OPT_PULL_SHARE = 7         /* PLUS_TIMES pull with one segment per step: waves that
                                    share a segment, each taking a range of its tiles:
                                    0 auto (default: enough to give every resident wave
                                    work, at most 4), 1, 2 or 4 forced.  Ignored with four
                                    segments per step.  Both options change only the work
                                    split (and the fp32 summation order), not the result's
                                    bound; they exist to test and measure every variant */
};
dbs_status dbs_set_option(dbs_handle A, int32_t option, int64_t value);
dbs_status dbs_get_option(dbs_handle A, int32_t option, int64_t *value);

typedef struct {
  /* format (fixed at build time) */
  int32_t m, n, mb, nb;            /* rows, columns, row blocks, column blocks */
  int64_t nnz, tiles;
  int64_t tiles_by_format[5];      /* indexed by dbs_tile_format */
  int64_t nnz_by_format[5];
  int64_t segments;                /* pull segments */
  int64_t payload_bytes;           /* tile payload arena */
  int64_t index_bytes;             /* block-CSR + block-CSC views and tile metadata */
  int64_t format_bytes;            /* payload + index + segment descriptors + (pattern
                                      matrices) the Boolean pull's own arrays */
  int64_t build_peak_bytes;        /* peak device memory held during dbs_build */
  /* last dbs_spmspv / dbs_spmspv_dense call (reading them synchronizes its stream) */
  int32_t last_path;               /* 0 push, 1 pull, -1 no call yet */
  int32_t last_n_nzblk;            /* nonzero vector blocks */
  int64_t last_push_chunks;        /* 64-tile work chunks listed ahead for push (0 when the
                                      pushing kernel takes them from the block list itself) */
  float last_meta_ms;              /* metadata kernel time (DBS_OPT_TIMING), else -1 */
  float last_compute_ms;           /* SpMSpV kernel time (DBS_OPT_TIMING), else -1 */
  /* sums over the SpMSpV calls made since DBS_OPT_TIMING was last set to 1 (HIP
     events recorded on each call's stream around each of its two kernels) */
  int64_t timed_calls;
  double sum_meta_ms;
  double sum_compute_ms;
  /* last dbs_bfs call */
  int32_t bfs_levels;              /* levels run (including the empty last one) */
  int32_t bfs_push_levels;         /* of which push */
  int64_t bfs_reached;             /* vertices with a level >= 0 (counted from the handle's
                                      visited bitmap when dbs_get_stats is called) */
  float bfs_ms;                    /* whole BFS (DBS_OPT_TIMING), else -1 */
  float bfs_kernel_ms;             /* sum of the level kernels (DBS_OPT_TIMING), else -1 */
} dbs_stats;

/* Fills `out`; synchronizes the stream of the last call.  Returns
 * DBS_ERR_BAD_VECTOR (and still fills `out`) if check mode flagged the last call. */
dbs_status dbs_get_stats(dbs_handle A, dbs_stats *out);

/* Internal arrays of the format, copied to HOST memory for inspection and
 * tests.  `bytes_out` (may be NULL) receives the array's size; `dst` may be
 * NULL to query the size only; otherwise `capacity` must be at least that
 * size.  Synchronous.  Layouts are described in the library's design notes. */
enum {
  DBS_ARR_RB_PTR = 0,      /* uint32[mb+1]   global_block_csr_row_ptr */
  DBS_ARR_T_CB = 1,        /* uint32[T]      global_block_csr_col_idx */
  DBS_ARR_T_META = 2,      /* uint64[T]      payload offset | (nnz-1)<<40 | format<<48
                                             | inline<<51 | pattern: row block in its
                                             Boolean-pull segment<<52 */
  DBS_ARR_CB_PTR = 3,      /* uint32[nb+1]   global_block_csc_col_ptr */
  DBS_ARR_CSC_RB = 4,      /* uint32[T]      global_block_csc_row_idx */
  DBS_ARR_CSC2CSR = 5,     /* uint32[T]      global_block_csc2csr */
  DBS_ARR_PAYLOAD = 6,     /* uint8[]        tile payload arena */
  DBS_ARR_SEGMENTS = 7,    /* uint32[4*S]    {row block | split<<31 | drain<<30 | slot
                                             class<<28, t0, t1, partial slot + 1 or 0}:
                                             value matrices: the segments of class 3 first, by
                                             first column block, then the others by row block */
  DBS_ARR_XMASK = 8,       /* uint16[nb]     blk_x_mask of the last call */
  DBS_ARR_ACTIVE = 9,      /* uint32[N_nzblk] nonzero vector blocks of the last call (any order) */
  DBS_ARR_CSC_CM = 10,     /* uint16[T]      columns of each tile that hold entries, CSC order */
  DBS_ARR_PAT_SEGS = 11,   /* uint32[4*S']   pattern matrices: Boolean-pull segments {first row
                                             block, t0, t1, row blocks}, in launch order */
  DBS_ARR_T_CBX = 12,      /* uint32[T]      pattern matrices, the Boolean pull's column-block
                                             words: at most 2^19 column blocks: column block |
                                             row block in its Boolean-pull segment<<19 | (one
                                             entry<<23 | that entry's (row<<4 | column)<<24, or
                                             else the tile's index among its segment's tiles of
                                             more than one entry<<24); more: column block | that
                                             row block<<27 */
  DBS_ARR_META2 = 13,      /* uint64[T']     pattern matrices: the T_META words of the tiles
                                             without bit 23 in T_CBX, in tile order */
  DBS_ARR_PAT_M2 = 14      /* uint32[2*S']   per Boolean-pull segment (PAT_SEGS order): its
                                             first entry in META2, and its entries */
};
dbs_status dbs_copy_array(dbs_handle A, int32_t which, void *dst, int64_t capacity,
                          int64_t *bytes_out);

/* Releases the handle and everything it owns (synchronizes its last stream).
 * NULL is accepted. */
dbs_status dbs_free(dbs_handle A);

/* Static description of a status code. */
const char *dbs_status_string(dbs_status s);

/*
 * dbs_probe_read — a measurement helper, not part of the method: reads the
 * `bytes` bytes at device address `buf` once, with 16-byte vector loads from
 * a grid of eight 256-thread workgroups per compute unit, and writes nothing
 * unless the XOR of some thread's words equals `never` (then that value goes
 * to the device word *sink; pick a value the data cannot produce).  Timing it
 * on a stream gives the streaming-read bandwidth of the device, the yardstick
 * beside the published HBM peak for the byte-model roofline of the SpMSpV
 * kernels.  `buf` 16-byte aligned, `bytes` a positive multiple of 16, `sink`
 * a device uint32; else DBS_ERR_INVALID_ARG.  Asynchronous on `stream`.
 */
dbs_status dbs_probe_read(const void *buf, int64_t bytes, uint32_t *sink, uint32_t never, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DBS_H */
