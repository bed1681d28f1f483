// Shared definitions of the HIP library: the handle, the tile-payload layout
// and wave64 helpers.  Citations refer to "DB-SpMSpV: Dual-View Blocked Sparse
// Matrix-Sparse Vector Multiplication for Dynamic GPU Workloads" (arXiv
// 2608.16308) by section / algorithm / figure.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dbs.h"

// ---------------------------------------------------------------------------
// Geometry: 16x16 tiles and 16-element vector blocks (sections 3.2.1, 3.2.2).
// ---------------------------------------------------------------------------
#define DBS_TILE 16
#define DBS_WAVE 64

// value kinds of the payload
enum { VK_F32 = 0, VK_BF16 = 1, VK_PAT = 2 };

__host__ __device__ inline int vk_size(int vk) { return vk == VK_F32 ? 4 : vk == VK_BF16 ? 2 : 0; }
__host__ __device__ inline uint32_t align_up(uint32_t x, uint32_t a) { return (x + a - 1) & ~(a - 1); }

// ---------------------------------------------------------------------------
// Tile payload layout (one arena, three sections: Dense | mask-based | COO).
// Offsets are bytes from the tile's payload start `vp`.
//
//   COO (values):    coord u8[nnz] (row<<4 | col, row-major) @0, padded to
//                    4 B by repeating the last coordinate, values @align4(nnz)
//   COO (pattern):   coord u8[nnz] @0 (padded to 4 B by repeating the last
//                    coordinate); up to COO_INLINE entries: no payload, the
//                    coordinate bytes (padded the same way) sit in the
//                    metadata word
//   Dense:           values[256] row-major @0 (tile start is 512/1024-B aligned)
//   ForceCSR:        row_mask u16[16] @0, row_ptr u8[16] @32, values @48
//                    (row-major, ascending column within a row)
//   ForceCSC:        col_mask u16[16] @0, col_ptr u8[16] @32, values @48
//                    (column-major, ascending row within a column)
//   patched CSR:     row_mask u16[16] @0, row_ptr u8[16] @32, col_ptr u8[16] @48,
//                    row_idx_csc2csr u8[nnz] @64 (column-major; byte = row<<4 |
//                    index of the entry inside its row), values
//                    @64+align16(nnz) row-major
//   any non-COO tile of a pattern matrix:
//                    row_mask u16[16] @0, col_mask u16[16] @32
// Dense tiles store absent entries as zeros, so their structure (needed by
// the OR-AND semiring, where stored zeros count) lives in a fourth section
// after the COO one: row_mask u16[16] per Dense tile, at
// dense_mask_off + 32 * (vp / (256 * value size)).
// Bit k of a row mask is local column k; bit k of a column mask is local row k
// (Figure 5 caption: a row mask of 10 = 0b1010 holds columns 1 and 3).
// ---------------------------------------------------------------------------
#define PL_MASK 0
#define PL_PTR 32
#define PL_FORCE_VAL 48
#define PL_CSR_COLPTR 48
#define PL_CSR_RC 64
#define PL_PAT_COLMASK 32

__host__ __device__ inline uint32_t coo_val_off(uint32_t nnz) { return align_up(nnz, 4); }
__host__ __device__ inline uint32_t csr_val_off(uint32_t nnz) { return PL_CSR_RC + align_up(nnz, 16); }

// Tile metadata word: payload offset (40 bits) | (nnz-1) << 40 | format << 48
// (| row block in its Boolean-pull segment << 52, pattern matrices).
// COO tiles of a pattern matrix with at most COO_INLINE entries keep their
// coordinate bytes in bits 0..31 instead of an offset (bit 51 set) and have
// no payload: the metadata load brings the whole tile.
#define COO_INLINE 4
#define META_INLINE (1ull << 51)
// pattern matrices: the tile's row block within its Boolean-pull segment
#define META_SEG_RB_SHIFT 52
#define META_SEG_RB (15ull << META_SEG_RB_SHIFT)

// Column-block word of the Boolean pull (pattern matrices).  With at most
// CBX_MAX_NB column blocks: the column block in bits 0..18, the tile's row
// block within its Boolean-pull segment in bits 19..22, and for a tile of a
// single entry bit 23 set and the entry's (row << 4 | column) in bits 24..31,
// so such a tile is decoded without its metadata word; for the other tiles
// bits 24..31 hold the tile's rank (its index among the segment's tiles not
// marked single).  Larger matrices: the column block in bits 0..26 and the
// row block within the segment in bits 27..30 (no tile is marked single; a
// tile's rank is its index in the segment).
#define CBX_CB_BITS 19
#define CBX_MAX_NB (1 << CBX_CB_BITS)
#define CBX_RI_SHIFT 19
#define CBX_SINGLE (1u << 23)
#define CBX_RC_SHIFT 24
#define CBX_RI_SHIFT_WIDE 27
__host__ __device__ inline uint64_t meta_pack(uint64_t vp, uint32_t nnz, uint32_t type) {
  return vp | ((uint64_t)(nnz - 1) << 40) | ((uint64_t)type << 48);
}
__host__ __device__ inline bool meta_inline(uint64_t m) { return (m & META_INLINE) != 0; }
__host__ __device__ inline bool coo_is_inline(int vk, uint32_t nnz) { return vk == VK_PAT && nnz <= COO_INLINE; }
__host__ __device__ inline uint64_t meta_vp(uint64_t m) { return m & ((1ull << 40) - 1); }
__host__ __device__ inline uint32_t meta_nnz(uint64_t m) { return (uint32_t)((m >> 40) & 0xFF) + 1; }
__host__ __device__ inline uint32_t meta_type(uint64_t m) { return (uint32_t)((m >> 48) & 0x7); }
// format | inline << 3, from the upper half of a metadata word
__host__ __device__ inline uint32_t meta_kind(uint32_t hi) { return (hi >> 16) & 0xFu; }

// section of a tile in the arena: 0 Dense, 1 mask-based, 2 COO
__host__ __device__ inline int tile_section(int type, int vk) {
  if (type == DBS_TILE_COO) return 2;
  if (type == DBS_TILE_DENSE && vk != VK_PAT) return 0;
  return 1;
}

__host__ __device__ inline uint32_t tile_payload_bytes(int type, uint32_t nnz, int vk) {
  const uint32_t vs = (uint32_t)vk_size(vk);
  if (type == DBS_TILE_COO) {
    if (coo_is_inline(vk, nnz)) return 0;
    return vk == VK_PAT ? align_up(nnz, 4) : coo_val_off(nnz) + align_up(nnz * vs, 4);
  }
  if (vk == VK_PAT) return 64;
  if (type == DBS_TILE_DENSE) return 256 * vs;
  if (type == DBS_TILE_CSR) return align_up(csr_val_off(nnz) + nnz * vs, 16);
  return align_up(PL_FORCE_VAL + nnz * vs, 16);  // ForceCSR / ForceCSC
}

// Pull segment descriptor: {row block | class << 28 | split << 31, first
// tile, end tile, partial slot + 1 (0: none)}.  Split: the row block has
// several segments.  Value matrices only: the row blocks of more than
// SEG_SLOT_MIN segments carry a size class (1: at most 32 segments, 2: at
// most 64, 3: more) and give each segment a partial slot, so that a call can
// write those segments' row sums to slots and add them with a fixed-order
// pairwise finalize instead of same-address atomics.  The class decides per
// call, from the number of waves that share a segment, which row blocks do:
// every other row block receives at most SEG_MAX_ADDS atomic adds per
// y entry (its segments x sharing waves).
#define SEG_SPLIT 0x80000000u
// the segment has a row with more than SEG_DRAIN_ROW entries in its COO tiles
#define SEG_DRAIN 0x40000000u
#define SEG_DRAIN_ROW 32
#define SEG_RB_MASK 0x0FFFFFFFu
#define SEG_CLS_SHIFT 28
#define SEG_SLOT_MIN 16
#define SEG_MAX_ADDS 64
// waves that share one PLUS_TIMES pull segment at most
#define DBS_MAX_SHARE 4
// a partial slot: the 16 row sums, then the epoch of the call that wrote
// them (a slot of another call counts as zero, so a segment with nothing to
// add writes nothing)
#define SLOT_WORDS 17
__host__ __device__ inline uint32_t seg_class(uint32_t nsegs) {
  return nsegs <= SEG_SLOT_MIN ? 0u : nsegs <= 32 ? 1u : nsegs <= 64 ? 2u : 3u;
}
// the smallest class whose row blocks take partial slots when `share` waves
// share a segment (1, 2 or 4): those of class below it have at most
// SEG_MAX_ADDS / share segments
__host__ __device__ inline uint32_t seg_slot_class(int share) { return share >= 4 ? 1u : share == 2 ? 2u : 3u; }
// zeroed bytes allocated after the payload: wide row loads that start inside
// the last tile stay inside the allocation
#define DBS_PAYLOAD_SLACK 256u
// The kernels read the payload, the tile arrays and the staged x through
// buffer descriptors with 32-bit byte offsets, 0xFFFFFFF0 marking a lane with
// nothing to load; every real offset must stay below it.
#define DBS_OFFSET_LIMIT 0xFFFFFFF0ull
// a built format: payload (with its slack) and per-tile metadata (8 B a tile)
__host__ __device__ inline bool dbs_format_fits_offsets(uint64_t payload_bytes, uint64_t tiles) {
  return payload_bytes + DBS_PAYLOAD_SLACK <= DBS_OFFSET_LIMIT && tiles * 8u <= DBS_OFFSET_LIMIT;
}
// the block-padded x of a PLUS_TIMES call: 16 values of vs bytes per block
__host__ __device__ inline bool dbs_x_fits_offsets(uint64_t nb, uint64_t vs) {
  return nb * 16u * vs <= DBS_OFFSET_LIMIT;
}
// tiles per pull segment at most, pattern matrices (the Boolean pull's wave
// holds four tiles per lane)
#define DBS_PAT_SEG_CAP 256
// row blocks per Boolean-pull segment at most (runs of short row blocks)
#define DBS_PAT_MAX_RB 16
static_assert(DBS_PAT_MAX_RB <= 16, "a tile's row block within its segment takes four metadata bits");

// ---------------------------------------------------------------------------
// The handle.
// ---------------------------------------------------------------------------
struct dbs_matrix {
  int device;
  int32_t m, n, mb, nb;
  int64_t nnz, T, nseg;
  int64_t npseg, nseg0;  // pattern matrices: Boolean-pull segments, and those of the first launch
  dbs_dtype dtype;
  int vk;
  dbs_build_options bopt;

  // dual-view blocked format (device)
  uint32_t *rb_ptr;     // [mb+1] block-CSR row pointer
  uint32_t *t_cb;       // [T]    block-CSR column block of each tile (primary order)
  uint64_t *t_meta;     // [T]    payload offset | nnz | format
  uint32_t *cb_ptr;     // [nb+1] block-CSC column pointer
  uint32_t *csc_rb;     // [T]    block-CSC row block
  uint32_t *csc2csr;    // [T]    primary tile id of each CSC position
  uint16_t *csc_cm;     // [T]    columns of the tile that hold entries, CSC order (lets push skip
                        //        tiles without an active column before reading their metadata)
  uint8_t *payload;     // arena
  uint64_t dense_mask_off;  // start of the Dense row-mask section in the arena
  uint32_t *segs;       // [4*nseg] pull segments
  uint32_t *t_cbx;      // [T] pattern matrices: column-block words of the Boolean pull
  uint64_t *meta2;      // pattern matrices: metadata of the tiles not marked single in t_cbx,
                        // tile order (nb > CBX_MAX_NB: t_meta itself, not owned)
  int64_t nmeta2;       // its entries
  uint32_t *m2seg;      // [2*npseg] per Boolean-pull segment: first entry in meta2, entries
  uint8_t *wown;        // pattern matrices: per 4-byte payload word of a COO tile, that tile's index
                        // in its Boolean-pull segment
  uint32_t *psegs;      // [4*npseg] pattern matrices: Boolean-pull segments (first row block, first
                        // tile, end tile, row blocks), first-launch ones ahead
  int64_t payload_bytes;
  uint32_t *rows_nz;    // [(mb+1)/2] rows holding an entry, 16 bits per row block
  // value matrices: row blocks of more than SEG_SLOT_MIN pull segments
  uint32_t *fin;        // [4*nfin] {row block, first slot, segments, class}
  int64_t nfin, nslots;
  int64_t fin_cls[4];   // entries of the list (sorted by segment count) of class >= c
  int64_t fin_big[3];   // leading entries of more than 256 slots with 1, 2 and 4 sharing waves
  float *partial;       // [nslots * DBS_MAX_SHARE * SLOT_WORDS] segment row sums of such row blocks

  // per-call scratch (device)
  uint32_t *xmask;       // [nb] (epoch << 16) | blk_x_mask
  uint32_t *xbits;       // pattern matrices: [2][nbw] a bit per nonzero vector block, by epoch parity
  int32_t nbw;           // (nb + 31) / 32
  void *xd;              // [n] staged x values (only active positions are meaningful)
  uint32_t *act_list;    // [nb] compacted nonzero vector blocks
  uint64_t *chunks;      // [max_chunks] push work: column block | chunk index << 32
  int64_t max_chunks;
  uint32_t *ctr;         // [2][8] double-buffered per-call counters
  uint32_t epoch;
  int cbuf;

  // BFS scratch (allocated on first use)
  uint32_t *bfs_bm;      // 3 frontier bitmaps of nb/2 words (16 bits per vertex block)
  uint32_t *bfs_vis;     // visited bitmap
  uint32_t *bfs_fbits;   // 3 x ceil(nb/64) words: a bit per nonzero word of each frontier bitmap
  uint32_t *bfs_list;    // 3 lists of nb vertex blocks
  uint64_t *bfs_chunks;  // 3 chunk lists
  uint32_t *bfs_ctr;     // 3 x 8 counters, then the frontier sizes of one batch of levels
  uint32_t *bfs_host;    // pinned host mirror of those frontier sizes
  int32_t bfs_src;       // source of the last BFS
  int32_t bfs_counted;   // the last BFS left its visited bitmap in bfs_vis (bfs_reached can be counted)

  // options and statistics
  int64_t opt[8];
  dbs_stats st;
  hipStream_t last_stream;
  // BFS: levels launched between two host reads of the frontier sizes
  static constexpr int kBfsBatch = 8;
  hipEvent_t ev[2 + 2 * kBfsBatch];  // BFS timing: whole run, then each level kernel of a batch
  // ring of per-call event quadruples: start and end of the metadata kernel,
  // start and end of the SpMSpV kernel, taken by the dispatches themselves
  static constexpr int kTimingRing = 64;
  hipEvent_t tev[kTimingRing][4];
  int tev_head, tev_used, tev_ready;
  int64_t mem_now, mem_peak;
};

// ---------------------------------------------------------------------------
// Host-side helpers implemented in the .hip files.
// ---------------------------------------------------------------------------
hipError_t dbs_dev_alloc(dbs_matrix *A, void **p, size_t bytes);
void dbs_dev_free(dbs_matrix *A, void *p, size_t bytes);

// exclusive scans writing n+1 values (out[n] = total)
hipError_t dbs_scan_u32(const uint32_t *in, uint32_t *out, int64_t n, void *tmp, hipStream_t s);
hipError_t dbs_scan_u64(const uint64_t *in, uint64_t *out, int64_t n, void *tmp, hipStream_t s);
size_t dbs_scan_tmp_bytes(int64_t n);
// stable LSD radix sort of (key, value) pairs by key < 2^bits
hipError_t dbs_radix_sort_pairs(uint32_t *keys, uint32_t *vals, uint32_t *keys_tmp,
                                uint32_t *vals_tmp, int64_t n, int bits, void *tmp,
                                hipStream_t s);
size_t dbs_radix_tmp_bytes(int64_t n);

dbs_status dbs_build_impl(dbs_matrix *A, const int32_t *row_ptr, const int32_t *col_idx,
                          const void *val, hipStream_t s);
// thr < 0: a dense x's entries are active iff nonzero; thr >= 0: iff |x_j| > thr
dbs_status dbs_spmspv_impl(dbs_matrix *A, int32_t nnz_x, const int32_t *x_idx,
                           const void *x_val, const void *x_dense, dbs_semiring sr, void *y,
                           hipStream_t s, float thr = -1.0f);
dbs_status dbs_bfs_impl(dbs_matrix *A, int32_t src, int32_t *levels, hipStream_t s);
// the same on the fixed device array, allocating nothing
dbs_status dbs_bfs_noalloc_impl(dbs_matrix *A, int32_t src, int32_t *levels, hipStream_t s);
// fills st.bfs_reached for the last BFS (counts its visited bitmap; synchronous)
dbs_status dbs_bfs_count_reached(dbs_matrix *A);
// next free event triple of the timing ring (folds the oldest into the sums
// when the ring is full); nullptr on a HIP error
hipEvent_t *dbs_timing_slot(dbs_matrix *A);

// Returns e; with DBS_VERBOSE=1 in the environment a failing call is printed
// to stderr with its source location.
hipError_t dbs_note(hipError_t e, const char *file, int line);
#define DBS_NOTE(expr) dbs_note((expr), __FILE__, __LINE__)

// Workgroups of `kernel` (blockDim `threads`) that fit on the device at once
// (occupancy x compute units), at least 1; cached by the caller.
template <class K>
inline unsigned dbs_resident_groups(K kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1024;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 1024;
  const long g = (long)cus * (per_cu > 0 ? per_cu : 1);
  return (unsigned)(g > 0 ? g : 1);
}

#define DBS_HIP_TRY(expr)                                \
  do {                                                   \
    hipError_t e_ = DBS_NOTE(expr);                      \
    if (e_ != hipSuccess) return e_;                     \
  } while (0)

// ---------------------------------------------------------------------------
// Device helpers (wave64).
// ---------------------------------------------------------------------------
#ifdef __HIP_DEVICE_COMPILE__
#define DBS_DEV __device__ __forceinline__
#else
#define DBS_DEV __device__ inline
#endif

DBS_DEV uint32_t below_mask(uint32_t k) { return (1u << k) - 1u; }

// reductions inside aligned groups of `W` lanes
template <int W>
DBS_DEV uint32_t group_min_u32(uint32_t v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, W));
  return v;
}
template <int W>
DBS_DEV uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, W));
  return v;
}
template <int W>
DBS_DEV uint32_t group_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o, W);
  return v;
}
template <int W>
DBS_DEV uint32_t group_or_u32(uint32_t v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, W);
  return v;
}
// inclusive prefix sum inside aligned groups of W lanes
template <int W>
DBS_DEV uint32_t group_incl_scan_u32(uint32_t v) {
  const int l = __lane_id() & (W - 1);
#pragma unroll
  for (int o = 1; o < W; o <<= 1) {
    uint32_t t = (uint32_t)__shfl_up((int)v, o, W);
    if (l >= o) v += t;
  }
  return v;
}

DBS_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
