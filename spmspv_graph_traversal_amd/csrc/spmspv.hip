// DB-SpMSpV on gfx950: vector-block metadata (section 4.1), the global
// push/pull selector (section 3.3.1), path-aware work lists (section 3.3.2)
// and hierarchical writeback (section 3.3.3) of "DB-SpMSpV: Dual-View Blocked
// Sparse Matrix-Sparse Vector Multiplication for Dynamic GPU Workloads".
//
// One call = two launches on the caller's stream:
//   k_xmeta_*   builds blk_x_mask (tagged with a per-call epoch so it never
//               needs clearing), stages x, counts the nonzero vector blocks
//               with one atomic per workgroup, lists them and clears y;
//   k_spmspv    reads N_nzblk, picks push or pull on the device, and walks
//               either the push work chunks (64 tiles of one column block
//               each, enumerated from the list by every workgroup) or the
//               static pull segments, one wave per chunk / segment,
//               grid-stride.  (When a push could involve more blocks than
//               that enumeration holds, k_xmeta_* cuts the chunks ahead.)
#include "meta.h"
#include <hip/hip_ext.h>

#include "pattern_pull.h"
#include "tile_kernels.h"

namespace {

constexpr int KT = 256;  // threads per workgroup (4 waves)

struct MetaOut {
  uint32_t *xmask;
  uint32_t epoch;
  // pattern matrices: this call's active-block bits (set here) and the next
  // call's (cleared here), nbw words each; null otherwise
  uint32_t *bits_set, *bits_clear;
  int32_t nbw;
  dbs_meta::Reg reg;    // this call's counters ([0] N_nzblk, [1] push chunks, [2] error flags, [3] done) and lists
  uint32_t *ctr_next;   // next call's counters, cleared here
  int32_t n, nb;
  // y clearing: head bytes, 16-B body, tail bytes
  uint8_t *y;
  int64_t y_head, y_body, y_tail;
};

DBS_DEV void clear_y(const MetaOut &o) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, gs = (int64_t)gridDim.x * blockDim.x;
  if (gt < o.y_head) o.y[gt] = 0;
  uint4 *body = (uint4 *)(o.y + o.y_head);
  for (int64_t k = gt; k < o.y_body; k += gs) body[k] = make_uint4(0, 0, 0, 0);
  if (gt < o.y_tail) o.y[o.y_head + 16 * o.y_body + gt] = 0;
  // the next call's active-block bits start from zero (this call's array was
  // cleared by the previous call, both in stream order)
  if (o.bits_clear)
    for (int64_t k = gt; k < o.nbw; k += gs) o.bits_clear[k] = 0u;
}

// The bits of the blocks that lanes with `on` register (a dense x), called
// by the whole wave.  Bits of one word are first ORed across the lanes that
// hold it (segmented by runs of equal words), and the first lane of each run
// sets them with one non-returning atomic.
DBS_DEV void set_block_bits(const MetaOut &o, bool on, uint32_t b) {
  if (!o.bits_set) return;  // uniform
  const int lane = __lane_id();
  const uint32_t wi = on ? b >> 5 : 0xFFFFFFFFu;
  uint32_t bits = on ? 1u << (b & 31u) : 0u;
#pragma unroll
  for (int d = 1; d < DBS_WAVE; d <<= 1) {
    const uint32_t ow = (uint32_t)__shfl_down((int)wi, d), ob = (uint32_t)__shfl_down((int)bits, d);
    if (lane + d < DBS_WAVE && ow == wi) bits |= ob;
  }
  const uint32_t pw = (uint32_t)__shfl_up((int)wi, 1);
  if (on && (lane == 0 || pw != wi)) atomicOr(&o.bits_set[wi], bits);
}

// The active-block bits of a sparse x, one round (1024 entries) of a
// workgroup at a time.  The round's leaders set their blocks' bits in an LDS
// window of words starting at the word of the round's first entry; the
// window's words are then written out, the words strictly between the
// round's first and last entries' words with plain stores (a sorted x_idx
// has no other entries there) and the others with non-returning atomics.
// Device-scope atomics on one cache line are served one after another, so
// one atomic per block (up to 1024 per line) cost more than the rest of the
// metadata kernel at high densities.  Blocks outside the window (an x_idx
// that is not sorted) take an atomic each.
constexpr uint32_t BITS_WIN = 1024;
DBS_DEV void block_bits_sparse(const MetaOut &o, int32_t nnz_x, const int32_t *x_idx) {
  __shared__ uint32_t s_w[BITS_WIN];
  __shared__ uint32_t s_lo, s_hi;
  if (!o.bits_set || nnz_x <= 0) return;  // uniform
  const int tid = (int)threadIdx.x;
  const int64_t rounds = ((int64_t)nnz_x + dbs_meta::MT - 1) / dbs_meta::MT;
  for (int64_t r = blockIdx.x; r < rounds; r += gridDim.x) {  // uniform
    const int64_t i0 = r * dbs_meta::MT, i1 = i0 + dbs_meta::MT < nnz_x ? i0 + dbs_meta::MT : nnz_x;
    if (tid == 0) {
      const int32_t f = x_idx[i0], l = x_idx[i1 - 1];
      s_lo = (f >= 0 && f < o.n) ? (uint32_t)f >> 9 : 0u;
      s_hi = (l >= 0 && l < o.n) ? (uint32_t)l >> 9 : 0u;
    }
    for (uint32_t k = (uint32_t)tid; k < BITS_WIN; k += dbs_meta::MT) s_w[k] = 0u;
    __syncthreads();
    const uint32_t lo = s_lo, hi = s_hi;
    const int64_t i = i0 + tid;
    if (i < i1) {
      const int32_t idx = x_idx[i], prev = i > 0 ? x_idx[i - 1] : -1;
      if (idx >= 0 && idx < o.n && (i == 0 || (prev >> 4) != (idx >> 4))) {
        const uint32_t b = (uint32_t)idx >> 4, w = b >> 5, bit = 1u << (b & 31u);
        if (w - lo < BITS_WIN) atomicOr(&s_w[w - lo], bit);  // LDS
        else atomicOr(&o.bits_set[w], bit);
      }
    }
    __syncthreads();
    for (uint32_t k = (uint32_t)tid; k < BITS_WIN; k += dbs_meta::MT) {
      const uint32_t v = s_w[k], w = lo + k;
      if (v != 0u && w < (uint32_t)o.nbw) {
        if (k > 0u && w < hi) o.bits_set[w] = v;
        else atomicOr(&o.bits_set[w], v);
      }
    }
    __syncthreads();
  }
}

// Sparse x: sorted x_idx.  The first entry of each vector block (the leader)
// writes the block's mask: a strictly increasing x_idx holds a block's
// entries one after another, so the mask is an OR over the run of lanes of
// the same block, taken within the wave by a segmented OR (shuffles of
// doubling distance that combine only lanes of equal block); the run of the
// wave's last lane may go on for up to 15 entries after the wave, which its
// leader reads with one load of the wave (lanes 0..14).  Each wave thus
// issues three loads of x_idx rather than one per following entry.
template <int VK>
__global__ __launch_bounds__(dbs_meta::MT) void k_xmeta_sparse(MetaOut o, int32_t nnz_x, const int32_t *x_idx,
                                                     const void *x_val, void *xd, int check) {
  if (blockIdx.x == 0 && threadIdx.x < 8) o.ctr_next[threadIdx.x] = 0;
  clear_y(o);
  dbs_meta::register_blocks(o.reg, nnz_x, [&](int64_t i, int pass, bool &leader, uint32_t &bo) {
    const bool valid = i < nnz_x;
    const int64_t ic = valid ? i : 0;  // clamped index (nnz_x > 0 whenever a round runs)
    const int32_t idx0 = x_idx[ic], prev0 = x_idx[ic > 0 ? ic - 1 : 0];
    const int32_t idx = valid ? idx0 : -1;
    const bool inb = valid && idx >= 0 && idx < o.n;
    const int32_t b = idx >> 4;
    const int32_t prev = (valid && i > 0) ? prev0 : -1;
    leader = inb && (i == 0 || (prev >> 4) != b);
    bo = (uint32_t)b;
    if (pass != 0) return;
    if (inb && VK != VK_PAT && x_val) {
      if (VK == VK_F32) ((float *)xd)[idx] = ((const float *)x_val)[i];
      else ((uint16_t *)xd)[idx] = ((const uint16_t *)x_val)[i];
    }
    // (a strictly increasing x_idx holds at most 16 entries per block, so the
    // check of every pair also rules out a 17th)
    if (check && valid && i > 0 && idx <= prev) atomicOr(&o.reg.ctr[2], 1u);
    const int lane = __lane_id();
    const int32_t key = inb ? b : -1;
    uint32_t mk = inb ? 1u << (idx & 15) : 0u;
#pragma unroll
    for (int d = 1; d < DBS_WAVE; d <<= 1) {
      const uint32_t om = (uint32_t)__shfl_down((int)mk, d);
      const int32_t ok = __shfl_down(key, d);
      if ((lane + d < DBS_WAVE) & (ok == key)) mk |= om;
    }
    // the entries after the wave that belong to its last lane's block
    const int32_t lastk = __builtin_amdgcn_readlane(key, DBS_WAVE - 1);
    const int64_t it = i + DBS_WAVE;  // lane j < 15: entry j after the wave
    const bool tin = (lane < 15) & (it < nnz_x);
    const int32_t tv = x_idx[tin ? it : ic];  // clamped: no branch around the load
    const uint32_t tb = wave_or((tin & (tv >= 0) & (tv < o.n) & ((tv >> 4) == lastk)) ? 1u << (tv & 15) : 0u);
    if (key == lastk) mk |= tb;
    if (leader) o.xmask[b] = (o.epoch << 16) | mk;
  });
  block_bits_sparse(o, nnz_x, x_idx);
}

// Dense x (decode, section 4.1): one ballot per wave gives the nonzero
// pattern of 64 consecutive entries, i.e. the masks of four vector blocks.
// thr >= 0: the activation is sparsified on the way (an entry is active iff
// |x_j| > thr, and the staged x holds 0 for the others).
template <int VK>
__global__ __launch_bounds__(dbs_meta::MT) void k_xmeta_dense(MetaOut o, const void *x, void *xd, float thr) {
  if (blockIdx.x == 0 && threadIdx.x < 8) o.ctr_next[threadIdx.x] = 0;
  clear_y(o);
  const int lane = __lane_id();
  const int64_t npad = (int64_t)o.nb * 16;
  dbs_meta::register_blocks(o.reg, npad, [&](int64_t j, int pass, bool &leader, uint32_t &b) {
    bool nz = false;
    if (j < o.n) {
      const uint32_t bits = VK == VK_BF16 ? (uint32_t)((const uint16_t *)x)[j] << 16 : __float_as_uint(((const float *)x)[j]);
      nz = thr < 0.0f ? (bits & 0x7FFFFFFFu) != 0u : fabsf(__uint_as_float(bits)) > thr;
    }
    const uint64_t bal = __ballot(nz);
    const uint32_t mk = (uint32_t)(bal >> (lane & 48)) & 0xFFFFu;
    const bool head = (lane & 15) == 0 && j < npad;
    b = (uint32_t)(j >> 4);
    leader = head && mk != 0u;
    if (pass == 0 && head) o.xmask[b] = (o.epoch << 16) | mk;
    if (pass == 0) set_block_bits(o, head && mk != 0u, b);
    // PLUS_TIMES: copy x into the block-padded staging vector (zero tail),
    // so the multiply reads whole column quarters of every vector block
    if (pass == 0 && xd && j < npad) {
      if (VK == VK_BF16) ((uint16_t *)xd)[j] = nz ? ((const uint16_t *)x)[j] : (uint16_t)0;
      else ((float *)xd)[j] = nz ? ((const float *)x)[j] : 0.0f;
    }
  });
}

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

struct SpmvParams {
  const uint32_t *t_cbx;   // pattern matrices: the Boolean pull's column-block words
  const uint64_t *meta2;   // pattern matrices: metadata of the tiles not marked single
  const uint32_t *m2seg;   // pattern matrices: per pull segment, first entry in meta2 and entries
  int32_t cbx_compact;     // nb <= CBX_MAX_NB: the words mark single tiles
  const uint32_t *t_cb;
  const uint64_t *t_meta;
  const uint32_t *cb_ptr;
  const uint32_t *csc_rb;
  const uint32_t *csc2csr;
  const uint16_t *csc_cm;   // columns of each tile with entries, CSC order
  const uint8_t *payload;
  uint64_t dense_mask_off;
  const uint32_t *segs;     // pull segments (pattern matrices: the Boolean pull's)
  const uint32_t *rb_ptr;
  const uint8_t *wown;     // pattern matrices: owner tile of each payload word
  int64_t nseg, T, payload_bytes;
  int32_t m, nb;
  const uint32_t *xmask;
  uint32_t epoch;
  const void *xd;
  const uint64_t *chunks;
  int64_t max_chunks;
  const uint32_t *ctr;
  int32_t force_path;
  int64_t th3_num, th3_den;
  int32_t local_cutoff;
  int32_t plus_u;  // segments per wave step of the PLUS_TIMES pull (1 or PULL_U_PLUS_WIDE)
  int32_t plus_parts;  // U = 1: waves sharing one segment (1, 2 or 4), each taking a lane range
  int32_t slot_cls;    // segments of row blocks of at least this class write partial slots
  float *partial;      // the partial slots (finalized by k_plus_finalize), < 4 GiB
  uint32_t partial_bytes;
  const uint32_t *xbits;  // pattern matrices with nbw <= PUSH_LIST_MAX: this call's active-block bits
  int32_t nbw;
  const uint32_t *xlist;  // this call's nonzero vector blocks (N_nzblk of them)
  int32_t list_push;      // push chunks come from xlist (none were built)
  void *y;
};

template <int VK>
DBS_DEV const uint8_t *dense_mask_ptr(const SpmvParams &P, uint64_t vp) {
  constexpr uint64_t TS = VK == VK_F32 ? 1024 : 512;
  return P.payload + P.dense_mask_off + 32 * (vp / TS);
}

// stage the 16 x values of vector block b (0 for inactive entries)
template <int VK>
DBS_DEV void stage_x(float *sx, const void *xd, uint32_t b, uint32_t m, int lane) {
  if (lane < 16) sx[lane] = ((m >> lane) & 1u) ? load_x<VK>(xd, (int64_t)b * 16 + lane) : 0.0f;
  __syncwarp();
}

// ---------------------------------------------------------------------------
// Push: one wave per chunk of up to 64 tiles of one active column block
// (section 3.3.2: tile-level tasks, long column blocks spread over the GPU).
// The block's x values are staged once per chunk (section 3.3.3).
// ---------------------------------------------------------------------------
template <int VK, int SR>
DBS_DEV void push_chunk(const SpmvParams &P, uint64_t own, float *sx, float *spart, int lane) {
  const uint32_t b = (uint32_t)own, j = (uint32_t)(own >> 32);
  const uint32_t m = P.xmask[b] & 0xFFFFu;
  const uint32_t k0 = P.cb_ptr[b] + j * 64u, kend = P.cb_ptr[b + 1];
  const uint32_t k = k0 + (uint32_t)lane;
  // a tile without an entry in an active column adds nothing: its metadata
  // is not read
  const bool act = k < kend && (P.csc_cm[k < kend ? k : k0] & m) != 0u;
  uint32_t rb = 0;
  uint64_t meta = 0;
  if (act) {
    rb = P.csc_rb[k];
    meta = P.t_meta[P.csc2csr[k]];
  }
  const uint32_t type = meta_type(meta);
  if (SR == DBS_PLUS_TIMES) stage_x<VK>(sx, P.xd, b, m, lane);
  // COO tiles: one per lane, contributions go straight to y
  if (act && type == DBS_TILE_COO) {
    const uint8_t *base = P.payload + meta_vp(meta);
    const uint32_t nnz = meta_nnz(meta);
    if (SR == DBS_OR_AND) {
      const uint32_t f = coo_or_meta(P.payload, meta, m);
      for (uint32_t ff = f; ff; ff &= ff - 1u) {
        const uint32_t row = rb * 16u + (uint32_t)(__ffs(ff) - 1);
        ((uint8_t *)P.y)[row] = 1;
      }
    } else {
      constexpr int VS = VK == VK_F32 ? 4 : 2;
      const uint8_t *vals = base + coo_val_off(nnz);
      for (uint32_t e0 = 0; e0 < nnz; e0 += 8) {  // 8 entries per round of independent loads
        const uint32_t w0 = ((const uint32_t *)base)[e0 >> 2];
        const uint32_t w1 = e0 + 4 < nnz ? ((const uint32_t *)base)[(e0 >> 2) + 1] : 0u;
        float a[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = e0 + k < nnz ? load_a<VK>(vals + (e0 + k) * VS) : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t rc = ((k < 4 ? w0 : w1) >> (8 * (k & 3))) & 0xFFu;
          const uint32_t c = rc & 15u;
          if (e0 + k < nnz && ((m >> c) & 1u))
            unsafeAtomicAdd((float *)P.y + rb * 16u + (rc >> 4), a[k] * sx[c]);
        }
      }
    }
  }
  // larger tiles: the whole wave per tile, then local merge and atomics
  uint64_t todo = __ballot(act && type != DBS_TILE_COO);
  while (todo) {
    const int src = __ffsll((unsigned long long)todo) - 1;
    todo &= todo - 1;
    const uint32_t trb = (uint32_t)__shfl((int)rb, src);
    const uint64_t tm = __shfl(meta, src);
    const uint8_t *base = P.payload + meta_vp(tm);
    const uint32_t tt = meta_type(tm);
    if (SR == DBS_OR_AND) {
      const uint32_t f = tile_or<VK>(base, dense_mask_ptr<VK>(P, meta_vp(tm)), tt, m, lane);
      if (lane < 16 && ((f >> lane) & 1u) && (int64_t)trb * 16 + lane < P.m) ((uint8_t *)P.y)[trb * 16u + lane] = 1;
    } else {
      const float part = tile_plus<VK>(base, tt, meta_nnz(tm), m, sx, spart, P.local_cutoff, lane);
      if (lane < 16 && part != 0.0f && (int64_t)trb * 16 + lane < P.m)
        unsafeAtomicAdd((float *)P.y + trb * 16u + lane, part);
    }
  }
}

// ---------------------------------------------------------------------------
// Pull: one wave per static segment of one row block (section 3.3.2).  COO
// tiles are handled one per lane into 16 row registers; larger tiles by the
// whole wave.  The row block's partial is merged in registers and written
// once: a plain store when the row block is one segment, an atomic add when
// several segments share it.
constexpr int PULL_U_PLUS_WIDE = 4;  // segments per wave step, PLUS_TIMES pull with many segments
constexpr int PLUS_MAX_PARTS = DBS_MAX_SHARE;  // waves sharing one PLUS_TIMES pull segment at most
constexpr int PULL_U_OR = 8;    // segments per wave step, OR_AND pull (value matrices)
constexpr int SP_BITS_MAX = sp_bits_max(KT / DBS_WAVE);  // very sparse pull: bits and buffers in s_cum

// ---------------------------------------------------------------------------
// PLUS_TIMES over the COO tiles of the U pull segments of a wave step,
// entries spread over the lanes: the COO tiles' payloads (coordinates, then
// values) follow one another in tile order, so entry j of a segment is entry
// j - start_t of the tile t whose first entry start_t (a wave prefix sum of
// the tiles' entry counts) is the last one at or below j, found by a wave
// max-scan of the tiles' marks.  Each vector memory instruction thus covers
// 64 entries, whatever the tiles' sizes.  Round i takes chunk i (entries
// 64i .. 64i+63 of the segment's run) of every segment that has one, and
// issues all their coordinate and value loads, then all their x loads,
// before any is used, so a step waits about twice per round for memory
// whatever U.
//
// The row sums (hierarchical writeback, section 3.3.3):
//   U == 1: lane l adds its product to its own slot s_acc[row * 64 + l] (16
//           rows x 64 lanes per wave; the LDS bank is the lane, so the adds
//           never conflict and no two lanes share an address); at the end
//           lane (q, r) adds the 16 slots of row r of quarter q's lanes (in
//           a bank-conflict-free order) and the quarters are merged; the
//           slots are cleared on the way;
//   U > 1:  the products go to 16 LDS row sums per segment (lanes of one
//           row add to one address; the hardware adds them one after the
//           other).  A row's chain of adds is then its number of COO entries
//           in the segment: the builder marks (SEG_DRAIN) the segments where
//           a row has more than SEG_DRAIN_ROW of them, and in those the
//           round's row sums are moved to a register after every round (at
//           most 64 adds per round).  Per lane-private slots or a drain of
//           every segment cost the COO-heavy pulls 10-40% more time.
// Every lane returns the total of row (lane & 15) of segment u in
// coo_sum[u]; a product passes through at most rounds + 17 additions
// (U = 1), SEG_DRAIN_ROW (U > 1, unmarked) or 64 + rounds (marked).
// ---------------------------------------------------------------------------
template <int VK, int U>
DBS_DEV void coo_entries_plus_u(const brsrc_t pay, const brsrc_t xr, const bool (&coo)[U], const uint64_t (&meta)[U],
                                const uint32_t (&m)[U], const uint32_t (&cb)[U], uint32_t drain,
                                uint32_t *s_mark, float *s_acc, float (&coo_sum)[U], int lane) {
  // drain: bit u set for a marked segment u (uniform)
  constexpr uint32_t VS = VK == VK_F32 ? 4u : 2u;
  uint32_t cnt[U], start[U], total[U], carry[U];
  uint32_t rounds = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    cnt[u] = coo[u] ? meta_nnz(meta[u]) : 0u;
    start[u] = wave_incl_add(cnt[u]) - cnt[u];
    total[u] = (uint32_t)__builtin_amdgcn_readlane((int)(start[u] + cnt[u]), 63);
    carry[u] = 0u;
    coo_sum[u] = 0.0f;
    const uint32_t r = (total[u] + 63u) >> 6;
    rounds = r > rounds ? r : rounds;
  }
  for (uint32_t i = 0; i < rounds; ++i) {
    const uint32_t j0 = 64u * i;
    int own[U];
    // owner tile of each entry of the round's chunks (lanes talk through
    // LDS, each step fenced at wave scope)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      own[u] = 0;
      if (j0 >= total[u]) continue;  // uniform
      __syncwarp();
      s_mark[lane] = 0u;
      __syncwarp();
      if ((cnt[u] != 0u) & (start[u] >= j0) & (start[u] < j0 + 64u)) s_mark[start[u] - j0] = (uint32_t)lane + 1u;
      __syncwarp();
      uint32_t o = wave_incl_max(s_mark[lane]);
      o = o > carry[u] ? o : carry[u];
      carry[u] = (uint32_t)__builtin_amdgcn_readlane((int)o, 63);
      own[u] = (int)o - 1;
    }
    uint32_t rc[U], ocb[U], om[U];
    float a[U], x[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = j0 + (uint32_t)lane;
      live[u] = j < total[u];
      const uint32_t ovp = (uint32_t)__shfl((int)(uint32_t)meta_vp(meta[u]), own[u]);
      const uint32_t ost = (uint32_t)__shfl((int)start[u], own[u]);
      const uint32_t ocnt = (uint32_t)__shfl((int)cnt[u], own[u]);
      ocb[u] = (uint32_t)__shfl((int)cb[u], own[u]);
      om[u] = (uint32_t)__shfl((int)m[u], own[u]);
      const uint32_t e = j - ost;
      rc[u] = __builtin_amdgcn_raw_buffer_load_b8(pay, live[u] ? ovp + e : OOB_OFF, 0, 0);
      const uint32_t aoff = live[u] ? ovp + coo_val_off(ocnt) + e * VS : OOB_OFF;
      if (VK == VK_F32) a[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pay, aoff, 0, 0));
      else a[u] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(pay, aoff, 0, 0) << 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = rc[u] & 15u;
      live[u] = live[u] & ((om[u] >> c) & 1u);
      const uint32_t xoff = live[u] ? (ocb[u] * 16u + c) * VS : OOB_OFF;
      if (VK == VK_F32) x[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xoff, 0, 0));
      else x[u] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(xr, xoff, 0, 0) << 16);
    }
    if constexpr (U == 1) {
      // lane-private slot: the address differs for every lane
      if (live[0]) atomicAdd(&s_acc[(rc[0] >> 4) * 64u + (uint32_t)lane], a[0] * x[0]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u]) atomicAdd(&s_acc[16 * u + (rc[u] >> 4)], a[u] * x[u]);
      if (drain != 0u) {  // uniform
        // a step with a segment where a row holds more than SEG_DRAIN_ROW COO
        // entries: the round's row sums of every segment go to a register at
        // once, so that no LDS address takes more than 64 adds in a row
        __syncwarp();
#pragma unroll
        for (int u = 0; u < U; ++u) coo_sum[u] += s_acc[16 * u + (lane & 15)];
        __syncwarp();
        if (lane < 16 * U) s_acc[lane] = 0.0f;
      }
    }
  }
  if constexpr (U > 1) {
    __syncwarp();
#pragma unroll
    for (int u = 0; u < U; ++u) coo_sum[u] += s_acc[16 * u + (lane & 15)];
    __syncwarp();
    if (lane < 16 * U) s_acc[lane] = 0.0f;
    __syncwarp();
  }
  if constexpr (U == 1) {
    if (rounds != 0u) {  // uniform
      // lane (q, r) sums row r's slots of quarter q's lanes, starting at a
      // lane that differs with r, so that the 64 reads of each step fall in
      // 64 different banks; then the quarters are added (17 additions)
      __syncwarp();
      const uint32_t q = (uint32_t)lane >> 4, r = (uint32_t)lane & 15u;
      float t = 0.0f;
#pragma unroll 2
      for (uint32_t k = 0; k < 16; ++k) {
        const uint32_t idx = r * 64u + 16u * q + ((k + r) & 15u);
        t += s_acc[idx];
        s_acc[idx] = 0.0f;
      }
      coo_sum[0] = quarter_merge(t);
      __syncwarp();
    }
  }
}

// ---------------------------------------------------------------------------
// Finish one PLUS_TIMES pull segment whose COO entries are summed
// (coo_sum) and whose other tiles are loaded: Dense and CSR-family tiles four
// at a time (row per lane), ForceCSC and few-column patched CSR tiles one at
// a time; then write the row block (section 3.3.3): a plain store when it is
// one segment, the segment's partial slot when its row block is summed by
// the finalize, else an atomic add.  Every product passes through at most
// 16 (within a tile row) + 16 (tiles per lane) + 2 (quarter merge), or the
// COO bound above, or 6 + 64 (one-at-a-time tiles) additions, plus 2 to join
// the three sums.
// ---------------------------------------------------------------------------
template <int VK, bool DENSE_PATH = true>
DBS_DEV void pull_finish(const SpmvParams &P, uint4 seg, uint32_t part, uint32_t cb, uint32_t m, uint64_t meta,
                         bool act, float *sx, float *spart, int lane, float coo_sum) {
  constexpr uint64_t VS = VK == VK_F32 ? 4 : 2;
  const uint32_t rb = seg.x & SEG_RB_MASK;
  const bool split = (seg.x & SEG_SPLIT) != 0u;
  const uint32_t type = meta_type(meta);
  const int64_t row0 = (int64_t)rb * 16;
  const brsrc_t pay = make_rsrc(P.payload, (uint64_t)P.payload_bytes + DBS_PAYLOAD_SLACK);
  const brsrc_t xr = make_rsrc(P.xd, (uint64_t)P.nb * 16 * VS);
  // patched CSR tiles with few active columns take the column variant
  // (section 3.3.3); Dense tiles go four at a time through the row-broadcast
  // path, the other row-major tiles four at a time through the row-per-lane
  // path; ForceCSC tiles one at a time
  const uint64_t colv = __ballot(act & (type == DBS_TILE_CSR) & (__popc(m) < P.local_cutoff));
  const uint64_t dent = DENSE_PATH ? __ballot(act & (type == DBS_TILE_DENSE)) : 0ull;
  const uint64_t rowt = __ballot(act & (type != DBS_TILE_COO) & (type != DBS_TILE_FORCE_CSC)) & ~colv & ~dent;
  float rsum = 0.0f;
  if (dent | rowt) {  // uniform
    float part_r = 0.0f;
    if (dent) part_r = dense_plus<VK>(pay, xr, dent, meta, m, cb, lane);
    if (rowt) part_r += rows_plus<VK>(pay, xr, rowt, meta, m, cb, lane);
    rsum = quarter_merge(part_r);
  }
  float tsum = 0.0f;
  uint64_t todo = __ballot(act & (type == DBS_TILE_FORCE_CSC)) | colv;
  while (todo) {
    const int src = __ffsll((unsigned long long)todo) - 1;
    todo &= todo - 1;
    const uint64_t tm = __shfl(meta, src);
    const uint32_t tmask = (uint32_t)__shfl((int)m, src);
    const uint32_t tcb = (uint32_t)__shfl((int)cb, src);
    stage_x<VK>(sx, P.xd, tcb, tmask, lane);
    tsum += tile_plus<VK>(P.payload + meta_vp(tm), meta_type(tm), meta_nnz(tm), tmask, sx, spart, P.local_cutoff,
                          lane);
    __syncwarp();
  }
  const float rowsum = coo_sum + (rsum + tsum);
  const uint32_t cls = (seg.x >> SEG_CLS_SHIFT) & 3u;
  if (seg.w != 0u && cls >= (uint32_t)P.slot_cls) {  // uniform
    // the row block is summed by the finalize: this segment's (and part's)
    // slot, row sums in lanes 0..15 and this call's epoch in lane 16.  Row
    // sums that are all zero are not written (a store in flight makes the
    // next wait for a load wait for every load in flight): a slot without
    // this call's epoch counts as zero.
    if (__ballot((lane < 16) & (rowsum != 0.0f)) != 0ull) {
      const uint32_t off = (((seg.w - 1u) * (uint32_t)P.plus_parts + part) * SLOT_WORDS + (uint32_t)lane) * 4u;
      const uint32_t v = lane < 16 ? __float_as_uint(rowsum) : P.epoch;
      if (lane < SLOT_WORDS) __builtin_amdgcn_raw_buffer_store_b32(v, make_rsrc(P.partial, P.partial_bytes), off, 0, 0);
    }
    return;
  }
  // y through a descriptor of the row block's entries (built in scalar
  // registers; rows past m fall outside it, so their lanes store nothing)
  const int64_t nrow = P.m - row0 < 16 ? P.m - row0 : 16;
  const brsrc_t yr = make_rsrc((float *)P.y + row0, (uint64_t)nrow * 4);
  if (lane < 16) {
    if (!split) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rowsum), yr, (uint32_t)lane * 4u, 0, 0);
    else if (rowsum != 0.0f) __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(rowsum, yr, lane * 4, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// PLUS_TIMES pull: static segments of one row block each (section 3.3.2),
// U per wave step, software-pipelined in three stages like the Boolean
// pull: while step i works, step i+1 has its mask gathers and step i+2 its
// descriptors, column blocks and (eager) metadata in flight; step i's lazy
// metadata is issued first in the step.
// U = 1 when there are too few segments to give every resident wave several
// (the decode layers), PULL_U_PLUS_WIDE otherwise.  With U = 1 and fewer
// segments than resident waves, two or four waves share a segment, each
// taking a range of its lanes (tiles) and adding its rows atomically.
// ---------------------------------------------------------------------------
struct AllRows {
  DBS_DEV uint32_t need(uint32_t) const { return 0xFFFFu; }
};

template <int VK, int U, bool EAGER>
DBS_DEV void plus_pull_wave(const SpmvParams &P, const PatSrc &S, const brsrc_t xm, int64_t s0, int64_t stride,
                            int parts, float *sx, float *spart, uint32_t *s_mark, float *s_acc, int lane) {
  // work items: segments (U of them per step), or with parts > 1 (U = 1)
  // lane ranges of a segment, item = segment * parts + part
  const int64_t nitems = S.nseg * parts;
  if (s0 >= nitems) return;
  auto seg_of = [&](int64_t it) { return parts == 1 ? it : it / parts; };
  auto lanes_of = [&](int64_t it) {  // lanes (tiles) of the item's part
    if (parts == 1) return ~0ull;
    const int w = 64 / parts;
    return ((1ull << w) - 1ull) << (w * (int)(it % parts));
  };
  const uint32_t l4 = (uint32_t)lane * 4u, l8 = (uint32_t)lane * 8u;
  const AllRows pol;
  const brsrc_t xr = make_rsrc(P.xd, (uint64_t)P.nb * 16 * (VK == VK_F32 ? 4 : 2));
  auto masks = [&](const PatRound<U> &g, uint32_t (&m)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w = bld32(xm, (uint32_t)lane < g.n[u] ? g.cb[u] * 4u : OOB_OFF);
      m[u] = ((w >> 16) == P.epoch) ? (w & 0xFFFFu) : 0u;  // an idle lane reads 0: no epoch
    }
  };
  PatRound<U> g0, g1, g2;
  uint32_t m0[U], m1[U];
  const int64_t s1 = s0 + stride;
  pat_issue<U, EAGER>(S, pol, seg_of(s0), true, l4, l8, g0);
  pat_issue<U, EAGER>(S, pol, seg_of(s1 < nitems ? s1 : s0), s1 < nitems, l4, l8, g1);
  masks(g0, m0);
  while (true) {
    if constexpr (!EAGER) {
      // metadata of this step's active tiles, before the later loads
#pragma unroll
      for (int u = 0; u < U; ++u)
        g0.meta[u] = bld64(make_rsrc(S.t_meta + g0.seg[u].y, (uint64_t)g0.n[u] * 8u), m0[u] != 0u ? l8 : OOB_OFF);
    }
    const int64_t s2 = s0 + 2 * stride;
    pat_issue<U, EAGER>(S, pol, seg_of(s2 < nitems ? s2 : s0), s2 < nitems, l4, l8, g2);
    masks(g1, m1);
    // this item's tiles; a segment shared by several waves adds its rows atomically
    const bool mine = (lanes_of(s0) >> lane) & 1ull;
    uint32_t ma[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ma[u] = mine ? m0[u] : 0u;
    // the COO entries of all U segments first (their loads batched), then
    // each segment's other tiles and writeback; a segment with no active
    // tile has nothing to add (y was cleared by the metadata kernel)
    bool coo[U];
    uint64_t any_coo = 0ull;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      coo[u] = (ma[u] != 0u) & (meta_type(g0.meta[u]) == DBS_TILE_COO);
      any_coo |= __ballot(coo[u]);
    }
    float coo_sum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) coo_sum[u] = 0.0f;
    if (any_coo != 0ull) {  // uniform
      uint32_t drain = 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) drain |= ((g0.seg[u].x >> 30) & 1u) << u;  // SEG_DRAIN
      coo_entries_plus_u<VK, U>(S.pay, xr, coo, g0.meta, ma, g0.cb, drain, s_mark, s_acc, coo_sum, lane);
    }
    const uint32_t part = (uint32_t)s0 & (uint32_t)(parts - 1);  // parts is 1, 2 or 4
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint4 sg = g0.seg[u];
      if (parts > 1) sg.x |= SEG_SPLIT;
      // a segment with no active tile has nothing to add (y was cleared by
      // the metadata kernel; a slot it does not write counts as zero)
      if ((s0 + u < nitems) && __ballot(ma[u] != 0u) != 0ull)  // uniform
        pull_finish<VK, U == 1>(P, sg, part, g0.cb[u], ma[u], g0.meta[u], ma[u] != 0u, sx, spart, lane,
                                coo_sum[u]);
    }
    s0 += stride;
    if (s0 >= nitems) break;
    g0 = g1;
    g1 = g2;
#pragma unroll
    for (int u = 0; u < U; ++u) m0[u] = m1[u];
  }
}

template <int VK, int U>
DBS_DEV void plus_pull(const SpmvParams &P, int64_t gw, int64_t nw, bool eager, float *sx, float *spart,
                       uint32_t *s_mark, float *s_acc, int lane) {
  const PatSrc S{P.t_cb, P.t_meta, P.segs, P.nseg,
                 make_rsrc(P.payload, (uint64_t)P.payload_bytes + DBS_PAYLOAD_SLACK), make_rsrc(nullptr, 0)};
  const brsrc_t xm = make_rsrc(P.xmask, (uint64_t)P.nb * 4);
  const int parts = U == 1 ? P.plus_parts : 1;
  // the COO slots start (and are left) at zero
  if constexpr (U == 1) {
#pragma unroll
    for (int k = 0; k < 16; ++k) s_acc[k * 64 + lane] = 0.0f;
  } else {
    if (lane < 16 * U) s_acc[lane] = 0.0f;
  }
  __syncwarp();
  if (eager) plus_pull_wave<VK, U, true>(P, S, xm, gw * U, nw * U, parts, sx, spart, s_mark, s_acc, lane);
  else plus_pull_wave<VK, U, false>(P, S, xm, gw * U, nw * U, parts, sx, spart, s_mark, s_acc, lane);
}

// OR-AND pull (the Boolean semiring of graph traversal): as pull_group, with
// buffer loads, out-of-range offsets for idle lanes, guard-free COO decoding
// and a DPP wave OR, which keeps the per-tile instruction count small enough
// for the hypersparse tiles of power-law graphs (mostly 1-4 entries).
// buffer descriptors of the arrays the pull reads per tile (built in the kernel)
struct PullRes {
  brsrc_t tcb, tmeta, pay, xmask;
};

// write the found rows of one segment's row block (lanes 0..15)
DBS_DEV void pull_or_store(const SpmvParams &P, uint4 seg, uint32_t f, int lane) {
  const uint32_t rb = seg.x & SEG_RB_MASK;
  const int64_t row = (int64_t)rb * 16 + lane;
  if (lane < 16 && row < P.m) {
    const uint8_t bit = (uint8_t)((f >> lane) & 1u);
    if (!(seg.x & SEG_SPLIT)) ((uint8_t *)P.y)[row] = bit;
    else if (bit) ((uint8_t *)P.y)[row] = 1;
  }
}

// OR-AND SpMSpV on a pattern matrix: every row is wanted, masks are this
// call's epoch-tagged blk_x_mask words, found rows are set in y (cleared by
// the metadata kernel, so only ones are written).  FILTER: the call's
// active-block bits are in LDS, and only the tiles whose column block is
// active read its mask word from memory.  Those reads (a cache line per lane)
// are the costliest part of the pull when few blocks are active.
template <bool FILTER>
struct OrPol {
  brsrc_t xmask;
  uint32_t epoch;
  int32_t m;
  uint8_t *y;
  const uint32_t *bits;  // FILTER: LDS, a bit per column block
  DBS_DEV uint32_t need_v(uint32_t, bool) const { return 0xFFFFu; }
  DBS_DEV uint32_t mask(uint32_t cb, bool in) const {
    if constexpr (FILTER) in = in && active(cb);  // idle lanes hold cb 0
    return mask_of(mask_raw(cb, in), cb);
  }
  // the column block is active this call (its LDS bit)
  DBS_DEV bool active(uint32_t cb) const { return (bits[cb >> 5] >> (cb & 31u)) & 1u; }
  // the mask word as loaded, and the mask it gives (split so that the load
  // can stay in flight)
  DBS_DEV uint32_t mask_raw(uint32_t cb, bool in) const { return bld32(xmask, in ? cb * 4u : OOB_OFF); }
  DBS_DEV uint32_t mask_of(uint32_t w, uint32_t) const {
    return ((w >> 16) == epoch) ? (w & 0xFFFFu) : 0u;  // an idle lane reads 0: no epoch
  }
  // found rows of n row blocks (LDS): four row blocks per pass, a lane per
  // row (every row is wanted: the very sparse pull's rows are the same)
  DBS_DEV void flush_new(const uint32_t *frb, const uint32_t *ff, int n, int lane) const { flush(frb, ff, n, lane); }
  DBS_DEV void flush(const uint32_t *frb, const uint32_t *ff, int n, int lane) const {
    for (int e0 = 0; e0 < n; e0 += 4) {
      const int e = e0 + (lane >> 4), r = lane & 15;
      const bool in = e < n;
      const uint32_t rb = frb[in ? e : 0], f = in ? ff[e] : 0u;
      const int64_t row = (int64_t)rb * 16 + r;
      if (((f >> r) & 1u) & (row < m)) y[row] = 1;
    }
  }
};

template <int VK, int U>
DBS_DEV void pull_or_group(const SpmvParams &P, const PullRes &R, int64_t s0, bool eager, int lane) {
  uint4 seg[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t si = s0 + u < P.nseg ? s0 + u : P.nseg - 1;
    seg[u] = ((const uint4 *)P.segs)[si];
  }
  uint32_t cb[U], m[U], pw0[U], pw1[U];
  uint64_t meta[U];
  bool act[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t t = seg[u].y + (uint32_t)lane;
    act[u] = s0 + u < P.nseg && t < seg[u].z;
    cb[u] = bld32(R.tcb, act[u] ? t * 4u : OOB_OFF);
    meta[u] = eager ? bld64(R.tmeta, act[u] ? t * 8u : OOB_OFF) : 0ull;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // an idle lane reads 0, which no epoch (>= 1) matches: the mask needs no
    // second test of act, so nothing makes the load conditional
    const uint32_t w = bld32(R.xmask, act[u] ? cb[u] * 4u : OOB_OFF);
    m[u] = ((w >> 16) == P.epoch) ? (w & 0xFFFFu) : 0u;
    act[u] = m[u] != 0u;
  }
  if (!eager) {
#pragma unroll
    for (int u = 0; u < U; ++u) meta[u] = bld64(R.tmeta, act[u] ? (seg[u].y + (uint32_t)lane) * 8u : OOB_OFF);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool pre = act[u] & (meta_type(meta[u]) == DBS_TILE_COO) & !meta_inline(meta[u]);
    const uint32_t off = pre ? (uint32_t)meta_vp(meta[u]) : OOB_OFF;
    pw0[u] = bld32(R.pay, off);
    pw1[u] = bld32(R.pay, (pre & (meta_nnz(meta[u]) > 4)) ? off + 4u : OOB_OFF);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (s0 + u >= P.nseg) break;
    uint32_t f = lane_coo_or(P.payload, meta[u], m[u], act[u], pw0[u], pw1[u]);
    uint64_t todo = __ballot(act[u] & (meta_type(meta[u]) != DBS_TILE_COO));
    while (todo) {
      const int src = __ffsll((unsigned long long)todo) - 1;
      todo &= todo - 1;
      const uint64_t tm = __shfl(meta[u], src);
      const uint32_t tmask = (uint32_t)__shfl((int)m[u], src);
      f |= tile_or<VK>(P.payload + meta_vp(tm), dense_mask_ptr<VK>(P, meta_vp(tm)), meta_type(tm), tmask,
                       lane);
    }
    pull_or_store(P, seg[u], wave_or(f), lane);
  }
}

// PU: segments per wave step of the PLUS_TIMES pull (1 or PULL_U_PLUS_WIDE;
// 1 for OR_AND), a kernel each so that each has its own register count.
// The bf16 PLUS_TIMES pull with PU = 1 (the decode layers) and the Boolean
// pull of pattern matrices run five waves per SIMD (at most 96 VGPRs), the
// wide PLUS_TIMES pull four (at most 128); the others keep their own
// register counts.
template <int VK, int SR, int PU>
__global__ __launch_bounds__(KT, ((VK == VK_BF16 && SR == DBS_PLUS_TIMES && PU == 1) ||
                                  (VK == VK_PAT && SR == DBS_OR_AND))
                                     ? 5
                                 : PU > 1 ? 4
                                          : 1) void k_spmspv(
    SpmvParams P) {
  __shared__ float s_x[KT / DBS_WAVE][16];
  __shared__ float s_part[KT / DBS_WAVE][64];
  __shared__ uint32_t s_mark[KT / DBS_WAVE][64];
  __shared__ uint32_t s_cum[SR == DBS_OR_AND ? dbs_meta::PUSH_LIST_MAX : 1];
  __shared__ uint32_t s_pat[VK == VK_PAT && SR == DBS_OR_AND ? KT / DBS_WAVE : 1][PAT_LDS_WORDS];
  // PLUS_TIMES pull: COO row sums, lane-private (16 rows x 64 lanes per wave)
  // with one segment per step, 16 per segment of a step otherwise
  __shared__ float s_acc[SR == DBS_PLUS_TIMES ? KT / DBS_WAVE : 1][SR == DBS_PLUS_TIMES ? (PU == 1 ? 1024 : 16 * PU) : 1];
  const int lane = __lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / DBS_WAVE);
  const uint32_t nz = dbs_meta::nzblk_clamped(P.ctr[0], P.nb);
  const bool push = dbs_meta::selector_push(nz, P.nb, P.force_path, P.th3_num, P.th3_den);
  const int64_t gw = (int64_t)blockIdx.x * (KT / DBS_WAVE) + w;
  const int64_t nw = (int64_t)gridDim.x * (KT / DBS_WAVE);
  if (push) {
    // OR_AND: the work chunks come from the block list (enumerated here);
    // PLUS_TIMES (whose pull kernels have no registers to spare) and OR_AND
    // calls that may push more blocks than the enumeration holds: from the
    // chunk list built ahead
    if (SR == DBS_OR_AND && P.list_push) {  // uniform
      dbs_meta::Listed L;
      const uint32_t nch = dbs_meta::listed_chunks<KT>(L, P.xlist, nz, P.cb_ptr, s_cum);
      for (int64_t c = gw; c < nch; c += nw)
        push_chunk<VK, SR>(P, dbs_meta::listed_chunk(L, (uint32_t)c), s_x[w], s_part[w], lane);
    } else {
      const int64_t nch = (int64_t)P.ctr[1] < P.max_chunks ? (int64_t)P.ctr[1] : P.max_chunks;
      for (int64_t c = gw; c < nch; c += nw) push_chunk<VK, SR>(P, P.chunks[c], s_x[w], s_part[w], lane);
    }
  } else {
    // metadata of every tile is loaded up front once most vector blocks are active
    const bool eager = (int64_t)nz * 4 > (int64_t)P.nb;
    if (SR == DBS_OR_AND) {
      constexpr int U = PULL_U_OR;
      PullRes R;
      R.tcb = make_rsrc(P.t_cb, (uint64_t)P.T * 4);
      R.tmeta = make_rsrc(P.t_meta, (uint64_t)P.T * 8);
      R.pay = make_rsrc(P.payload, (uint64_t)P.payload_bytes + DBS_PAYLOAD_SLACK);
      R.xmask = make_rsrc(P.xmask, (uint64_t)P.nb * 4);
      if constexpr (VK == VK_PAT) {
        const PatSrc S{P.t_cb,
                       P.t_meta,
                       P.segs,
                       P.nseg,
                       R.pay,
                       make_rsrc(P.wown, (uint64_t)(P.payload_bytes + DBS_PAYLOAD_SLACK) / 4),
                       P.t_cbx,
                       P.cbx_compact ? (uint32_t)(CBX_MAX_NB - 1) : (1u << CBX_RI_SHIFT_WIDE) - 1u,
                       P.cbx_compact ? CBX_SINGLE : 0u,
                       P.cbx_compact ? (uint32_t)CBX_RI_SHIFT : (uint32_t)CBX_RI_SHIFT_WIDE,
                       P.meta2,
                       (const uint2 *)P.m2seg};
        if (!eager && P.xbits) {  // uniform
          // the active-block bits in the push enumeration's LDS
          for (int i = (int)threadIdx.x; i < P.nbw; i += KT) s_cum[i] = P.xbits[i];
          __syncthreads();
          const OrPol<true> pol{R.xmask, P.epoch, P.m, (uint8_t *)P.y, s_cum};
          if (P.nbw <= SP_BITS_MAX)  // uniform: the found-row buffers fit after the bits
            pattern_pull_sparse<PAT_K>(S, pol, gw, nw, lane, s_pat[w], s_cum + SP_BITS_MAX + w * 2 * SP_FOUND_CAP);
          else pattern_pull<true>(S, pol, gw, nw, false, lane, s_pat[w]);
        } else {
          const OrPol<false> pol{R.xmask, P.epoch, P.m, (uint8_t *)P.y, nullptr};
          pattern_pull(S, pol, gw, nw, eager, lane, s_pat[w]);
        }
      } else {
        for (int64_t s = gw * U; s < P.nseg; s += nw * U) pull_or_group<VK, U>(P, R, s, eager, lane);
      }
    } else {
      plus_pull<VK, PU>(P, gw, nw, eager, s_x[w], s_part[w], s_mark[w], s_acc[w], lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Finalize of the row blocks whose pull segments wrote partial slots this
// call (long row blocks split over many segments, section 3.3.2; the last
// level of the hierarchical writeback, section 3.3.3): y of each of their
// rows is the sum of K = segments x sharing waves row sums, in one fixed
// order, so the result does not depend on the order the waves ran in.  The
// list runs from the longest row block down (only its first entries take
// slots at a given sharing).  The first nbig entries (more than 256 slots)
// get a workgroup of 1024 threads each, the others a wave each (16 per
// workgroup).  Thread (g, r) of a row block's G groups of 16 takes the
// blocks of 16 consecutive slots b = g, g + G, ..., sums each block pairwise
// for row r (four levels) and keeps the block sums in a binary counter
// (level k holds the sum of 2^k consecutive blocks, earlier blocks on the
// left); the G group sums of a row are then added pairwise (through LDS for
// G = 64, by lane exchanges for G = 4).  A slot's value passes through at
// most 4 + 2 ceil(log2(blocks per group)) + 1 + log2(G) additions here.  A
// slot that does not carry this call's epoch was not written by this call
// (its segment had nothing to add) and counts as zero.
// ---------------------------------------------------------------------------
constexpr int FIN_LV = 24;  // counter levels: up to 2^24 blocks per group

// one block of 16 slots for row r: the values and, from lane j of the
// 16-lane group, slot j's epoch tag
struct FinBlock {
  float v[16];
  uint32_t tag;
};

DBS_DEV FinBlock fin_load(const float *partial, uint64_t base, uint32_t K, uint32_t b, int r) {
  FinBlock f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t k = b * 16u + (uint32_t)j;
    f.v[j] = partial[(base + (k < K ? k : 0u)) * SLOT_WORDS + (uint32_t)r];
  }
  const uint32_t kr = b * 16u + (uint32_t)r;
  f.tag = kr < K ? __float_as_uint(partial[(base + kr) * SLOT_WORDS + 16u]) : 0u;
  return f;
}

template <int J = 0>
DBS_DEV void fin_mask(FinBlock &f, uint32_t epoch) {
  if constexpr (J < 16) {
    const uint32_t t = quarter_bcast<J>(f.tag);  // slot J's tag, from lane J of the group
    f.v[J] = t == epoch ? f.v[J] : 0.0f;
    fin_mask<J + 1>(f, epoch);
  }
}

// group g's sum of row r over blocks g, g + G, ... (every lane of the wave
// takes part: the tag broadcast works on whole rows of 16 lanes)
DBS_DEV float fin_group(const float *partial, uint64_t base, uint32_t K, uint32_t g, uint32_t G, int r,
                        uint32_t epoch) {
  const uint32_t nblk = (K + 15u) >> 4;
  float st[FIN_LV];
#pragma unroll
  for (int lv = 0; lv < FIN_LV; ++lv) st[lv] = 0.0f;
  uint32_t cnt = 0;
  uint32_t b = g;
  FinBlock cur = fin_load(partial, base, K, b < nblk ? b : 0u, r);
  const uint32_t iters = (nblk + G - 1u) / G;  // the same for every group of the row block
  for (uint32_t it = 0; it < iters; ++it) {    // the next block's loads in flight
    const uint32_t bn = b + G;
    const FinBlock nxt = fin_load(partial, base, K, bn < nblk ? bn : 0u, r);
    fin_mask(cur, epoch);
#pragma unroll
    for (int w = 1; w < 16; w <<= 1)
#pragma unroll
      for (int j = 0; j < 16; j += 2 * w) cur.v[j] = cur.v[j] + cur.v[j + w];
    if (b < nblk) {
      // binary counter: merge the levels below the first free one
      float bs = cur.v[0];
      const uint32_t t = (uint32_t)__builtin_ctz(~cnt);
#pragma unroll
      for (int lv = 0; lv < FIN_LV; ++lv)
        if ((uint32_t)lv < t) bs = st[lv] + bs;
#pragma unroll
      for (int lv = 0; lv < FIN_LV; ++lv)
        if ((uint32_t)lv == t) st[lv] = bs;
      ++cnt;
    }
    cur = nxt;
    b = bn;
  }
  // fold the counter, the most recent (lowest) level first
  float tot = 0.0f;
  bool have = false;
#pragma unroll
  for (int lv = 0; lv < FIN_LV; ++lv) {
    if ((cnt >> lv) & 1u) {
      tot = have ? st[lv] + tot : st[lv];
      have = true;
    }
  }
  return tot;
}

__global__ __launch_bounds__(1024) void k_plus_finalize(const uint32_t *fin, int64_t nfin, int64_t nbig,
                                                       const float *partial, int32_t parts, uint32_t epoch,
                                                       const uint32_t *ctr, int32_t nb, int32_t force_path,
                                                       int64_t th3_num, int64_t th3_den, float *y, int32_t m) {
  __shared__ float s_g[64][16];  // [thread group][row]
  const uint32_t nz = dbs_meta::nzblk_clamped(ctr[0], nb);
  if (dbs_meta::selector_push(nz, nb, force_path, th3_num, th3_den)) return;  // uniform: pushed, no slots
  const int tid = (int)threadIdx.x, r = tid & 15;
  if ((int64_t)blockIdx.x < nbig) {
    // a long row block: 64 groups of 16 threads
    const int64_t e = blockIdx.x;
    const uint32_t rb = fin[4 * e], slot0 = fin[4 * e + 1], nsegs = fin[4 * e + 2];
    const int g = tid >> 4;
    const float tot = fin_group(partial, (uint64_t)slot0 * (uint32_t)parts, nsegs * (uint32_t)parts, (uint32_t)g,
                                64u, r, epoch);
    s_g[g][r] = tot;
    __syncthreads();
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) {
      if ((g & (2 * w - 1)) == 0) s_g[g][r] = s_g[g][r] + s_g[g + w][r];
      __syncthreads();
    }
    const int64_t row = (int64_t)rb * 16 + r;
    if (g == 0 && row < m) y[row] = s_g[0][r];
    return;
  }
  // the others: a wave each, 4 groups of 16 lanes
  const int64_t e = nbig + ((int64_t)blockIdx.x - nbig) * 16 + (tid >> 6);
  if (e >= nfin) return;  // uniform per wave
  const uint32_t rb = fin[4 * e], slot0 = fin[4 * e + 1], nsegs = fin[4 * e + 2];
  const int lane = tid & 63;
  const float tot = fin_group(partial, (uint64_t)slot0 * (uint32_t)parts, nsegs * (uint32_t)parts,
                              (uint32_t)(lane >> 4), 4u, r, epoch);
  const float sum = quarter_merge(tot);  // (g0 + g1) + (g2 + g3)
  const int64_t row = (int64_t)rb * 16 + r;
  if (lane < 16 && row < m) y[row] = sum;
}

inline unsigned grid_for(int64_t waves, unsigned cap) {
  int64_t g = (waves + (KT / DBS_WAVE) - 1) / (KT / DBS_WAVE);
  if (g < 1) g = 1;
  return (unsigned)(g < cap ? g : cap);
}

// launch; with timing events, the dispatch itself records its start and end
// (the extended launch costs the host more, so only then)
template <typename K, typename... Args>
void launch_k(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1, Args... args) {
  if (e0 || e1) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// returns the number of waves that share a segment (1 unless PLUS_TIMES
// with one segment per step)
template <int VK, int SR, int PU = 1>
int launch_spmspv(SpmvParams P, int64_t waves, int share, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  static const unsigned resident = dbs_resident_groups(k_spmspv<VK, SR, PU>, KT);
  P.plus_parts = 1;
  if (SR == DBS_PLUS_TIMES && PU == 1 && P.nseg > 0) {
    // fewer segments than resident waves: waves share segments by lane
    // range, so that every resident wave has work (or as forced)
    const int64_t rw = (int64_t)resident * (KT / DBS_WAVE);
    const int64_t parts = (rw + P.nseg - 1) / P.nseg;
    P.plus_parts = share ? share : parts >= PLUS_MAX_PARTS ? PLUS_MAX_PARTS : parts >= 2 ? 2 : 1;
    if (P.nseg * P.plus_parts > waves) waves = P.nseg * P.plus_parts;
  }
  P.slot_cls = (int32_t)seg_slot_class(P.plus_parts);
  launch_k(k_spmspv<VK, SR, PU>, dim3(grid_for(waves, resident)), dim3(KT), s, e0, e1, P);
  return P.plus_parts;
}

}  // namespace

#define SPMV_TRY(expr)                                   \
  do {                                                   \
    if (DBS_NOTE(expr) != hipSuccess) return DBS_ERR_DEVICE;     \
  } while (0)

dbs_status dbs_spmspv_impl(dbs_matrix *A, int32_t nnz_x, const int32_t *x_idx, const void *x_val,
                           const void *x_dense, dbs_semiring sr, void *y, hipStream_t s, float thr) {
  const bool timing = A->opt[DBS_OPT_TIMING] != 0;
  // epoch tag of this call's masks; a full clear every 65535 calls
  A->epoch++;
  if (A->epoch > 0xFFFFu) {
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((A->nb + 255) / 256)), dim3(256), 0, s, A->xmask,
                       (int64_t)A->nb, 0u);
    SPMV_TRY(hipGetLastError());
    if (A->partial) {  // the partial slots' epoch tags too
      const int64_t words = A->nslots * DBS_MAX_SHARE * SLOT_WORDS;
      hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, (uint32_t *)A->partial,
                         words, 0u);
      SPMV_TRY(hipGetLastError());
    }
    A->epoch = 1;
  }
  MetaOut o;
  o.xmask = A->xmask;
  o.epoch = A->epoch;
  o.nbw = A->nbw;
  // the active-block bits serve only pulls that read metadata lazily (under
  // a quarter of the blocks active); a sorted sparse x of more than 4 N_blk
  // entries has more active blocks than that, so they are not written (the
  // array this call would fill stays as the last call cleared it)
  const bool lazy_possible = x_dense != nullptr || (int64_t)nnz_x <= 4 * (int64_t)A->nb;
  o.bits_set = A->xbits && lazy_possible ? A->xbits + (size_t)(A->epoch & 1u) * A->nbw : nullptr;
  o.bits_clear = A->xbits ? A->xbits + (size_t)((A->epoch + 1u) & 1u) * A->nbw : nullptr;
  o.reg.ctr = A->ctr + 8 * A->cbuf;
  o.reg.list = A->act_list;
  o.reg.chunks = A->chunks;
  o.reg.list_cap = A->nb;
  o.reg.chunk_cap = A->max_chunks;
  o.reg.cb_ptr = A->cb_ptr;
  o.reg.nb = A->nb;
  o.reg.force_path = (int32_t)A->opt[DBS_OPT_PATH];
  o.reg.th3_num = A->opt[DBS_OPT_TH3_NUM];
  o.reg.th3_den = A->opt[DBS_OPT_TH3_DEN];
  const bool list_push =
      sr == DBS_OR_AND &&
      dbs_meta::push_from_list(A->nb, A->opt[DBS_OPT_PATH], A->opt[DBS_OPT_TH3_NUM], A->opt[DBS_OPT_TH3_DEN]);
  o.reg.build_chunks = list_push ? 0 : 1;
  o.ctr_next = A->ctr + 8 * (1 - A->cbuf);
  o.n = A->n;
  o.nb = A->nb;
  const int64_t ybytes = (int64_t)A->m * (sr == DBS_OR_AND ? 1 : 4);
  o.y = (uint8_t *)y;
  int64_t head = (int64_t)((16 - ((uintptr_t)y & 15)) & 15);
  if (head > ybytes) head = ybytes;
  o.y_head = head;
  o.y_body = (ybytes - head) / 16;
  o.y_tail = ybytes - head - 16 * o.y_body;

  const bool dense = x_dense != nullptr;
  const int64_t xwork = dense ? (int64_t)A->nb * 16 : (int64_t)nnz_x;
  const unsigned mgrid = dbs_meta::groups_for(xwork, o.y_body);

  // metadata uses the value kind of x: the matrix kind, or f32 for a
  // dense x on a pattern matrix
  int xk = A->vk;
  if (xk == VK_PAT) xk = dense ? VK_F32 : VK_PAT;

  hipEvent_t *tev = nullptr;
  if (timing) {
    tev = dbs_timing_slot(A);
    if (!tev) return DBS_ERR_DEVICE;
  }
  hipEvent_t m0 = tev ? tev[0] : nullptr, m1 = tev ? tev[1] : nullptr;
  hipEvent_t c0 = tev ? tev[2] : nullptr, c1 = tev ? tev[3] : nullptr;
  if (dense) {
    void *xd = sr == DBS_PLUS_TIMES ? A->xd : nullptr;
    if (xk == VK_BF16)
      launch_k(k_xmeta_dense<VK_BF16>, dim3(mgrid), dim3(dbs_meta::MT), s, m0, m1, o, x_dense, xd, thr);
    else launch_k(k_xmeta_dense<VK_F32>, dim3(mgrid), dim3(dbs_meta::MT), s, m0, m1, o, x_dense, xd, thr);
  } else {
    const int check = (int)A->opt[DBS_OPT_CHECK];
    const void *xv = sr == DBS_PLUS_TIMES ? x_val : nullptr;
    if (xk == VK_F32)
      launch_k(k_xmeta_sparse<VK_F32>, dim3(mgrid), dim3(dbs_meta::MT), s, m0, m1, o, nnz_x, x_idx, xv, A->xd, check);
    else if (xk == VK_BF16)
      launch_k(k_xmeta_sparse<VK_BF16>, dim3(mgrid), dim3(dbs_meta::MT), s, m0, m1, o, nnz_x, x_idx, xv, A->xd, check);
    else
      launch_k(k_xmeta_sparse<VK_PAT>, dim3(mgrid), dim3(dbs_meta::MT), s, m0, m1, o, nnz_x, x_idx, xv, A->xd, check);
  }
  SPMV_TRY(hipGetLastError());

  SpmvParams P;
  P.T = A->T;
  P.payload_bytes = A->payload_bytes;
  P.t_cb = A->t_cb;
  P.t_cbx = A->t_cbx;
  P.meta2 = A->meta2;
  P.m2seg = A->m2seg;
  P.cbx_compact = A->nb <= CBX_MAX_NB;
  P.t_meta = A->t_meta;
  P.cb_ptr = A->cb_ptr;
  P.csc_rb = A->csc_rb;
  P.csc2csr = A->csc2csr;
  P.csc_cm = A->csc_cm;
  P.payload = A->payload;
  P.dense_mask_off = A->dense_mask_off;
  P.segs = A->vk == VK_PAT ? A->psegs : A->segs;
  P.nseg = A->vk == VK_PAT ? A->npseg : A->nseg;
  P.rb_ptr = A->rb_ptr;
  P.wown = A->wown;
  P.m = A->m;
  P.nb = A->nb;
  P.xmask = A->xmask;
  P.epoch = A->epoch;
  // the Boolean pull stages the active-block bits in LDS when they fit
  P.xbits = (A->xbits && sr == DBS_OR_AND && A->nbw <= dbs_meta::PUSH_LIST_MAX) ? o.bits_set : nullptr;
  P.nbw = A->nbw;
  P.xd = A->xd;  // PLUS_TIMES only: the staged x (OR_AND reads the masks alone)
  P.partial = A->partial;
  P.partial_bytes = (uint32_t)(A->nslots * DBS_MAX_SHARE * SLOT_WORDS * 4);
  P.slot_cls = 4;  // set per launch
  P.chunks = A->chunks;
  P.max_chunks = A->max_chunks;
  P.xlist = A->act_list;
  P.list_push = list_push ? 1 : 0;
  P.ctr = o.reg.ctr;
  P.force_path = (int32_t)A->opt[DBS_OPT_PATH];
  P.th3_num = A->opt[DBS_OPT_TH3_NUM];
  P.th3_den = A->opt[DBS_OPT_TH3_DEN];
  P.local_cutoff = (int32_t)A->opt[DBS_OPT_LOCAL_PUSH_CUTOFF];
  P.y = y;
  // one wave per group of pull segments (PULL_U_OR or PULL_U_PLUS of them), capped at the resident grid
  // PLUS_TIMES: several segments per wave step only when there are enough
  // for every resident wave (about 8 per SIMD) to get several steps
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 256;
    return n;
  }();
  const int64_t fw = A->opt[DBS_OPT_PULL_WIDTH];
  P.plus_u = fw == 1 ? 1
             : fw == 4 ? PULL_U_PLUS_WIDE
                       : (A->nseg >= (int64_t)PULL_U_PLUS_WIDE * 32 * cus * 4 ? PULL_U_PLUS_WIDE : 1);
  const int share = (int)A->opt[DBS_OPT_PULL_SHARE];
  const int pu = sr == DBS_PLUS_TIMES ? P.plus_u : A->vk == VK_PAT ? 1 : PULL_U_OR;
  const int64_t pull_waves = (P.nseg + pu - 1) / pu;
  const int64_t waves = pull_waves > A->max_chunks ? pull_waves : A->max_chunks;
  const int vk = A->vk;
  if (sr == DBS_OR_AND) {
    if (vk == VK_F32) launch_spmspv<VK_F32, DBS_OR_AND>(P, waves, 0, s, c0, c1);
    else if (vk == VK_BF16) launch_spmspv<VK_BF16, DBS_OR_AND>(P, waves, 0, s, c0, c1);
    else launch_spmspv<VK_PAT, DBS_OR_AND>(P, waves, 0, s, c0, c1);
  } else {
    const bool wide = P.plus_u == PULL_U_PLUS_WIDE;
    // the parts (waves sharing a segment) are fixed before the launch: the
    // same rule as launch_spmspv's, so that the finalize is known here
    int parts = 1;
    if (!wide && P.nseg > 0) {
      parts = share;
      if (!parts) {
        static const unsigned res1_f = dbs_resident_groups(k_spmspv<VK_F32, DBS_PLUS_TIMES, 1>, KT);
        static const unsigned res1_b = dbs_resident_groups(k_spmspv<VK_BF16, DBS_PLUS_TIMES, 1>, KT);
        const int64_t rw = (int64_t)(vk == VK_F32 ? res1_f : res1_b) * (KT / DBS_WAVE);
        const int64_t pp = (rw + P.nseg - 1) / P.nseg;
        parts = pp >= PLUS_MAX_PARTS ? PLUS_MAX_PARTS : pp >= 2 ? 2 : 1;
      }
    }
    // a sparse x has N_nzblk <= nnz_x (whatever its order), so a call that
    // must push is known here: it needs no finalize launch
    const int64_t fp = A->opt[DBS_OPT_PATH];
    const bool must_push =
        fp == 1 || (!dense && fp == 0 && (int64_t)nnz_x * A->opt[DBS_OPT_TH3_DEN] <
                                             (int64_t)A->nb * A->opt[DBS_OPT_TH3_NUM]);
    // the list is sorted by segment count: its first fin_cls[c] entries are
    // those of class c or above, the ones that took slots
    const int64_t nfin_used = A->nfin > 0 ? A->fin_cls[seg_slot_class(parts)] : 0;
    const bool fin = nfin_used > 0 && !must_push;
    // with a finalize, the call's compute time runs from the pull's start to
    // the finalize's end
    hipEvent_t pe1 = fin ? nullptr : c1;
    int used = 0;
    if (vk == VK_F32) {
      if (wide) used = launch_spmspv<VK_F32, DBS_PLUS_TIMES, PULL_U_PLUS_WIDE>(P, waves, parts, s, c0, pe1);
      else used = launch_spmspv<VK_F32, DBS_PLUS_TIMES, 1>(P, waves, parts, s, c0, pe1);
    } else {
      if (wide) used = launch_spmspv<VK_BF16, DBS_PLUS_TIMES, PULL_U_PLUS_WIDE>(P, waves, parts, s, c0, pe1);
      else used = launch_spmspv<VK_BF16, DBS_PLUS_TIMES, 1>(P, waves, parts, s, c0, pe1);
    }
    SPMV_TRY(hipGetLastError());
    if (used != parts) return DBS_ERR_DEVICE;  // cannot happen: both follow the same rule
    if (fin) {
      // entries of more than 256 slots get a workgroup each, the others a wave
      const int64_t nbig = A->fin_big[parts == 4 ? 2 : parts == 2 ? 1 : 0] < nfin_used
                               ? A->fin_big[parts == 4 ? 2 : parts == 2 ? 1 : 0]
                               : nfin_used;
      const int64_t g = nbig + (nfin_used - nbig + 15) / 16;
      launch_k(k_plus_finalize, dim3((unsigned)g), dim3(1024), s, nullptr, c1, (const uint32_t *)A->fin, nfin_used,
               nbig, (const float *)A->partial, (int32_t)parts, A->epoch, (const uint32_t *)o.reg.ctr, A->nb,
               (int32_t)A->opt[DBS_OPT_PATH], A->opt[DBS_OPT_TH3_NUM], A->opt[DBS_OPT_TH3_DEN], (float *)y, A->m);
    }
  }
  SPMV_TRY(hipGetLastError());
  A->cbuf ^= 1;
  A->last_stream = s;
  A->st.last_path = -2;  // resolved from the device counters by dbs_get_stats
  return DBS_OK;
}
