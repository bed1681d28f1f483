// Boolean pull over a pattern matrix (section 3.3 of "DB-SpMSpV: Dual-View
// Blocked Sparse Matrix-Sparse Vector Multiplication for Dynamic GPU
// Workloads"), shared by the OR-AND SpMSpV and the BFS level step.  The
// caller's policy says which rows of a row block are still wanted, gives the
// blk_x_mask of a column block and writes out the found rows.  Found rows
// are collected in LDS (row block, rows) and written out 48 to 64 row blocks
// at a time: this GPU counts stores and loads on one counter, and a store in
// flight makes the next wait for a load wait for every load in flight, so a
// store per segment would undo the pipelining.
#pragma once

#include "tile_kernels.h"

typedef __attribute__((address_space(4))) const uint32_t cu32_t;  // read-only: scalar loads

// the arrays the pull reads
struct PatSrc {
  const uint32_t *t_cb;     // value matrices (pat_issue)
  const uint64_t *t_meta;   // value matrices (pat_issue)
  const uint32_t *segs;  // padded with 16 zeroed descriptors
  int64_t nseg;
  brsrc_t pay;  // payload and its zeroed slack
  brsrc_t own;  // per payload word of a COO tile: the tile's rank in its segment (below)
  // Pattern matrices: the column-block word of every tile (column block, row
  // block within the segment, and with CBX_SINGLE a tile of one entry with
  // that entry), and the metadata of the other tiles ("ranked" tiles),
  // consecutive per segment in tile order: a ranked tile's rank is its index
  // among its segment's ranked tiles.  Matrices of more than CBX_MAX_NB
  // column blocks mark no tile single: every tile is ranked, and this
  // metadata is t_meta itself.
  const uint32_t *t_cbx = nullptr;
  uint32_t cbm = ~0u;               // column block of a word
  uint32_t sbit = 0u;               // CBX_SINGLE, or 0
  uint32_t rish = CBX_RI_SHIFT_WIDE;  // row block within the segment: (word >> rish) & 15
  const uint64_t *meta2 = nullptr;
  const uint2 *m2seg = nullptr;     // per segment: its first ranked tile in meta2, and their count
};

template <int U>
struct PatRound {
  uint4 seg[U];
  uint32_t n[U], cb[U], need[U];
  uint64_t meta[U];
};

// Descriptors of the U segments from s0 (scalar loads; `live` false reads
// the current ones again and marks them empty), then their column blocks and,
// EAGER, metadata through buffer ranges cut to each segment; a segment whose
// rows are all found already reads nothing.  Every load is issued
// unconditionally (idle lanes read out of range, which costs nothing): a load
// under a branch makes the compiler wait for every outstanding load, which
// would undo the pipelining below.
template <int U, bool EAGER, class Pol>
DBS_DEV void pat_issue(const PatSrc &S, const Pol &pol, int64_t s0, bool live, uint32_t l4, uint32_t l8,
                       PatRound<U> &r) {
  const cu32_t *q = (const cu32_t *)S.segs + 4 * s0;
#pragma unroll
  for (int u = 0; u < U; ++u) r.seg[u] = make_uint4(q[4 * u], q[4 * u + 1], q[4 * u + 2], q[4 * u + 3]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    r.need[u] = pol.need(r.seg[u].x & SEG_RB_MASK);
    r.n[u] = (live & (s0 + u < S.nseg) & (r.need[u] != 0u)) ? r.seg[u].z - r.seg[u].y : 0u;
    const brsrc_t rcb = make_rsrc(S.t_cb + r.seg[u].y, (uint64_t)r.n[u] * 4u);
    r.cb[u] = __builtin_amdgcn_raw_buffer_load_b32(rcb, l4, 0, 0);
    if constexpr (EAGER) r.meta[u] = bld64(make_rsrc(S.t_meta + r.seg[u].y, (uint64_t)r.n[u] * 8u), l8);
    else r.meta[u] = 0ull;
  }
}

// Pattern matrices (the graph workloads), pull.  A wave takes one segment of
// up to 64*K tiles per step (K slices of 64 consecutive tiles, lane i holding
// tile 64k+i of slice k), software-pipelined: the next segment's column-block
// words and, when most vector blocks are active, its ranked tiles' metadata
// are in flight while the current one waits for its masks and words.  Both
// come through buffer ranges cut to the segment, so lanes past its end read 0
// without any address arithmetic.  A tile of one entry is decoded from its
// word; the ranked tiles are decoded in rank order: COO tiles of up to four
// entries from their metadata word, the coordinate words of the other COO
// tiles (consecutive in the COO section) as one run spread over the lanes
// (word j by lane j) with each word's owner rank (a byte per word, recorded
// at build), whose mask the lane reads from LDS, and the rare larger tiles
// (Dense, ForceCSR, ForceCSC, patched CSR: all keep the 16 row masks for
// pattern matrices) per lane.  The work per segment that does not grow with
// its tiles (descriptor, ballots, word setup, wave OR, writeback) is a large
// part of this pull's cost, hence segments of up to 256 tiles.
template <int K>
struct PatSeg {  // stage A: descriptor, column-block words, EAGER the ranked tiles' metadata (n == 0: no segment)
  uint32_t rb, t0, n, nrb;  // first row block, first tile, tiles, row blocks (uniform)
  uint32_t m2b, n2;         // first ranked tile in meta2, ranked tiles (uniform)
  uint32_t needl;           // lane j < nrb: rows wanted in row block rb + j
  uint32_t cb[K];           // column-block words, lane i of slice k: tile 64k+i
  uint64_t meta[K];         // metadata, lane i of slice k: ranked tile 64k+i
};

template <int K>
struct PatMasks {  // stage B: masks, and (EAGER) the first chunk of coordinate words and their owners
  uint32_t m[K];  // lane i of slice k: mask of tile 64k+i
  int tf, tl;     // first and last rank of a COO tile (not inline) whose words are read (uniform; tl < 0: none)
  uint32_t base, nwords, word, own;
};

// Found rows of a wave not yet written: entry i is row block rb[i], rows f[i]
// (LDS), n entries (uniform).
constexpr int PAT_FOUND_CAP = 64;
struct FoundBuf {
  uint32_t *rb, *f;
  int n;
};

// The descriptors of a wave's next 64 segments (lane j: segment next +
// j*stride) and the ballot of those with wanted rows.  Read 64 at a time, a
// descriptor costs no round trip of its own, and segments with nothing to do
// (all rows found) are skipped without a step.  A descriptor is (first row
// block, first tile, end tile, row blocks): several consecutive short row
// blocks may share one segment (at most PAT_MAX_RB).
constexpr int PAT_MAX_RB = DBS_PAT_MAX_RB;

struct SegWin {
  uint32_t rb, t0, m2b;  // per lane: first row block, first tile, first entry in meta2
  uint32_t pk;           // per lane: tiles | row blocks << 9 | entries in meta2 << 14
  uint64_t live;         // lanes whose segment has tiles and wanted rows
  int64_t next;          // first segment of the next window
};

template <class Pol>
DBS_DEV void win_fill(const PatSrc &S, const Pol &pol, int64_t stride, int lane, SegWin &w) {
  const int64_t s = w.next + (int64_t)lane * stride;
  const bool in = s < S.nseg;
  const uint4 d = ((const uint4 *)S.segs)[in ? s : 0];  // unconditional: no branch around the load
  const uint2 e = S.m2seg[in ? s : 0];
  const uint32_t nrb = d.w > 1u ? d.w : 1u;
  w.rb = d.x & ~SEG_SPLIT;
  w.t0 = d.y;
  w.m2b = e.x;
  w.pk = (d.z - d.y) | (nrb << 9) | (e.y << 14);  // at most 256 tiles, 16 row blocks
  uint32_t need = 0u;
#pragma unroll
  for (int j = 0; j < PAT_MAX_RB; ++j) {
    const bool jin = (uint32_t)j < nrb;
    need |= pol.need_v(w.rb + j, in & jin) & (0u - (uint32_t)jin);
  }
  w.live = __ballot(in & (need != 0u) & (d.z > d.y));
  w.next += 64 * stride;
}

struct SegDesc {
  uint32_t rb, t0, n, nrb, m2b, n2;  // uniform
};

// next segment with work, false once the wave's share is done (uniform)
template <class Pol>
DBS_DEV bool win_next(const PatSrc &S, const Pol &pol, int64_t stride, int lane, SegWin &w, SegDesc &d) {
  while (w.live == 0ull) {
    if (w.next >= S.nseg) return false;
    win_fill(S, pol, stride, lane, w);
  }
  const int j = __ffsll((unsigned long long)w.live) - 1;
  w.live &= w.live - 1ull;
  d.rb = (uint32_t)__builtin_amdgcn_readlane((int)w.rb, j);
  d.t0 = (uint32_t)__builtin_amdgcn_readlane((int)w.t0, j);
  d.m2b = (uint32_t)__builtin_amdgcn_readlane((int)w.m2b, j);
  const uint32_t pk = (uint32_t)__builtin_amdgcn_readlane((int)w.pk, j);
  d.n = pk & 511u;
  d.nrb = (pk >> 9) & 31u;
  d.n2 = pk >> 14;
  return true;
}

template <int K, bool EAGER, class Pol>
DBS_DEV void patk_issue(const PatSrc &S, const Pol &pol, int64_t stride, int lane, SegWin &w, uint32_t l4,
                        uint32_t l8, PatSeg<K> &r) {
  SegDesc d{0u, 0u, 0u, 1u, 0u, 0u};
  const bool any = win_next(S, pol, stride, lane, w, d);
  r.rb = d.rb;
  r.t0 = d.t0;
  r.nrb = d.nrb;
  r.n = any ? d.n : 0u;
  r.m2b = d.m2b;
  r.n2 = any ? d.n2 : 0u;
  const brsrc_t rcb = make_rsrc(S.t_cbx + d.t0, (uint64_t)r.n * 4u);
  const brsrc_t rmt = make_rsrc(S.meta2 + d.m2b, (uint64_t)r.n2 * 8u);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    r.cb[k] = __builtin_amdgcn_raw_buffer_load_b32(rcb, l4 + 256u * k, 0, 0);
    if constexpr (EAGER) r.meta[k] = bld64(rmt, l8 + 512u * k);
    else r.meta[k] = 0ull;
  }
  const bool mine = any & ((uint32_t)lane < d.nrb);
  r.needl = pol.need_v(d.rb + (uint32_t)lane, mine);
}

// lane l's value of slice k (both wave-uniform), read from every slice so
// that no array is indexed at run time (the compiler would place it in
// scratch memory)
template <int K>
DBS_DEV uint32_t slice_lane(const uint32_t (&v)[K], int k, int l) {
  uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v[0], l);
#pragma unroll
  for (int i = 1; i < K; ++i) {
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v[i], l);
    r = k == i ? c : r;
  }
  return r;
}

// the non-inline COO tiles whose words are read (every such ranked tile when
// EAGER: an inactive tile's words meet a zero mask; else those with a
// nonzero mask in s_tm), the run of their words, and its first chunk with
// the words' owners (ranks)
template <int K, bool EAGER>
DBS_DEV void pat_words(const PatSrc &S, const uint64_t (&meta)[K], uint32_t n2, const uint32_t *s_tm,
                       PatMasks<K> &b, int lane, uint32_t l4) {
  uint32_t lo[K], hi[K];  // halves of the metadata words
  b.tf = 1 << 20;
  b.tl = -1;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    lo[k] = (uint32_t)meta[k];
    hi[k] = (uint32_t)(meta[k] >> 32);
    const uint32_t r = 64u * k + (uint32_t)lane;
    const bool live = EAGER ? (r < n2) : ((r < n2) && ((s_tm[r] & 0xFFFFu) != 0u));
    const uint64_t nb = __ballot(live & (meta_kind(hi[k]) == DBS_TILE_COO));  // COO, not inline
    if (nb != 0ull) {
      const int f = 64 * k + __ffsll((unsigned long long)nb) - 1, l = 64 * k + 63 - __clzll((long long)nb);
      b.tf = f < b.tf ? f : b.tf;
      b.tl = l > b.tl ? l : b.tl;
    }
  }
  b.base = 0u;
  b.nwords = 0u;
  if (b.tl >= 0) {
    // the run starts at the first tile's words and ends after the last one's
    b.base = slice_lane<K>(lo, b.tf >> 6, b.tf & 63);
    const uint32_t lvp = slice_lane<K>(lo, b.tl >> 6, b.tl & 63);
    const uint32_t lhi = slice_lane<K>(hi, b.tl >> 6, b.tl & 63);
    b.nwords = (lvp + coo_val_off(((lhi >> 8) & 0xFFu) + 1u) - b.base) >> 2;
  }
  const bool in = (uint32_t)lane < b.nwords;
  b.word = bld32(S.pay, in ? b.base + l4 : OOB_OFF);
  b.own = __builtin_amdgcn_raw_buffer_load_b8(S.own, in ? (b.base >> 2) + (uint32_t)lane : OOB_OFF, 0, 0);
}

// rank of the ranked tile of word w in lane `lane` of slice k: in the word
// when it can mark single tiles, else the tile's index in the segment
DBS_DEV uint32_t rank_of(const PatSrc &S, uint32_t w, int k, int lane) {
  return S.sbit ? w >> CBX_RC_SHIFT : 64u * k + (uint32_t)lane;
}

// A segment is finished in two parts around the next segments' loads.
// pat_pre, in tile order: a tile of one entry is decoded from its word; every
// other tile writes its mask (| its row block within the segment << 16) to
// s_tm at its rank; without EAGER, the ranked tiles with a nonzero mask then
// read their metadata.  pat_post, in rank order (lane i of slice k: ranked
// tile 64k+i): inline COO tiles from the metadata word; the coordinate words
// of the other COO tiles, spread over the lanes, each finding its tile's mask
// at s_tm[owner]; the 16 row masks of the larger tiles, per lane.  MULTI: the
// segment holds several row blocks, and each found row goes to its row block
// through an LDS OR (s_f, one word per row block).  SKIP: slices without an
// active tile skip their decode (worth its test when few vector blocks are
// active).  `f` keeps the found rows of a one-row-block segment in between.
template <int K, bool MULTI, bool SKIP, bool EAGER, class Pol>
DBS_DEV void pat_pre(const PatSrc &S, const Pol &pol, PatSeg<K> &a, const PatMasks<K> &b, int lane, uint32_t l8,
                     uint32_t *s_tm, uint32_t *s_f, uint32_t &f) {
  const uint32_t n = a.n;  // uniform
  f = 0u;
  if constexpr (MULTI) {
    if (lane < PAT_MAX_RB) s_f[lane] = 0u;
    __syncwarp();
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (64u * k >= n) break;  // uniform
    const uint32_t w = a.cb[k];
    const bool in = 64u * k + (uint32_t)lane < n;
    const bool single = (w & S.sbit) != 0u;  // lanes past the end read 0
    const uint32_t ri = (w >> S.rish) & 15u;
    if (in & !single) s_tm[rank_of(S, w, k, lane)] = b.m[k] | (ri << 16);
    const uint32_t m = b.m[k];
    const bool hit = single & (m != 0u);
    if (SKIP && __ballot(hit) == 0ull) continue;  // uniform
    const uint32_t rc = w >> CBX_RC_SHIFT;
    const uint32_t x = hit ? ((m >> (rc & 15u)) & 1u) << (rc >> 4) : 0u;
    if constexpr (MULTI) {
      if (x) atomicOr(&s_f[ri], x);
    } else {
      f |= x;
    }
  }
  if constexpr (!EAGER) {
    __syncwarp();
    // metadata of the ranked tiles with a nonzero mask
    const brsrc_t rmt = make_rsrc(S.meta2 + a.m2b, (uint64_t)a.n2 * 8u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t r = 64u * k + (uint32_t)lane;
      const bool act = (r < a.n2) && ((s_tm[r] & 0xFFFFu) != 0u);
      a.meta[k] = bld64(rmt, act ? l8 + 512u * k : OOB_OFF);
    }
  }
}

template <int K, bool MULTI, bool SKIP, bool EAGER, class Pol>
DBS_DEV void pat_post(const PatSrc &S, const Pol &pol, const PatSeg<K> &a, const PatMasks<K> &b0, int lane,
                      uint32_t l4, uint32_t *s_tm, uint32_t *s_f, FoundBuf &fb, uint32_t f) {
  const uint32_t n2 = a.n2;  // uniform
  __syncwarp();
  // rank order: lane i of slice k reads mask | row block << 16 of ranked tile 64k+i
  auto tm_of = [&](int k) {
    const uint32_t r = 64u * k + (uint32_t)lane;
    return r < n2 ? s_tm[r] : 0u;
  };
  PatMasks<K> bl;
  if constexpr (!EAGER) pat_words<K, false>(S, a.meta, n2, s_tm, bl, lane, l4);
  const PatMasks<K> &b = EAGER ? b0 : bl;
  auto add = [&](uint32_t ri, uint32_t x) {
    if constexpr (MULTI) {
      if (x) atomicOr(&s_f[ri], x);
    } else {
      f |= x;
    }
  };
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (64u * k >= n2) break;  // uniform
    const uint32_t tm = tm_of(k), m = tm & 0xFFFFu;
    if (SKIP && __ballot(m != 0u) == 0ull) continue;  // uniform
    const uint64_t meta = a.meta[k];
    // COO tiles with at most four entries: the coordinates are in the metadata
    // word (a zero mask decodes to nothing)
    add(tm >> 16, meta_kind((uint32_t)(meta >> 32)) == (DBS_TILE_COO | 8u) ? coo_or4((uint32_t)meta, m) : 0u);
  }
  if (b.tl >= 0) {
    for (uint32_t j0 = 0; j0 < b.nwords; j0 += 64u) {
      const uint32_t j = j0 + (uint32_t)lane;
      const bool in = j < b.nwords;
      const uint32_t wd = j0 == 0u ? b.word : bld32(S.pay, in ? b.base + 4u * j : OOB_OFF);
      const uint32_t ow =
          j0 == 0u ? b.own : __builtin_amdgcn_raw_buffer_load_b8(S.own, in ? (b.base >> 2) + j : OOB_OFF, 0, 0);
      const uint32_t tm = s_tm[ow & 255u];
      const uint32_t x = in ? coo_or4(wd, tm & 0xFFFFu) : 0u;
      if constexpr (MULTI) {
        if (x) atomicOr(&s_f[tm >> 16], x);
      } else {
        f |= x;
      }
    }
  }
  // larger tiles: 16 row masks each
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (64u * k >= n2) break;  // uniform
    const uint32_t tm = tm_of(k), m = tm & 0xFFFFu;
    const bool big = (m != 0u) & (meta_type(a.meta[k]) != DBS_TILE_COO);
    if (__ballot(big) != 0ull) {
      const uint32_t o = big ? (uint32_t)meta_vp(a.meta[k]) : OOB_OFF;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(S.pay, o, 0, 0);
      const auto y = __builtin_amdgcn_raw_buffer_load_b128(S.pay, big ? o + 16u : OOB_OFF, 0, 0);
      const uint32_t rm[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
      uint32_t g = 0;
      // row r found iff its 16-bit row mask meets the active columns; the
      // 0/1 bit comes from a carry ((x + 0xFFFF) >> 16), so no per-row
      // constant is held in a register
#pragma unroll
      for (int r = 0; r < 16; ++r) g |= ((((rm[r >> 1] >> (16 * (r & 1))) & m) + 0xFFFFu) >> 16) << r;
      add(tm >> 16, g);
    }
  }
  if constexpr (MULTI) {
    __syncwarp();
    const uint32_t fl = ((uint32_t)lane < a.nrb) ? s_f[lane] & a.needl : 0u;
    const uint64_t any = __ballot(fl != 0u);
    if (fl != 0u) {
      // entries of the lanes below this one (mbcnt: no 64-bit lane mask kept)
      const int pos = fb.n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(any >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)any, 0u));
      fb.rb[pos] = a.rb + (uint32_t)lane;
      fb.f[pos] = fl;
    }
    fb.n += __popcll(any);
    __syncwarp();
  } else {
    f = wave_or(f) & (uint32_t)__builtin_amdgcn_readlane((int)a.needl, 0);
    if (f != 0u) {  // uniform
      if (lane == 0) {
        fb.rb[fb.n] = a.rb;
        fb.f[fb.n] = f;
      }
      fb.n += 1;
    }
    __syncwarp();
  }
}

// write out the collected found rows (the policy's flush) once the buffer
// may not take another segment's row blocks
template <class Pol>
DBS_DEV void pat_flush(const Pol &pol, FoundBuf &fb, int lane, bool all) {
  if (fb.n > (all ? 0 : PAT_FOUND_CAP - PAT_MAX_RB)) {  // uniform
    __syncwarp();
    pol.flush(fb.rb, fb.f, fb.n, lane);
    __syncwarp();
    fb.n = 0;
  }
}

// One wave's share: segments s0, s0 + stride, ... that have work.  Three
// steps are in flight: while segment i is finished, segment i+1 has its
// masks (and, EAGER, its coordinate words) and segment i+2 its column-block
// words and (EAGER) metadata in flight.  Loads are issued in that order, so a
// wait for segment i's data never waits for the loads of the later segments
// (a new window of descriptors, once per 64 segments, does wait).  Without
// EAGER, segment i's metadata (of its active ranked tiles) is read at the
// start of its step, before the later segments' loads, and its coordinate
// words after them; a deeper pipeline that reads them one and two steps ahead
// ran slower (more registers and moves per step, and this pull is bound by
// the vector-memory instructions it issues, not by waits).
template <int K, bool EAGER, bool MULTI, class Pol>
DBS_DEV void pat_step(const PatSrc &S, const Pol &pol, int64_t stride, int lane, uint32_t l4, uint32_t l8,
                      SegWin &w, PatSeg<K> &a0, PatSeg<K> &a1, PatSeg<K> &a2, PatMasks<K> &b0, PatMasks<K> &b1,
                      uint32_t *s_tm, uint32_t *s_f, FoundBuf &fb) {
  uint32_t f;
  pat_pre<K, MULTI, !EAGER, EAGER>(S, pol, a0, b0, lane, l8, s_tm, s_f, f);
  patk_issue<K, EAGER>(S, pol, stride, lane, w, l4, l8, a2);
#pragma unroll
  for (int k = 0; k < K; ++k) b1.m[k] = pol.mask(a1.cb[k] & S.cbm, 64u * k + (uint32_t)lane < a1.n);
  if constexpr (EAGER) pat_words<K, true>(S, a1.meta, a1.n2, s_tm, b1, lane, l4);
  pat_post<K, MULTI, !EAGER, EAGER>(S, pol, a0, b0, lane, l4, s_tm, s_f, fb, f);
}

template <int K, bool EAGER, class Pol>
DBS_DEV void pattern_pull_wave(const PatSrc &S, const Pol &pol, int64_t s0, int64_t stride, int lane,
                               uint32_t *s_tm, uint32_t *s_f, FoundBuf &fb) {
  if (s0 >= S.nseg) return;
  const uint32_t l4 = (uint32_t)lane * 4u, l8 = (uint32_t)lane * 8u;
  SegWin w;
  w.next = s0;
  w.live = 0ull;
  PatSeg<K> a0, a1, a2;
  PatMasks<K> b0, b1;
  patk_issue<K, EAGER>(S, pol, stride, lane, w, l4, l8, a0);
  patk_issue<K, EAGER>(S, pol, stride, lane, w, l4, l8, a1);
#pragma unroll
  for (int k = 0; k < K; ++k) b0.m[k] = pol.mask(a0.cb[k] & S.cbm, 64u * k + (uint32_t)lane < a0.n);
  if constexpr (EAGER) pat_words<K, true>(S, a0.meta, a0.n2, s_tm, b0, lane, l4);
  while (a0.n != 0u) {
    if (a0.nrb > 1u)  // uniform
      pat_step<K, EAGER, true>(S, pol, stride, lane, l4, l8, w, a0, a1, a2, b0, b1, s_tm, s_f, fb);
    else pat_step<K, EAGER, false>(S, pol, stride, lane, l4, l8, w, a0, a1, a2, b0, b1, s_tm, s_f, fb);
    pat_flush(pol, fb, lane, false);
    a0 = a1;
    a1 = a2;
    b0 = b1;
  }
}

// ---------------------------------------------------------------------------
// Very sparse x (a few percent of the vector blocks active, active-block
// bits in LDS).  A segment then holds a handful of active tiles, and the
// per-segment finish above (ballots, decode and writeback of every slice)
// is mostly idle work.  Here a wave only tests each tile's column block
// against the active-block bits and queues the active tiles in an LDS
// ring; every 64 queued tiles are finished together, one tile per lane: its
// mask word and (a ranked tile) its metadata, then its coordinates (a single
// entry from its word, inline ones from the metadata word, its coordinate
// words, or the 16 row masks of a larger tile), and the found rows go to the
// wave's found-row buffer (a tile's row block is its segment's first plus
// the offset in its word).  The words of the next two segments are in
// flight while one is tested.
// ---------------------------------------------------------------------------
constexpr uint32_t PAT_Q = 128;  // ring entries: 64 queued at most before a batch, plus one slice

template <int K>
struct ScanSeg {
  uint32_t rb, t0, n, m2b;  // first row block, first tile, tiles, first ranked tile (uniform; n == 0: none)
  uint32_t cb[K];           // column-block words
};

template <int K, class Pol>
DBS_DEV void scan_issue(const PatSrc &S, const Pol &pol, int64_t stride, int lane, SegWin &w, uint32_t l4,
                        ScanSeg<K> &r) {
  SegDesc d{0u, 0u, 0u, 1u, 0u, 0u};
  const bool any = win_next(S, pol, stride, lane, w, d);
  r.rb = d.rb;
  r.t0 = d.t0;
  r.n = any ? d.n : 0u;
  r.m2b = d.m2b;
  const brsrc_t rcb = make_rsrc(S.t_cbx + d.t0, (uint64_t)r.n * 4u);
#pragma unroll
  for (int k = 0; k < K; ++k) r.cb[k] = __builtin_amdgcn_raw_buffer_load_b32(rcb, l4 + 256u * k, 0, 0);
}

// A batch of queued tiles (n <= 64, lane j holding the j-th): its mask
// words and the metadata of its ranked tiles are loaded when it leaves the
// ring, and it is finished when the next batch leaves (or at the end), so
// its loads are in flight while the wave scans on.  A queue entry is (the
// tile's entry in meta2 if it is ranked, its column-block word, its
// segment's first row block).
struct SpBatch {
  uint32_t n;  // tiles (uniform; 0: none)
  uint32_t rb0, cbx, w;
  uint64_t meta;
};

template <class Pol>
DBS_DEV void sp_issue(const PatSrc &S, const Pol &pol, const uint32_t *q, uint32_t head, uint32_t n, int lane,
                      SpBatch &b) {
  const bool in = (uint32_t)lane < n;
  const uint32_t i = (head + (uint32_t)lane) & (PAT_Q - 1u);
  const uint32_t e = q[i];
  b.n = n;
  b.cbx = q[PAT_Q + i];
  b.rb0 = q[2 * PAT_Q + i];
  b.w = pol.mask_raw(b.cbx & S.cbm, in);
  // idle lanes and single tiles repeat lane 0's entry (an entry of meta2, or
  // its first word, which exists: meta2 is allocated with one word at least)
  b.meta = S.meta2[(in & ((b.cbx & S.sbit) == 0u)) ? e : q[head & (PAT_Q - 1u)]];
}

// found rows of a batch's tiles: a tile of one entry from its column-block
// word; inline COO tiles from the metadata word; the coordinate words of the
// other COO tiles are read 16 entries per 16-byte load, one load per round
// (the words past a tile's end are not decoded), the 16 row masks of the
// larger tiles in two loads.  The rows found go to the wave's found-row buffer.
template <class Pol>
DBS_DEV void sp_finish(const PatSrc &S, const Pol &pol, const SpBatch &b, int lane, FoundBuf &fb, int cap) {
  const bool in = (uint32_t)lane < b.n;
  const uint32_t m = in ? pol.mask_of(b.w, b.cbx & S.cbm) : 0u;
  const bool single = (b.cbx & S.sbit) != 0u;
  const uint32_t lo = (uint32_t)b.meta, hi = (uint32_t)(b.meta >> 32);
  const uint32_t kind = meta_kind(hi);
  const bool live = (m != 0u) & !single;
  const uint32_t rc = b.cbx >> CBX_RC_SHIFT;
  uint32_t f = single ? ((m >> (rc & 15u)) & 1u) << (rc >> 4) : 0u;
  f |= (live & (kind == (DBS_TILE_COO | 8u))) ? coo_or4(lo, m) : 0u;
  const uint32_t nw = (live & (kind == DBS_TILE_COO)) ? ((hi >> 8) & 0xFFu) / 4u + 1u : 0u;
  const bool big = live & (meta_type(b.meta) != DBS_TILE_COO);
  const uint32_t nq = wave_max((nw + 3u) >> 2);  // uniform
  for (uint32_t jq = 0; jq < nq; ++jq) {  // most tiles have at most 16 entries: one round
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(S.pay, 4u * jq < nw ? lo + 16u * jq : OOB_OFF, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) f |= (4u * jq + (uint32_t)e < nw) ? coo_or4(v[e], m) : 0u;
  }
  if (__ballot(big) != 0ull) {  // uniform
    const uint32_t o = big ? lo : OOB_OFF;
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(S.pay, o, 0, 0);
    const auto y = __builtin_amdgcn_raw_buffer_load_b128(S.pay, big ? o + 16u : OOB_OFF, 0, 0);
    const uint32_t rm[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    uint32_t g = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) g |= ((((rm[r >> 1] >> (16 * (r & 1))) & m) + 0xFFFFu) >> 16) << r;
    f |= big ? g : 0u;
  }
  const uint64_t any = __ballot(f != 0u);
  if (f != 0u) {
    const int pos = fb.n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(any >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)any, 0u));
    fb.rb[pos] = b.rb0 + ((b.cbx >> S.rish) & 15u);
    fb.f[pos] = f;
  }
  fb.n += __popcll(any);
  if (fb.n > cap - 64) {  // uniform: no room for another batch
    __syncwarp();
    pol.flush_new(fb.rb, fb.f, fb.n, lane);
    __syncwarp();
    fb.n = 0;
  }
}

// LDS per wave of the very sparse pull: the ring (tile, column block, row
// block), and apart from it the found-row buffer (2 x SP_FOUND_CAP words).
// The found rows are not checked against the rows still wanted: the
// policy's flush_new does that.
constexpr int SP_FOUND_CAP = 128;
constexpr int SP_LDS_WORDS = 3 * (int)PAT_Q;
// with the active-block bits staged in an LDS array of PUSH_LIST_MAX words
// for a workgroup of `waves` waves, the bits may take this many words and
// leave room for the waves' found-row buffers after them
constexpr int sp_bits_max(int waves) { return dbs_meta::PUSH_LIST_MAX - waves * 2 * SP_FOUND_CAP; }

template <int K, class Pol>
DBS_DEV void pattern_pull_sparse(const PatSrc &S, const Pol &pol, int64_t s0, int64_t stride, int lane,
                                 uint32_t *q, uint32_t *found) {
  if (s0 >= S.nseg) return;
  const uint32_t l4 = (uint32_t)lane * 4u;
  FoundBuf fb{found, found + SP_FOUND_CAP, 0};
  SegWin w;
  w.next = s0;
  w.live = 0ull;
  ScanSeg<K> a0, a1, a2;
  scan_issue<K>(S, pol, stride, lane, w, l4, a0);
  scan_issue<K>(S, pol, stride, lane, w, l4, a1);
  SpBatch pb;
  pb.n = 0u;
  uint32_t head = 0u, qn = 0u;  // uniform
  while (a0.n != 0u) {
    scan_issue<K>(S, pol, stride, lane, w, l4, a2);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (64u * k >= a0.n) break;  // uniform
      const bool in = 64u * k + (uint32_t)lane < a0.n;
      const uint32_t cw = a0.cb[k];
      const bool act = in & pol.active(cw & S.cbm);
      const uint64_t bal = __ballot(act);
      if (bal != 0ull) {  // uniform
        const uint32_t pos =
            (head + qn + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))) &
            (PAT_Q - 1u);
        if (act) {
          q[pos] = a0.m2b + rank_of(S, cw, k, lane);  // unused for a single tile
          q[PAT_Q + pos] = cw;
          q[2 * PAT_Q + pos] = a0.rb;
        }
        qn += (uint32_t)__popcll(bal);
        if (qn >= 64u) {  // uniform
          __syncwarp();
          if (pb.n != 0u) sp_finish(S, pol, pb, lane, fb, SP_FOUND_CAP);
          sp_issue(S, pol, q, head, 64u, lane, pb);
          __syncwarp();
          head = (head + 64u) & (PAT_Q - 1u);
          qn -= 64u;
        }
      }
    }
    a0 = a1;
    a1 = a2;
  }
  __syncwarp();
  if (pb.n != 0u) sp_finish(S, pol, pb, lane, fb, SP_FOUND_CAP);
  if (qn != 0u) {
    sp_issue(S, pol, q, head, qn, lane, pb);
    sp_finish(S, pol, pb, lane, fb, SP_FOUND_CAP);
  }
  if (fb.n != 0) {
    __syncwarp();
    pol.flush_new(fb.rb, fb.f, fb.n, lane);
  }
}

constexpr int PAT_K = DBS_PAT_SEG_CAP / 64;  // slices of 64 tiles per pattern-pull segment

// LDS per wave: masks of a segment's tiles (64*K), found rows per row block,
// the found-row buffer (2 x PAT_FOUND_CAP); or the very sparse pull's ring
constexpr int PAT_LDS_WORDS = 64 * PAT_K + PAT_MAX_RB + 2 * PAT_FOUND_CAP;
static_assert(PAT_LDS_WORDS >= SP_LDS_WORDS, "the very sparse pull's ring takes the same LDS");

// LAZY_ONLY: the policy is only used with the metadata of the active tiles
// (no instantiation for `eager`)
template <bool LAZY_ONLY = false, class Pol>
DBS_DEV void pattern_pull(const PatSrc &S, const Pol &pol, int64_t s0, int64_t stride, bool eager, int lane,
                          uint32_t *s_lds) {
  uint32_t *s_tm = s_lds, *s_f = s_lds + 64 * PAT_K;
  FoundBuf fb{s_f + PAT_MAX_RB, s_f + PAT_MAX_RB + PAT_FOUND_CAP, 0};
  if (!LAZY_ONLY && eager) pattern_pull_wave<PAT_K, !LAZY_ONLY>(S, pol, s0, stride, lane, s_tm, s_f, fb);
  else pattern_pull_wave<PAT_K, false>(S, pol, s0, stride, lane, s_tm, s_f, fb);
  pat_flush(pol, fb, lane, true);
}
