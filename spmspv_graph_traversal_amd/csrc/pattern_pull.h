// Boolean pull over a pattern matrix (section 3.3 of "DB-SpMSpV: Dual-View
// Blocked Sparse Matrix-Sparse Vector Multiplication for Dynamic GPU
// Workloads"), shared by the OR-AND SpMSpV and the BFS level step.  The
// caller's policy says which rows of a row block are still wanted, gives the
// blk_x_mask of a column block and takes the found rows of each segment.
#pragma once

#include "tile_kernels.h"

typedef __attribute__((address_space(4))) const uint32_t cu32_t;  // read-only: scalar loads

// the arrays the pull reads
struct PatSrc {
  const uint32_t *t_cb;
  const uint64_t *t_meta;
  const uint32_t *segs;  // padded with 16 zeroed descriptors
  int64_t nseg;
  brsrc_t pay;  // payload and its zeroed slack
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
  for (int u = 0; u < U; ++u) r.seg[u] = make_uint4(q[4 * u], q[4 * u + 1], q[4 * u + 2], 0u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    r.need[u] = pol.need(r.seg[u].x & ~SEG_SPLIT);
    r.n[u] = (live & (s0 + u < S.nseg) & (r.need[u] != 0u)) ? r.seg[u].z - r.seg[u].y : 0u;
    const brsrc_t rcb = make_rsrc(S.t_cb + r.seg[u].y, (uint64_t)r.n[u] * 4u);
    r.cb[u] = __builtin_amdgcn_raw_buffer_load_b32(rcb, l4, 0, 0);
    if constexpr (EAGER) r.meta[u] = bld64(make_rsrc(S.t_meta + r.seg[u].y, (uint64_t)r.n[u] * 8u), l8);
    else r.meta[u] = 0ull;
  }
}

// Pattern matrices (the graph workloads), pull.  Per step a wave takes U
// segments and issues each load phase for all of them: segment descriptors
// (scalar loads), column blocks (and, when most vector blocks are active,
// metadata) through a buffer range cut to the segment, so lanes past its end
// read 0 without any address arithmetic; the blk_x_mask gather; metadata of
// the active tiles; then the coordinate words of the active COO tiles that do
// not fit in their metadata word.  Those tiles' payloads are consecutive in the
// COO section, so the segment reads them as one run of words spread over the
// lanes (word j by lane j), each lane finding the tile of its word by a wave
// max-scan of the tiles' first-word marks.  A segment thus costs two to five
// vector memory instructions whatever its size mix, and each instruction
// covers up to 64 tiles or words.  Larger tiles (Dense, ForceCSR, ForceCSC,
// patched CSR: all keep the 16 row masks for pattern matrices) are rare and
// take a separate step.
// One wave's share of the pull, software-pipelined over its steps: the
// descriptors, column blocks and metadata of step i+1 are in flight while
// step i waits for its masks and coordinate words.  EAGER (most vector
// blocks active): metadata comes with the column blocks and the coordinate
// words of every non-inline COO tile are read with the masks (an inactive
// tile's words meet a zero mask).  Otherwise metadata and words are read for
// the active tiles only, after their masks.
template <int U, bool EAGER, class Pol>
DBS_DEV void pattern_pull_wave(const PatSrc &S, const Pol &pol, int64_t s0, int64_t stride, int lane,
                               uint32_t *s_mark) {
  if (s0 >= S.nseg) return;
  const uint32_t l4 = (uint32_t)lane * 4u, l8 = (uint32_t)lane * 8u;
  PatRound<U> cur, nxt;
  pat_issue<U, EAGER>(S, pol, s0, true, l4, l8, cur);
  while (true) {
    uint32_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m[u] = pol.mask(cur.cb[u], (uint32_t)lane < cur.n[u]);
    }
    // coordinate words of the non-inline COO tiles: [base, base + 4 * nwords)
    uint32_t word[U], base[U], nwords[U];
    uint64_t nicb[U];
    auto issue_words = [&]() {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool live = EAGER ? ((uint32_t)lane < cur.n[u]) : (m[u] != 0u);
        const bool nic = live & (meta_type(cur.meta[u]) == DBS_TILE_COO) & !meta_inline(cur.meta[u]);
        nicb[u] = __ballot(nic);
        const int first = nicb[u] ? __ffsll((unsigned long long)nicb[u]) - 1 : 0;
        const int last = nicb[u] ? 63 - __clzll((long long)nicb[u]) : 0;
        const uint32_t vp = (uint32_t)meta_vp(cur.meta[u]);
        const uint32_t vend = vp + coo_val_off(meta_nnz(cur.meta[u]));
        base[u] = (uint32_t)__builtin_amdgcn_readlane((int)vp, first);
        nwords[u] = nicb[u] ? ((uint32_t)__builtin_amdgcn_readlane((int)vend, last) - base[u]) >> 2 : 0u;
        word[u] = bld32(S.pay, (uint32_t)lane < nwords[u] ? base[u] + l4 : OOB_OFF);
      }
    };
    const int64_t s1 = s0 + stride;
    const bool more = s1 < S.nseg;  // uniform
    if constexpr (EAGER) {
      issue_words();
      pat_issue<U, EAGER>(S, pol, more ? s1 : s0, more, l4, l8, nxt);
    } else {
      pat_issue<U, EAGER>(S, pol, more ? s1 : s0, more, l4, l8, nxt);
#pragma unroll
      for (int u = 0; u < U; ++u)
        cur.meta[u] = bld64(make_rsrc(S.t_meta + cur.seg[u].y, (uint64_t)cur.n[u] * 8u), m[u] != 0u ? l8 : OOB_OFF);
      issue_words();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= S.nseg) break;
      const uint64_t meta = cur.meta[u];
      const uint32_t type = meta_type(meta);
      // COO tiles with at most four entries: the coordinates are in the metadata word
      uint32_t f = ((m[u] != 0u) & (type == DBS_TILE_COO) & meta_inline(meta)) ? coo_or4((uint32_t)meta, m[u]) : 0u;
      if (nicb[u] != 0ull) {
        const bool nic = (nicb[u] >> lane) & 1ull;
        // words [slot, send) of this lane's tile; the end test leaves out words
        // of tiles that are not marked
        const uint32_t slot = ((uint32_t)meta_vp(meta) - base[u]) >> 2;
        const uint32_t send = slot + (coo_val_off(meta_nnz(meta)) >> 2);
        uint32_t carry = 0u;
        for (uint32_t j0 = 0; j0 < nwords[u]; j0 += 64u) {
          // lanes talk through LDS: each step is fenced at wave scope, or the
          // compiler may hand a lane back its own earlier store
          __syncwarp();
          s_mark[lane] = 0u;
          __syncwarp();
          if (nic & (slot >= j0) & (slot < j0 + 64u)) s_mark[slot - j0] = (uint32_t)lane + 1u;
          __syncwarp();
          uint32_t own = wave_incl_max(s_mark[lane]);
          own = own > carry ? own : carry;
          carry = (uint32_t)__builtin_amdgcn_readlane((int)own, 63);  // owner of the next chunk's first word
          const uint32_t mw = (uint32_t)__shfl((int)m[u], (int)own - 1);
          const uint32_t oend = (uint32_t)__shfl((int)send, (int)own - 1);
          const uint32_t j = j0 + (uint32_t)lane;
          const uint32_t wd = j0 == 0u ? word[u] : bld32(S.pay, j < nwords[u] ? base[u] + 4u * j : OOB_OFF);
          f |= ((j < nwords[u]) & (j < oend)) ? coo_or4(wd, mw) : 0u;
        }
      }
      // larger tiles: 16 row masks each
      const bool big = (m[u] != 0u) & (type != DBS_TILE_COO);
      if (__ballot(big) != 0ull) {
        const uint32_t vp = big ? (uint32_t)meta_vp(meta) : OOB_OFF;
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(S.pay, vp, 0, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(S.pay, big ? vp + 16u : OOB_OFF, 0, 0);
        const uint32_t rm[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        uint32_t g = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) g |= (((rm[r >> 1] >> (16 * (r & 1))) & m[u]) != 0u) ? (1u << r) : 0u;
        f |= g;
      }
      f = wave_or(f) & cur.need[u];
      if (f != 0u) pol.found(cur.seg[u].x & ~SEG_SPLIT, f, lane);  // uniform
    }
    if (!more) break;
    cur = nxt;
    s0 = s1;
  }
}

template <int U, class Pol>
DBS_DEV void pattern_pull(const PatSrc &S, const Pol &pol, int64_t s0, int64_t stride, bool eager, int lane,
                          uint32_t *s_mark) {
  if (eager) pattern_pull_wave<U, true>(S, pol, s0, stride, lane, s_mark);
  else pattern_pull_wave<U, false>(S, pol, s0, stride, lane, s_mark);
}

