// Registration of the nonzero vector blocks (section 4.1 of "DB-SpMSpV:
// Dual-View Blocked Sparse Matrix-Sparse Vector Multiplication for Dynamic
// GPU Workloads"): N_nzblk and the compacted list of nonzero blocks.  The
// push path's work chunks (64 tiles of one column block each, section 3.3.2)
// are enumerated from that list by the pushing kernel itself
// (listed_chunks) whenever a push can involve at most PUSH_LIST_MAX blocks;
// otherwise (Reg::build_chunks) they are cut here, as follows.
//
// Same-address device atomics serialize on this GPU (about 11 ns each, one
// after the other), so a workgroup first counts its blocks over all its
// rounds, reserves its range of the list with ONE atomic, then runs its
// rounds again and writes the entries (a workgroup with a single round, the
// usual case, does it all in one pass).  The value that atomic returns plus
// the workgroup's own count is a lower bound of N_nzblk: once it rules the
// push path out (section 3.2 selector), the workgroup skips the chunks, so at
// the densities that pull the chunk list costs next to nothing.  When the
// call does push, no workgroup could have ruled it out, so every chunk is
// written.
#pragma once

#include "common.h"

namespace dbs_meta {

constexpr int MT = 1024;         // threads per workgroup (16 waves: one round covers 1024 items)
constexpr int MAX_GROUPS = 512;  // workgroups of a registration kernel (<= 512 atomics per counter)

struct Reg {
  uint32_t *ctr;  // [0] nonzero blocks, [1] push chunks (zero on entry)
  uint32_t *list;
  uint64_t *chunks;
  int64_t list_cap, chunk_cap;
  const uint32_t *cb_ptr;
  // selector: push iff force_path == 1, or force_path == 0 and N_nzblk * th3_den < nb * th3_num
  int32_t nb, force_path;
  int64_t th3_num, th3_den;
  int32_t build_chunks;  // 0: the pushing kernel enumerates the chunks from the list itself
};

// The selector of section 3.3.1 on an integer count: push iff the path is
// forced to push, or it is automatic and N_nzblk / N_blk < th3 = num / den.
__host__ __device__ inline bool selector_push(uint32_t nz, int32_t nb, int32_t force_path, int64_t th3_num,
                                              int64_t th3_den) {
  return force_path == 1 || (force_path == 0 && (int64_t)nz * th3_den < (int64_t)nb * th3_num);
}

// N_nzblk as every consumer of the count uses it.  The registration counts
// one list entry per leader (an x entry whose predecessor lies in another
// vector block).  A strictly increasing x_idx has exactly one leader per
// nonzero block, so the count is at most nb; an x_idx that is not strictly
// increasing may have several leaders per block (up to 16 nb counted), and
// the list holds only nb entries.  Every position below the clamped count
// has been written with a valid block (workgroups reserve contiguous ranges
// from 0 and write each position below the list's capacity), so reading the
// list up to the clamped count stays in bounds whatever x_idx holds.
__host__ __device__ inline uint32_t nzblk_clamped(uint32_t raw, int32_t nb) {
  return raw < (uint32_t)nb ? raw : (uint32_t)nb;
}

DBS_DEV bool takes_push(const Reg &o, uint32_t nz) {
  return selector_push(nzblk_clamped(nz, o.nb), o.nb, o.force_path, o.th3_num, o.th3_den);
}

// exclusive workgroup scan; total in t
DBS_DEV void wg_scan(uint32_t a, uint32_t &e, uint32_t &t) {
  __shared__ uint32_t s_a[MT / DBS_WAVE];
  const int lane = __lane_id(), w = threadIdx.x / DBS_WAVE;
  const uint32_t ia = group_incl_scan_u32<64>(a);
  if (lane == 63) s_a[w] = ia;
  __syncthreads();
  uint32_t pa = 0;
  t = 0;
#pragma unroll
  for (int i = 0; i < MT / DBS_WAVE; ++i) {
    if (i < w) pa += s_a[i];
    t += s_a[i];
  }
  __syncthreads();
  e = pa + ia - a;
}

// `item(i, pass, leader, b)` names the vector block b of item i and whether
// this thread registers it (pass 0 also performs the item's side effects,
// e.g. writing the mask).  It is called by every thread of the workgroup for
// every round, so it may use wave-wide operations.
template <class Item>
DBS_DEV void register_blocks(const Reg &o, int64_t nitems, Item item) {
  __shared__ uint32_t s_pref[MT], s_ex[MT], s_blk[MT];
  __shared__ uint32_t s_base, s_cbase;
  const int tid = threadIdx.x;
  const int64_t rounds = (nitems + MT - 1) / MT;
  // the list entries and push chunks of one round, given the round's scan
  // (e, t) and the list position run of its first entry
  auto emit = [&](bool leader, uint32_t b, uint32_t e, uint32_t t, uint32_t run, bool chunks) {
    if (leader && (int64_t)run + e < o.list_cap) o.list[run + e] = b;
    if (!chunks) return;  // uniform
    const uint32_t nch = leader ? (o.cb_ptr[b + 1] - o.cb_ptr[b] + 63u) >> 6 : 0u;
    uint32_t ec, tc;
    wg_scan(nch, ec, tc);
    if (tc == 0u) return;  // uniform
    if (tid == 0) s_cbase = atomicAdd(&o.ctr[1], tc);
    s_pref[tid] = ec + nch;
    s_ex[tid] = ec;
    s_blk[tid] = b;
    __syncthreads();
    const uint32_t cbase = s_cbase;
    for (uint32_t j = (uint32_t)tid; j < tc; j += MT) {
      int lo = 0, hi = MT - 1;  // first thread whose inclusive prefix exceeds j
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] > j) hi = mid;
        else lo = mid + 1;
      }
      const int64_t pos = (int64_t)cbase + j;
      if (pos < o.chunk_cap) o.chunks[pos] = (uint64_t)s_blk[lo] | ((uint64_t)(j - s_ex[lo]) << 32);
    }
    __syncthreads();
  };
  if (blockIdx.x < rounds && blockIdx.x + (int64_t)gridDim.x >= rounds) {
    // one round for this workgroup: count, reserve and write in one pass
    bool leader = false;
    uint32_t b = 0;
    item((int64_t)blockIdx.x * MT + tid, 0, leader, b);
    uint32_t e, t;
    wg_scan(leader ? 1u : 0u, e, t);
    if (t == 0u) return;  // uniform
    if (tid == 0) s_base = atomicAdd(&o.ctr[0], t);
    __syncthreads();
    const uint32_t run = s_base;
    // N_nzblk >= run + t: once that already rules push out, no chunks
    emit(leader, b, e, t, run,
         o.build_chunks != 0 && (o.force_path == 1 || (o.force_path == 0 && takes_push(o, run + t))));
    return;
  }
  uint32_t tot = 0;
  for (int r = blockIdx.x; r < rounds; r += gridDim.x) {  // pass 0: count
    bool leader = false;
    uint32_t b = 0;
    item((int64_t)r * MT + tid, 0, leader, b);
    uint32_t e, t;
    wg_scan(leader ? 1u : 0u, e, t);
    tot += t;
  }
  if (tot == 0u) return;  // uniform
  if (tid == 0) s_base = atomicAdd(&o.ctr[0], tot);
  __syncthreads();
  uint32_t run = s_base;
  // N_nzblk >= run + tot: once that already rules push out, no chunks
  const bool chunks =
      o.build_chunks != 0 && (o.force_path == 1 || (o.force_path == 0 && takes_push(o, run + tot)));
  for (int r = blockIdx.x; r < rounds; r += gridDim.x) {  // pass 1: write
    bool leader = false;
    uint32_t b = 0;
    item((int64_t)r * MT + tid, 1, leader, b);
    uint32_t e, t;
    wg_scan(leader ? 1u : 0u, e, t);
    emit(leader, b, e, t, run, chunks);
    run += t;
  }
}

// Push work taken straight from the compacted list: each workgroup lists the
// chunks (64 tiles of one column block, section 3.3.2) of the n listed blocks
// on its own, as inclusive prefix sums of their chunk counts (returning the
// number of chunks), and finds chunk c of the grid-stride loop by a search
// (listed_chunk).  So no chunk list is built ahead of a call that may not
// push.  Up to 64 blocks each wave keeps the sums in registers (lane i:
// block i); more go to LDS (s_cum, at most PUSH_LIST_MAX entries), and then
// every thread of the workgroup calls listed_chunks.
constexpr int PUSH_LIST_MAX = 6144;

struct Listed {
  const uint32_t *list, *s_cum;
  uint32_t n;
  uint32_t cum, blk;  // n <= 64: this lane's block and inclusive chunk sum
};

template <int KTH>
DBS_DEV uint32_t listed_chunks(Listed &L, const uint32_t *list, uint32_t n, const uint32_t *cb_ptr,
                               uint32_t *s_cum) {
  __shared__ uint32_t s_wtot[KTH / DBS_WAVE];
  // a pushing call that enumerates from the list has n <= PUSH_LIST_MAX
  // (push_from_list and the clamped count guarantee it); the clamp keeps
  // s_cum in bounds even if a caller broke that
  n = n < (uint32_t)PUSH_LIST_MAX ? n : (uint32_t)PUSH_LIST_MAX;
  L.list = list;
  L.s_cum = s_cum;
  L.n = n;
  if (n <= (uint32_t)DBS_WAVE) {  // uniform
    const uint32_t lane = (uint32_t)__lane_id();
    const bool in = lane < n;
    const uint32_t b = list[in ? lane : 0u];
    const uint32_t cnt = in ? (cb_ptr[b + 1] - cb_ptr[b] + 63u) >> 6 : 0u;
    L.blk = b;
    L.cum = group_incl_scan_u32<64>(cnt);
    return (uint32_t)__builtin_amdgcn_readlane((int)L.cum, DBS_WAVE - 1);
  }
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < n; i += KTH) {
    const uint32_t b = list[i];
    s_cum[i] = (cb_ptr[b + 1] - cb_ptr[b] + 63u) >> 6;
  }
  __syncthreads();
  // thread t scans its run of entries, then the runs are offset by the
  // workgroup's exclusive scan of their sums
  const uint32_t per = (n + KTH - 1) / KTH, i0 = tid * per;
  const uint32_t i1 = i0 + per < n ? i0 + per : n;
  uint32_t loc = 0;
  for (uint32_t i = i0; i < i1; ++i) {
    loc += s_cum[i];
    s_cum[i] = loc;
  }
  const uint32_t inc = group_incl_scan_u32<64>(loc);
  const int w = (int)(tid / DBS_WAVE);
  if ((tid & (DBS_WAVE - 1)) == DBS_WAVE - 1) s_wtot[w] = inc;
  __syncthreads();
  uint32_t off = inc - loc;
  for (int k = 0; k < w; ++k) off += s_wtot[k];
  for (uint32_t i = i0; i < i1; ++i) s_cum[i] += off;
  __syncthreads();
  return s_cum[n - 1];
}

// chunk c (wave-uniform, below the count listed_chunks returned) as (block,
// chunk of the block << 32); called by every lane of the wave
DBS_DEV uint64_t listed_chunk(const Listed &L, uint32_t c) {
  uint32_t lo, before;
  if (L.n <= (uint32_t)DBS_WAVE) {  // uniform: the first lane whose inclusive sum exceeds c
    lo = (uint32_t)(__ffsll((unsigned long long)__ballot(L.cum > c)) - 1);
    before = lo ? (uint32_t)__builtin_amdgcn_readlane((int)L.cum, (int)lo - 1) : 0u;
    return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)L.blk, (int)lo) | ((uint64_t)(c - before) << 32);
  }
  lo = 0;
  uint32_t hi = L.n - 1;  // first entry whose inclusive sum exceeds c
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (L.s_cum[mid] > c) hi = mid;
    else lo = mid + 1;
  }
  before = lo ? L.s_cum[lo - 1] : 0u;
  return (uint64_t)L.list[lo] | ((uint64_t)(c - before) << 32);
}

// Host side: whether every call whose selector can pick push has at most
// PUSH_LIST_MAX nonzero blocks (then the pushing kernel enumerates its chunks
// from the list and the metadata kernel builds none).
inline bool push_from_list(int64_t nb, int64_t force_path, int64_t th3_num, int64_t th3_den) {
  if (force_path == 2) return true;  // never pushes
  if (force_path == 1) return nb <= PUSH_LIST_MAX;
  // push iff N * den < nb * num, so N <= (nb * num - 1) / den
  const __int128 lim = (__int128)nb * th3_num;
  if (lim <= 0) return true;
  if (th3_den <= 0) return false;
  return (lim - 1) / th3_den <= PUSH_LIST_MAX;
}

inline unsigned groups_for(int64_t nitems, int64_t other_work) {
  int64_t w = nitems > other_work ? nitems : other_work;
  int64_t g = (w + MT - 1) / MT;
  if (g < 1) g = 1;
  return (unsigned)(g < MAX_GROUPS ? g : MAX_GROUPS);
}

}  // namespace dbs_meta
