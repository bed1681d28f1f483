// Registration of the nonzero vector blocks (section 4.1 of "DB-SpMSpV:
// Dual-View Blocked Sparse Matrix-Sparse Vector Multiplication for Dynamic
// GPU Workloads"): N_nzblk, the compacted list of nonzero blocks and the push
// work chunks (64 tiles of one column block each, section 3.3.2).
//
// Same-address device atomics serialize on this GPU (about 11 ns each, one
// after the other), so a workgroup first counts its blocks and chunks over
// all its rounds, reserves both ranges with ONE packed 64-bit atomic, then
// runs its rounds again and writes: the list entries by their leaders, the
// chunk entries by the whole workgroup (each thread finds the block of a
// chunk by binary search over the round's prefix sums).
#pragma once

#include "common.h"

namespace dbs_meta {

constexpr int MT = 1024;         // threads per workgroup (16 waves: one round covers 1024 items)
constexpr int MAX_GROUPS = 512;  // workgroups of a registration kernel (<= 512 atomics)

struct Reg {
  uint32_t *ctr;  // [0] blocks (low word), [1] chunks (high word), 8-B aligned
  uint32_t *list;
  uint64_t *chunks;
  int64_t list_cap, chunk_cap;
  const uint32_t *cb_ptr;
};

// exclusive workgroup scans of two counters; totals in ta / tb
DBS_DEV void wg_scan2(uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb, uint32_t &ta, uint32_t &tb) {
  __shared__ uint32_t s_a[MT / DBS_WAVE], s_b[MT / DBS_WAVE];
  const int lane = __lane_id(), w = threadIdx.x / DBS_WAVE;
  const uint32_t ia = group_incl_scan_u32<64>(a), ib = group_incl_scan_u32<64>(b);
  if (lane == 63) {
    s_a[w] = ia;
    s_b[w] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int i = 0; i < MT / DBS_WAVE; ++i) {
    if (i < w) {
      pa += s_a[i];
      pb += s_b[i];
    }
    ta += s_a[i];
    tb += s_b[i];
  }
  __syncthreads();
  ea = pa + ia - a;
  eb = pb + ib - b;
}

// `item(i, pass, leader, b)` names the vector block b of item i and whether
// this thread registers it (pass 0 also performs the item's side effects,
// e.g. writing the mask).  It is called by every thread of the workgroup for
// every round, so it may use wave-wide operations.
template <class Item>
DBS_DEV void register_blocks(const Reg &o, int64_t nitems, Item item) {
  __shared__ uint32_t s_pref[MT], s_ex[MT], s_blk[MT];
  __shared__ unsigned long long s_base;
  const int tid = threadIdx.x;
  const int64_t rounds = (nitems + MT - 1) / MT;
  uint32_t tot_l = 0, tot_c = 0, base_l = 0, base_c = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (tid == 0) {
        const unsigned long long add = ((unsigned long long)tot_c << 32) | tot_l;
        s_base = add ? atomicAdd((unsigned long long *)o.ctr, add) : 0ull;
      }
      __syncthreads();
      base_l = (uint32_t)s_base;
      base_c = (uint32_t)(s_base >> 32);
      if (tot_l == 0u) return;  // uniform: nothing of this workgroup to write
    }
    uint32_t run_l = 0, run_c = 0;
    for (int64_t r = blockIdx.x; r < rounds; r += gridDim.x) {
      bool leader = false;
      uint32_t b = 0;
      item(r * MT + tid, pass, leader, b);
      const uint32_t nch = leader ? (o.cb_ptr[b + 1] - o.cb_ptr[b] + 63u) >> 6 : 0u;
      uint32_t el, ec, tl, tc;
      wg_scan2(leader ? 1u : 0u, nch, el, ec, tl, tc);
      if (pass == 0) {
        tot_l += tl;
        tot_c += tc;
        continue;
      }
      if (leader && (int64_t)base_l + run_l + el < o.list_cap) o.list[base_l + run_l + el] = b;
      s_pref[tid] = ec + nch;
      s_ex[tid] = ec;
      s_blk[tid] = b;
      __syncthreads();
      for (uint32_t j = (uint32_t)tid; j < tc; j += MT) {
        int lo = 0, hi = MT - 1;  // first thread whose inclusive prefix exceeds j
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_pref[mid] > j) hi = mid;
          else lo = mid + 1;
        }
        const int64_t pos = (int64_t)base_c + run_c + j;
        if (pos < o.chunk_cap) o.chunks[pos] = (uint64_t)s_blk[lo] | ((uint64_t)(j - s_ex[lo]) << 32);
      }
      __syncthreads();
      run_l += tl;
      run_c += tc;
    }
  }
}

inline unsigned groups_for(int64_t nitems, int64_t other_work) {
  int64_t w = nitems > other_work ? nitems : other_work;
  int64_t g = (w + MT - 1) / MT;
  if (g < 1) g = 1;
  return (unsigned)(g < MAX_GROUPS ? g : MAX_GROUPS);
}

}  // namespace dbs_meta
