// DB-BFS (section 4.2 and Algorithm 5 of "DB-SpMSpV: Dual-View Blocked Sparse
// Matrix-Sparse Vector Multiplication for Dynamic GPU Workloads").
//
// The frontier is kept as a bitmap, 16 bits per vertex block, which serves
// unchanged as the blk_x_mask array of the SpMSpV (section 4.1 treats the
// frontier as such a mask set).  Per level:
//   k_bfs_level  masked Boolean SpMSpV next = A f & ~visited, push or pull
//                chosen on the device from the frontier's nonzero-block count;
//                rows found that were unvisited when the level started are
//                claimed with non-returning atomic ORs on the next and
//                visited bitmaps, and their level is stored.  On a pattern
//                matrix a pull level is two launches, the first segment of
//                each row block and then the others, so that a long row
//                block whose rows are all found by its first segment is not
//                read further (the bottom-up early exit, per row block);
//   k_bfs_meta   counts the nonzero blocks of the next bitmap, lists them
//                (one atomic per workgroup) and clears the bitmap two levels
//                back.  A pushing level takes its work chunks from that list
//                (each workgroup enumerates them); only when a push could
//                involve more blocks than that enumeration holds does the
//                metadata kernel cut the chunks ahead, while push is still
//                possible.
// Three bitmaps rotate: current frontier, next frontier, and one being
// cleared.  The host launches levels in batches without waiting: each level
// kernel records its frontier's nonzero-block count, and one read of those
// counts per batch finds the first empty frontier, where the traversal ends.
// Levels of a batch past that point see an empty frontier and return at
// once (no vertex is found, nothing is written but cleared counters).
#include <mutex>

#include "meta.h"
#include "pattern_pull.h"
#include "tile_kernels.h"

namespace {

constexpr int KT = 256;

struct BfsParams {
  const uint32_t *t_cb;
  const uint32_t *t_cbx;   // pattern matrices: the Boolean pull's column-block words
  const uint64_t *meta2;   // pattern matrices: metadata of the tiles not marked single
  const uint32_t *m2seg;   // pattern matrices: per pull segment, first entry in meta2 and entries
  bool cbx_compact;        // nb <= CBX_MAX_NB: the words mark single tiles
  const uint64_t *t_meta;
  const uint32_t *cb_ptr;
  const uint32_t *csc_rb;
  const uint32_t *csc2csr;
  const uint16_t *csc_cm;   // columns of each tile with entries, CSC order
  const uint8_t *payload;
  uint64_t dense_mask_off;
  const uint32_t *segs;
  const uint32_t *psegs;    // pattern matrices: Boolean-pull segments, the nseg0 of the first launch ahead
  const uint32_t *rb_ptr;
  const uint8_t *wown;      // pattern matrices: owner tile of each payload word
  int64_t nseg, npseg, nseg0, T, payload_bytes;
  int32_t m, nb;
  const uint32_t *cur_bm;   // frontier of this level
  const uint32_t *cur_fbits;  // a bit per frontier bitmap word (two blocks) that is nonzero, fw words
  int32_t fw;
  uint32_t *next_bm;        // frontier of the next level (cleared)
  uint32_t *vis;            // visited bitmap
  const uint32_t *cur_ctr;  // [0] nonzero blocks, [1] push chunks
  const uint64_t *cur_chunks;
  const uint32_t *cur_list; // nonzero blocks of the frontier
  int32_t list_push;        // push chunks come from cur_list (none were built)
  uint32_t *hist;           // nonzero blocks of the current frontier, stored at [level % batch]
  int32_t *levels;
  int32_t level;            // level of the current frontier
  int32_t phase;            // 0: push, or the first segment of each row block; 1: the other segments
  int32_t force_path;
  int64_t th3_num, th3_den;
};

DBS_DEV uint32_t bm_get(const uint32_t *bm, uint32_t b) { return (bm[b >> 1] >> ((b & 1u) * 16u)) & 0xFFFFu; }

DBS_DEV uint32_t rows_valid(int32_t m, uint32_t rb) {
  const int64_t left = (int64_t)m - (int64_t)rb * 16;
  return left >= 16 ? 0xFFFFu : (left <= 0 ? 0u : ((1u << left) - 1u));
}

// Claim rows `f` of row block rb for the next level.  Every row in f was
// unvisited when this level started, so its distance is level + 1 whoever
// claims it: the bitmaps take plain (non-returning) atomic ORs and a row
// found twice in this level just has the same level stored twice.
DBS_DEV void claim(const BfsParams &P, uint32_t rb, uint32_t f) {
  const uint32_t sh = (rb & 1u) * 16u;
  atomicOr(&P.next_bm[rb >> 1], f << sh);
  atomicOr(&P.vis[rb >> 1], f << sh);
}

// the same for a wave-uniform f: lane 0 takes the atomics, lanes 0..15
// store the levels
DBS_DEV void claim_wave(const BfsParams &P, uint32_t rb, uint32_t f, int lane) {
  if (lane == 0) claim(P, rb, f);
  if (lane < 16 && ((f >> lane) & 1u)) P.levels[rb * 16u + (uint32_t)lane] = P.level + 1;
}

// one lane's rows, not yet checked against the visited bitmap
DBS_DEV void discover(const BfsParams &P, uint32_t rb, uint32_t f) {
  f &= ~bm_get(P.vis, rb) & rows_valid(P.m, rb);
  if (!f) return;
  claim(P, rb, f);
  for (uint32_t b = f; b; b &= b - 1u) P.levels[rb * 16u + (uint32_t)(__ffs(b) - 1)] = P.level + 1;
}

template <int VK>
DBS_DEV const uint8_t *dmask(const BfsParams &P, uint64_t vp) {
  constexpr uint64_t TS = VK == VK_F32 ? 1024 : 512;
  return P.payload + P.dense_mask_off + 32 * (vp / TS);
}

template <int VK>
DBS_DEV void bfs_push_chunk(const BfsParams &P, uint64_t own, int lane) {
  const uint32_t b = (uint32_t)own, j = (uint32_t)(own >> 32);
  const uint32_t m = bm_get(P.cur_bm, b);
  const uint32_t k0 = P.cb_ptr[b] + j * 64u, k = k0 + (uint32_t)lane;
  // a tile without an entry in a frontier column finds nothing: its
  // metadata is not read
  const bool act = k < P.cb_ptr[b + 1] && (P.csc_cm[k < P.cb_ptr[b + 1] ? k : k0] & m) != 0u;
  uint32_t rb = 0;
  uint64_t meta = 0;
  if (act) {
    rb = P.csc_rb[k];
    meta = P.t_meta[P.csc2csr[k]];
  }
  const uint32_t type = meta_type(meta);
  if (act && type == DBS_TILE_COO) discover(P, rb, coo_or_meta(P.payload, meta, m));
  uint64_t todo = __ballot(act && type != DBS_TILE_COO);
  while (todo) {
    const int src = __ffsll((unsigned long long)todo) - 1;
    todo &= todo - 1;
    const uint32_t trb = (uint32_t)__shfl((int)rb, src);
    const uint64_t tm = __shfl(meta, src);
    const uint32_t f = tile_or<VK>(P.payload + meta_vp(tm), dmask<VK>(P, meta_vp(tm)), meta_type(tm), m, lane);
    if (lane == 0) discover(P, trb, f);
  }
}

// Pull: a wave takes U consecutive segments and issues each load phase for
// all of them before using any result, with buffer loads (idle lanes pass an
// out-of-range offset instead of branching), guard-free COO decoding and a
// DPP wave OR, as in the OR-AND SpMSpV pull.
struct BfsRes {
  brsrc_t tcb, tmeta, pay, bm;
};

template <int VK, int U>
DBS_DEV void bfs_pull_group(const BfsParams &P, const BfsRes &R, int64_t s0, bool eager, int lane) {
  uint4 seg[U];
  uint32_t need[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t si = s0 + u < P.nseg ? s0 + u : P.nseg - 1;
    seg[u] = ((const uint4 *)P.segs)[si];
  }
  // rows still to be found in each row block; a fully visited row block is
  // skipped without reading its tiles
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t rb = seg[u].x & SEG_RB_MASK;
    need[u] = s0 + u < P.nseg ? (~bm_get(P.vis, rb) & rows_valid(P.m, rb)) : 0u;
  }
  uint32_t cb[U], m[U], pw0[U], pw1[U];
  uint64_t meta[U];
  bool act[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t t = seg[u].y + (uint32_t)lane;
    act[u] = (need[u] != 0u) & (t < seg[u].z);
    cb[u] = bld32(R.tcb, act[u] ? t * 4u : OOB_OFF);
    meta[u] = eager ? bld64(R.tmeta, act[u] ? t * 8u : OOB_OFF) : 0ull;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t w = bld32(R.bm, act[u] ? (cb[u] >> 1) * 4u : OOB_OFF);
    m[u] = (w >> ((cb[u] & 1u) * 16u)) & 0xFFFFu;
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
    if (!need[u]) continue;
    uint32_t f = lane_coo_or(P.payload, meta[u], m[u], act[u], pw0[u], pw1[u]);
    f = wave_or(f);
    uint64_t todo = __ballot(act[u] & (meta_type(meta[u]) != DBS_TILE_COO));
    while (todo && (f & need[u]) != need[u]) {
      const int src = __ffsll((unsigned long long)todo) - 1;
      todo &= todo - 1;
      const uint64_t tm = __shfl(meta[u], src);
      const uint32_t tmask = (uint32_t)__shfl((int)m[u], src);
      f |= tile_or<VK>(P.payload + meta_vp(tm), dmask<VK>(P, meta_vp(tm)), meta_type(tm), tmask, lane);
    }
    if (f & need[u]) claim_wave(P, seg[u].x & SEG_RB_MASK, f & need[u], lane);  // uniform
  }
}

// BFS pull on a pattern matrix: rows of a row block not yet visited are
// wanted, masks come from the frontier bitmap, found rows are claimed for
// the next level.  The visited word may miss rows claimed earlier in this
// level (that only costs work), never rows of earlier levels.
// FILTER: the frontier's word bits are in LDS, and only the tiles whose
// column block lies in a nonzero bitmap word read that word from memory
// (the reads of the others would find a zero mask).
template <bool FILTER>
struct BfsPol {
  const BfsParams *P;
  brsrc_t bm, vis;
  const uint32_t *bits;  // FILTER: LDS
  DBS_DEV uint32_t need_v(uint32_t rb, bool in) const {
    const uint32_t w = bld32(vis, in ? (rb >> 1) * 4u : OOB_OFF);
    return ~(w >> ((rb & 1u) * 16u)) & rows_valid(P->m, rb);
  }
  DBS_DEV uint32_t mask(uint32_t cb, bool in) const {
    if constexpr (FILTER) in = in && active(cb);  // idle lanes hold cb 0
    return mask_of(mask_raw(cb, in), cb);
  }
  // FILTER: the frontier bitmap word of the block is nonzero (LDS bit)
  DBS_DEV bool active(uint32_t cb) const { return (bits[cb >> 6] >> ((cb >> 1) & 31u)) & 1u; }
  // the frontier bitmap word as loaded, and the block's mask in it
  DBS_DEV uint32_t mask_raw(uint32_t cb, bool in) const { return bld32(bm, in ? (cb >> 1) * 4u : OOB_OFF); }
  DBS_DEV uint32_t mask_of(uint32_t w, uint32_t cb) const { return (w >> ((cb & 1u) * 16u)) & 0xFFFFu; }
  // rows found by the very sparse pull (n entries, LDS), not yet checked
  // against the visited bitmap: an entry per lane
  DBS_DEV void flush_new(const uint32_t *frb, const uint32_t *ff, int n, int lane) const {
    for (int e = lane; e < n; e += DBS_WAVE) discover(*P, frb[e], ff[e]);
  }
  // rows found in n row blocks (LDS): lane j claims row block j, then the
  // levels are stored four row blocks per pass, a lane per row
  DBS_DEV void flush(const uint32_t *frb, const uint32_t *ff, int n, int lane) const {
    if (lane < n) claim(*P, frb[lane], ff[lane]);
    for (int e0 = 0; e0 < n; e0 += 4) {
      const int e = e0 + (lane >> 4), r = lane & 15;
      const bool in = e < n;
      const uint32_t rb = frb[in ? e : 0], f = in ? ff[e] : 0u;
      if ((f >> r) & 1u) P->levels[rb * 16u + (uint32_t)r] = P->level + 1;
    }
  }
};

// pattern matrices: five waves per SIMD (at most 96 VGPRs), as the Boolean
// SpMSpV pull
template <int VK>
__global__ __launch_bounds__(KT, VK == VK_PAT ? 4 : 1) void k_bfs_level(BfsParams P) {
  __shared__ uint32_t s_pat[VK == VK_PAT ? KT / DBS_WAVE : 1][PAT_LDS_WORDS];
  __shared__ uint32_t s_cum[dbs_meta::PUSH_LIST_MAX];
  const int lane = __lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / DBS_WAVE);
  // the frontier's blocks are registered once each (one per nonzero bitmap
  // word half), so the count is at most nb; clamped all the same
  const uint32_t nz = dbs_meta::nzblk_clamped(P.cur_ctr[0], P.nb);
  if (P.phase == 0 && blockIdx.x == 0 && threadIdx.x == 0) P.hist[P.level % dbs_matrix::kBfsBatch] = nz;
  if (nz == 0u) return;  // uniform: empty frontier, nothing to find
  const bool push = dbs_meta::selector_push(nz, P.nb, P.force_path, P.th3_num, P.th3_den);
  // the second launch only pulls the remaining segments of a pattern matrix
  if (P.phase != 0 && (push || VK != VK_PAT)) return;  // uniform
  const int64_t gw = (int64_t)blockIdx.x * (KT / DBS_WAVE) + w;
  const int64_t nw = (int64_t)gridDim.x * (KT / DBS_WAVE);
  if (push) {
    dbs_meta::Listed L;
    const int64_t nch =
        P.list_push ? (int64_t)dbs_meta::listed_chunks<KT>(L, P.cur_list, nz, P.cb_ptr, s_cum) : (int64_t)P.cur_ctr[1];
    for (int64_t c = gw; c < nch; c += nw)
      bfs_push_chunk<VK>(P, P.list_push ? dbs_meta::listed_chunk(L, (uint32_t)c) : P.cur_chunks[c], lane);
  } else {
    constexpr int U = 8;
    const bool eager = (int64_t)nz * 4 > (int64_t)P.nb;
    BfsRes R;
    R.tcb = make_rsrc(P.t_cb, (uint64_t)P.T * 4);
    R.tmeta = make_rsrc(P.t_meta, (uint64_t)P.T * 8);
    R.pay = make_rsrc(P.payload, (uint64_t)P.payload_bytes);
    R.bm = make_rsrc(P.cur_bm, (uint64_t)((P.nb + 1) / 2) * 4);
    if constexpr (VK == VK_PAT) {
      const uint32_t *sg = P.phase == 0 ? P.psegs : P.psegs + 4 * P.nseg0;
      const PatSrc S{P.t_cb,
                     P.t_meta,
                     sg,
                     P.phase == 0 ? P.nseg0 : P.npseg - P.nseg0,
                     make_rsrc(P.payload, (uint64_t)P.payload_bytes + DBS_PAYLOAD_SLACK),
                     make_rsrc(P.wown, (uint64_t)(P.payload_bytes + DBS_PAYLOAD_SLACK) / 4),
                     P.t_cbx,
                     P.cbx_compact ? (uint32_t)(CBX_MAX_NB - 1) : (1u << CBX_RI_SHIFT_WIDE) - 1u,
                     P.cbx_compact ? CBX_SINGLE : 0u,
                     P.cbx_compact ? (uint32_t)CBX_RI_SHIFT : (uint32_t)CBX_RI_SHIFT_WIDE,
                     P.meta2,
                     (const uint2 *)P.m2seg + (P.phase == 0 ? 0 : P.nseg0)};
      const brsrc_t rv = make_rsrc(P.vis, (uint64_t)((P.nb + 1) / 2) * 4);
      if (!eager && P.fw <= dbs_meta::PUSH_LIST_MAX) {  // uniform
        // the frontier's word bits in the push enumeration's LDS
        for (int i = (int)threadIdx.x; i < P.fw; i += KT) s_cum[i] = P.cur_fbits[i];
        __syncthreads();
        const BfsPol<true> pol{&P, R.bm, rv, s_cum};
        constexpr int SP_BITS_MAX = sp_bits_max(KT / DBS_WAVE);
        // the very sparse pull when under 1/128 of the vertex blocks are in
        // the frontier (and its found-row buffers fit after the bits): at a
        // percent or more the frontier's blocks include hub columns that hold
        // most tiles, and per-segment finishing does better (R-MAT scale 22)
        if ((int64_t)nz * 128 < (int64_t)P.nb && P.fw <= SP_BITS_MAX)  // uniform
          pattern_pull_sparse<PAT_K>(S, pol, gw, nw, lane, s_pat[w], s_cum + SP_BITS_MAX + w * 2 * SP_FOUND_CAP);
        else pattern_pull<true>(S, pol, gw, nw, false, lane, s_pat[w]);
      } else {
        const BfsPol<false> pol{&P, R.bm, rv, nullptr};
        pattern_pull(S, pol, gw, nw, eager, lane, s_pat[w]);
      }
    } else {
      for (int64_t s = gw * U; s < P.nseg; s += nw * U) bfs_pull_group<VK, U>(P, R, s, eager, lane);
    }
  }
}

// bit k of the result: block bit 2k or 2k+1 of v (the blocks of one bitmap word)
DBS_DEV uint32_t word_bits(uint64_t v) {
  v = (v | (v >> 1)) & 0x5555555555555555ull;
  v = (v | (v >> 1)) & 0x3333333333333333ull;
  v = (v | (v >> 2)) & 0x0F0F0F0F0F0F0F0Full;
  v = (v | (v >> 4)) & 0x00FF00FF00FF00FFull;
  v = (v | (v >> 8)) & 0x0000FFFF0000FFFFull;
  v = (v | (v >> 16)) & 0x00000000FFFFFFFFull;
  return (uint32_t)v;
}

// Frontier metadata: nonzero blocks of `bm`, their list and push chunks, and
// a bit per nonzero bitmap word (fbits);
// clears `clr_bm` / `clr_ctr` (the buffers two levels back) when given.
// After the traversal has ended (the level's own frontier, counted in
// in_ctr, was empty) only the counters two levels back are cleared: the next
// frontier is empty and its counters are zero already, and with those
// cleared too every later level of the batch sees an empty frontier and
// returns at once (the bitmaps are cleared by the next BFS's start).
__global__ __launch_bounds__(dbs_meta::MT) void k_bfs_meta(const uint32_t *bm, int32_t nb, dbs_meta::Reg reg,
                                                 uint32_t *clr_bm, uint32_t *clr_ctr, int64_t nwords,
                                                 const uint32_t *in_ctr, uint32_t *fbits) {
  if (in_ctr[0] == 0u) {  // uniform
    if (clr_ctr && blockIdx.x == 0 && threadIdx.x < 8) clr_ctr[threadIdx.x] = 0;
    return;
  }
  const int64_t gs = (int64_t)gridDim.x * dbs_meta::MT;
  if (clr_bm) {
    for (int64_t k = (int64_t)blockIdx.x * dbs_meta::MT + threadIdx.x; k < nwords; k += gs) clr_bm[k] = 0;
    if (blockIdx.x == 0 && threadIdx.x < 8) clr_ctr[threadIdx.x] = 0;
  }
  dbs_meta::register_blocks(reg, nb, [&](int64_t b, int pass, bool &leader, uint32_t &bo) {
    leader = b < nb && bm_get(bm, (uint32_t)b) != 0u;
    bo = (uint32_t)b;
    // the bitmap's word bits: a wave holds 64 consecutive blocks (32 words)
    // from a multiple of 64, one bit word
    const uint64_t bal = __ballot(leader);
    if (pass == 0 && __lane_id() == 0 && b < nb) fbits[b >> 6] = word_bits(bal);
  });
}

// Start of a BFS in one launch: levels (0 at the source, -1 elsewhere), the
// three frontier bitmaps cleared but for the source's bit, the visited
// bitmap (rows without an entry start out visited: no level can reach them,
// and a row block whose remaining rows are all such is skipped by the pull),
// and the first frontier's metadata: one nonzero block, listed, and, when
// level 0 pushes from chunks built ahead, the push chunks of its column block.
__global__ void k_bfs_init(int32_t *levels, int32_t m, uint32_t *bm3, int64_t bm_words3, uint32_t *vis,
                           const uint32_t *rows_nz, int64_t nwords, uint32_t *ctr3, int32_t src,
                           const uint32_t *cb_ptr, uint32_t *list0, uint64_t *chunks0, int64_t chunk_cap, int push0,
                           uint32_t *fbits0, int32_t fw) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gs = (int64_t)gridDim.x * blockDim.x;
  const uint32_t b = (uint32_t)src >> 4;
  const int64_t ws = b >> 1;
  const uint32_t bits = (1u << ((uint32_t)src & 15u)) << ((b & 1u) * 16u);
  for (int64_t k = i; k < m; k += gs) levels[k] = k == src ? 0 : -1;
  for (int64_t k = i; k < bm_words3; k += gs) bm3[k] = k == ws ? bits : 0u;
  for (int64_t k = i; k < nwords; k += gs) vis[k] = ~rows_nz[k] | (k == ws ? bits : 0u);
  for (int64_t k = i; k < fw; k += gs) fbits0[k] = k == (int64_t)(b >> 6) ? 1u << ((b >> 1) & 31u) : 0u;
  const uint32_t t = cb_ptr[b + 1] - cb_ptr[b];
  int64_t nch = push0 ? (int64_t)((t + 63u) >> 6) : 0;
  nch = nch < chunk_cap ? nch : chunk_cap;
  for (int64_t k = i; k < nch; k += gs) chunks0[k] = (uint64_t)b | ((uint64_t)k << 32);
  if (i < 24) ctr3[i] = i == 0 ? 1u : i == 1 ? (uint32_t)nch : 0u;
  if (i == 0) list0[0] = b;
}

// Vertices reached by the last BFS: the visited bitmap holds every row
// without an entry (set at the start: such a row cannot be reached) and the
// reached rows, so the reached rows are the visited rows that hold an entry,
// plus the source when its row holds none.  One workgroup sum, one atomic
// per workgroup.
__global__ __launch_bounds__(256) void k_bfs_reached(const uint32_t *vis, const uint32_t *rows_nz, int64_t nwords,
                                                     uint32_t *out) {
  __shared__ uint32_t s_w[256 / DBS_WAVE];
  uint32_t c = 0;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < nwords; k += (int64_t)gridDim.x * 256)
    c += (uint32_t)__popc(vis[k] & rows_nz[k]);
  c = group_sum_u32<64>(c);
  if (__lane_id() == 0) s_w[threadIdx.x / DBS_WAVE] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 256 / DBS_WAVE; ++i) t += s_w[i];
    if (t) atomicAdd(out, t);
  }
}

}  // namespace

#define BFS_TRY(expr)                                                                            \
  do {                                                                                           \
    hipError_t e_ = DBS_NOTE(expr);                                                                      \
    if (e_ != hipSuccess)                                                                        \
      return (e_ == hipErrorOutOfMemory || e_ == hipErrorMemoryAllocation) ? DBS_ERR_OUT_OF_MEMORY \
                                                                       : DBS_ERR_DEVICE;        \
  } while (0)

namespace {

// Device scratch of one BFS run: three rotating frontier bitmaps, the
// visited bitmap, three block lists, three chunk lists (only when a push may
// need chunks cut ahead), 3 x 8 counters then the frontier sizes of one batch
// of levels and a spare counter, and a host buffer that receives the sizes.
struct BfsScratch {
  uint32_t *bm, *vis, *list;
  uint32_t *fbits;  // 3 x fw words: the bits of each frontier bitmap's nonzero words
  uint64_t *chunks;
  uint32_t *ctr;
  uint32_t *host;  // 64 B of host memory (pinned for dbs_bfs)
};

// whether push chunks come from the frontier's block list (then no chunk
// list is needed)
bool bfs_list_push(const dbs_matrix *A) {
  return dbs_meta::push_from_list(A->nb, A->opt[DBS_OPT_PATH], A->opt[DBS_OPT_TH3_NUM], A->opt[DBS_OPT_TH3_DEN]);
}

dbs_status bfs_run(dbs_matrix *A, const BfsScratch &S, int32_t src, int32_t *levels, hipStream_t s);

}  // namespace

dbs_status dbs_bfs_impl(dbs_matrix *A, int32_t src, int32_t *levels, hipStream_t s) {
  const int64_t nwords = ((int64_t)A->nb + 1) / 2;
  const int64_t chunk_cap = A->max_chunks;
  if (!A->bfs_bm) {
    BFS_TRY(dbs_dev_alloc(A, (void **)&A->bfs_bm, (size_t)(3 * nwords + 1) * 4));
    BFS_TRY(dbs_dev_alloc(A, (void **)&A->bfs_vis, (size_t)(nwords + 1) * 4));
    BFS_TRY(dbs_dev_alloc(A, (void **)&A->bfs_fbits, (size_t)(3 * (((int64_t)A->nb + 63) / 64) + 1) * 4));
    BFS_TRY(dbs_dev_alloc(A, (void **)&A->bfs_list, (size_t)(3 * (int64_t)A->nb + 1) * 4));
    BFS_TRY(dbs_dev_alloc(A, (void **)&A->bfs_chunks, (size_t)(3 * chunk_cap + 1) * 8));
    BFS_TRY(dbs_dev_alloc(A, (void **)&A->bfs_ctr, (24 + dbs_matrix::kBfsBatch + 1) * 4));
    BFS_TRY(hipHostMalloc((void **)&A->bfs_host, 64, hipHostMallocDefault));
  }
  const BfsScratch S{A->bfs_bm, A->bfs_vis, A->bfs_list, A->bfs_fbits, A->bfs_chunks, A->bfs_ctr, A->bfs_host};
  const dbs_status st = bfs_run(A, S, src, levels, s);
  A->bfs_counted = st == DBS_OK ? 1 : 0;  // its visited bitmap stays in the handle
  return st;
}

namespace {

dbs_status bfs_run(dbs_matrix *A, const BfsScratch &S, int32_t src, int32_t *levels, hipStream_t s) {
  const int64_t nwords = ((int64_t)A->nb + 1) / 2;
  const int64_t chunk_cap = A->max_chunks;
  const bool timing = A->opt[DBS_OPT_TIMING] != 0;
  if (timing) BFS_TRY(hipEventRecord(A->ev[0], s));
  const int64_t fp = A->opt[DBS_OPT_PATH];
  const bool list_push = bfs_list_push(A);
  const int push0 =
      !list_push && (fp == 1 || (fp == 0 && A->opt[DBS_OPT_TH3_DEN] < (int64_t)A->nb * A->opt[DBS_OPT_TH3_NUM]));
  const int32_t fw = (int32_t)(((int64_t)A->nb + 63) / 64);
  hipLaunchKernelGGL(k_bfs_init, dim3(1024), dim3(256), 0, s, levels, A->m, S.bm, 3 * nwords, S.vis,
                     (const uint32_t *)A->rows_nz, nwords, S.ctr, src, (const uint32_t *)A->cb_ptr, S.list,
                     S.chunks, chunk_cap, push0, S.fbits, fw);
  BFS_TRY(hipGetLastError());
  const unsigned mgrid = dbs_meta::groups_for(A->nb, nwords);
  auto reg_for = [&](int buf) {
    dbs_meta::Reg r;
    r.ctr = S.ctr + 8 * buf;
    r.list = S.list + (int64_t)buf * A->nb;
    r.chunks = S.chunks ? S.chunks + buf * chunk_cap : nullptr;  // none: chunks come from the list
    r.list_cap = A->nb;
    r.chunk_cap = chunk_cap;
    r.cb_ptr = A->cb_ptr;
    r.nb = A->nb;
    r.force_path = (int32_t)A->opt[DBS_OPT_PATH];
    r.th3_num = A->opt[DBS_OPT_TH3_NUM];
    r.th3_den = A->opt[DBS_OPT_TH3_DEN];
    r.build_chunks = list_push ? 0 : 1;
    return r;
  };

  BfsParams P;
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
  P.segs = A->segs;
  P.psegs = A->psegs;
  P.rb_ptr = A->rb_ptr;
  P.wown = A->wown;
  P.nseg = A->nseg;
  P.npseg = A->npseg;
  P.nseg0 = A->nseg0;
  P.T = A->T;
  P.payload_bytes = A->payload_bytes;
  P.m = A->m;
  P.nb = A->nb;
  P.vis = S.vis;
  P.levels = levels;
  P.force_path = (int32_t)A->opt[DBS_OPT_PATH];
  P.th3_num = A->opt[DBS_OPT_TH3_NUM];
  P.th3_den = A->opt[DBS_OPT_TH3_DEN];
  P.list_push = list_push ? 1 : 0;
  P.fw = fw;
  const int pu = A->vk == VK_PAT ? 1 : 8;
  const int64_t ns = A->vk == VK_PAT ? A->npseg : A->nseg;
  int64_t waves = (ns + pu - 1) / pu > chunk_cap ? (ns + pu - 1) / pu : chunk_cap;
  int64_t g = (waves + 3) / 4;
  static const unsigned res_f32 = dbs_resident_groups(k_bfs_level<VK_F32>, KT);
  static const unsigned res_bf16 = dbs_resident_groups(k_bfs_level<VK_BF16>, KT);
  static const unsigned res_pat = dbs_resident_groups(k_bfs_level<VK_PAT>, KT);
  const unsigned cap = A->vk == VK_F32 ? res_f32 : A->vk == VK_BF16 ? res_bf16 : res_pat;
  const unsigned grid = (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));

  constexpr int B = dbs_matrix::kBfsBatch;
  static_assert(B * 4 <= 64, "pinned mirror holds 16 counts");
  P.hist = S.ctr + 24;
  int32_t L = -1, push_levels = 0;
  float kms = 0.0f;
  for (int64_t L0 = 0; L < 0; L0 += B) {
    if (L0 > (int64_t)A->m + 1) return DBS_ERR_DEVICE;  // cannot happen: every level adds a vertex
    for (int i = 0; i < B; ++i) {
      const int64_t l = L0 + i;
      const int cur = (int)(l % 3), nxt = (int)((l + 1) % 3), clr = (int)((l + 2) % 3);
      P.cur_bm = S.bm + cur * nwords;
      P.next_bm = S.bm + nxt * nwords;
      P.cur_ctr = S.ctr + 8 * cur;
      P.cur_chunks = S.chunks ? S.chunks + cur * chunk_cap : nullptr;
      P.cur_list = S.list + (int64_t)cur * A->nb;
      P.cur_fbits = S.fbits + (int64_t)cur * fw;
      P.level = (int32_t)l;
      if (timing) BFS_TRY(hipEventRecord(A->ev[2 + 2 * i], s));
      if (A->vk == VK_F32) {
        P.phase = 0;
        hipLaunchKernelGGL(k_bfs_level<VK_F32>, dim3(grid), dim3(KT), 0, s, P);
      } else if (A->vk == VK_BF16) {
        P.phase = 0;
        hipLaunchKernelGGL(k_bfs_level<VK_BF16>, dim3(grid), dim3(KT), 0, s, P);
      } else {
        // a pull level in two launches: the first segment of every row block,
        // then the rest, which skips row blocks with nothing left to find
        P.phase = 0;
        hipLaunchKernelGGL(k_bfs_level<VK_PAT>, dim3(grid), dim3(KT), 0, s, P);
        BFS_TRY(hipGetLastError());
        P.phase = 1;
        hipLaunchKernelGGL(k_bfs_level<VK_PAT>, dim3(grid), dim3(KT), 0, s, P);
      }
      BFS_TRY(hipGetLastError());
      if (timing) BFS_TRY(hipEventRecord(A->ev[3 + 2 * i], s));
      hipLaunchKernelGGL(k_bfs_meta, dim3(mgrid), dim3(dbs_meta::MT), 0, s, (const uint32_t *)P.next_bm, A->nb,
                         reg_for(nxt), S.bm + clr * nwords, S.ctr + 8 * clr, nwords,
                         (const uint32_t *)P.cur_ctr, S.fbits + (int64_t)nxt * fw);
      BFS_TRY(hipGetLastError());
    }
    BFS_TRY(hipMemcpyAsync(S.host, P.hist, B * 4, hipMemcpyDeviceToHost, s));
    BFS_TRY(hipStreamSynchronize(s));
    for (int i = 0; i < B; ++i) {
      const uint32_t nz = S.host[i];  // nonzero blocks of frontier L0 + i
      if (nz == 0u) {
        L = (int32_t)(L0 + i);
        break;
      }
      const bool was_push = dbs_meta::selector_push(nz, A->nb, (int32_t)A->opt[DBS_OPT_PATH],
                                                    A->opt[DBS_OPT_TH3_NUM], A->opt[DBS_OPT_TH3_DEN]);
      push_levels += was_push ? 1 : 0;
      if (timing) {
        float ms = 0.0f;
        BFS_TRY(hipEventElapsedTime(&ms, A->ev[2 + 2 * i], A->ev[3 + 2 * i]));
        kms += ms;
      }
    }
  }
  if (timing) {
    BFS_TRY(hipEventRecord(A->ev[1], s));
    BFS_TRY(hipEventSynchronize(A->ev[1]));
    float ms = 0.0f;
    BFS_TRY(hipEventElapsedTime(&ms, A->ev[0], A->ev[1]));
    A->st.bfs_ms = ms;
    A->st.bfs_kernel_ms = kms;
  } else {
    A->st.bfs_ms = -1.0f;
    A->st.bfs_kernel_ms = -1.0f;
  }
  A->st.bfs_levels = L;
  A->st.bfs_push_levels = push_levels;
  A->st.bfs_reached = -1;  // counted from the visited bitmap when the statistics are read
  A->bfs_src = src;
  A->last_stream = s;
  return DBS_OK;
}

}  // namespace

dbs_status dbs_bfs_count_reached(dbs_matrix *A) {
  if (!A->bfs_counted || !A->bfs_vis || A->st.bfs_levels <= 0 || A->st.bfs_reached >= 0) return DBS_OK;
  const int64_t nwords = ((int64_t)A->nb + 1) / 2;
  hipStream_t s = A->last_stream;
  // the counter: the slot after the batch's frontier sizes
  uint32_t *cnt = A->bfs_ctr + 24 + dbs_matrix::kBfsBatch;
  BFS_TRY(hipMemsetAsync(cnt, 0, 4, s));
  const int64_t g = (nwords + 255) / 256;
  hipLaunchKernelGGL(k_bfs_reached, dim3((unsigned)(g < 1024 ? (g < 1 ? 1 : g) : 1024)), dim3(256), 0, s,
                     (const uint32_t *)A->bfs_vis, (const uint32_t *)A->rows_nz, nwords, cnt);
  BFS_TRY(hipGetLastError());
  uint32_t h = 0, src_word = 0;
  BFS_TRY(hipMemcpyAsync(&h, cnt, 4, hipMemcpyDeviceToHost, s));
  BFS_TRY(hipMemcpyAsync(&src_word, A->rows_nz + ((uint32_t)A->bfs_src >> 5), 4, hipMemcpyDeviceToHost, s));
  BFS_TRY(hipStreamSynchronize(s));
  const bool src_has_entry = (src_word >> ((uint32_t)A->bfs_src & 31u)) & 1u;
  A->st.bfs_reached = (int64_t)h + (src_has_entry ? 0 : 1);
  return DBS_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free BFS (dbs_bfs_noalloc): the same steps as dbs_bfs, with the
// scratch of the run carved from a fixed device array instead of memory the
// handle allocates.  Each device holds its own copy of the array until the
// process ends; its address is looked up once per device, with that device
// current, and kept.  Kernels receive that address, never the array's name
// (which in host code does not name device memory).  Every call on a device
// shares the array: calls that overlap in time on one device race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[DBS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// address of this device's array (looked up on the first call on the device)
hipError_t noalloc_scratch(int dev, uint8_t **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = (uint8_t *)g_scratch_ptr[dev];
  return hipSuccess;
}

// Carve the run's scratch out of `base` (256-B aligned pieces); returns the
// bytes needed, so that a null base only measures.
size_t carve(const dbs_matrix *A, bool list_push, uint8_t *base, BfsScratch &S) {
  const int64_t nwords = ((int64_t)A->nb + 1) / 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t *p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  S.bm = (uint32_t *)take((size_t)(3 * nwords + 1) * 4);
  S.vis = (uint32_t *)take((size_t)(nwords + 1) * 4);
  S.list = (uint32_t *)take((size_t)(3 * (int64_t)A->nb + 1) * 4);
  S.fbits = (uint32_t *)take((size_t)(3 * (((int64_t)A->nb + 63) / 64) + 1) * 4);
  S.ctr = (uint32_t *)take((size_t)(24 + dbs_matrix::kBfsBatch + 1) * 4);
  S.chunks = list_push ? nullptr : (uint64_t *)take((size_t)(3 * A->max_chunks + 1) * 8);
  return off;
}

}  // namespace

dbs_status dbs_bfs_noalloc_impl(dbs_matrix *A, int32_t src, int32_t *levels, hipStream_t s) {
  int dev = -1;
  BFS_TRY(hipGetDevice(&dev));
  if (dev != A->device) return DBS_ERR_INVALID_ARG;
  const bool list_push = bfs_list_push(A);
  BfsScratch S{};
  if (carve(A, list_push, nullptr, S) > (size_t)DBS_NOALLOC_SCRATCH_BYTES) return DBS_ERR_TOO_LARGE;
  uint8_t *base = nullptr;
  BFS_TRY(noalloc_scratch(dev, &base));
  carve(A, list_push, base, S);
  uint32_t host[16];  // the batch's frontier sizes (the run synchronizes before reading them)
  S.host = host;
  const dbs_status st = bfs_run(A, S, src, levels, s);
  A->bfs_counted = 0;  // the visited bitmap lives in the shared array: not counted later
  return st;
}
