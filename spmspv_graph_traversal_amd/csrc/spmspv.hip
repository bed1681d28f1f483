// DB-SpMSpV on gfx950: vector-block metadata (section 4.1), the global
// push/pull selector (section 3.3.1), path-aware work lists (section 3.3.2)
// and hierarchical writeback (section 3.3.3) of "DB-SpMSpV: Dual-View Blocked
// Sparse Matrix-Sparse Vector Multiplication for Dynamic GPU Workloads".
//
// One call = two launches on the caller's stream:
//   k_xmeta_*   builds blk_x_mask (tagged with a per-call epoch so it never
//               needs clearing), stages x, counts the nonzero vector blocks
//               with one atomic per workgroup, lists them, reserves push
//               work chunks (64 tiles of one column block each) and clears y;
//   k_spmspv    reads N_nzblk, picks push or pull on the device, and walks
//               either the push chunks or the static pull segments, one wave
//               per chunk / segment, grid-stride.
#include "tile_kernels.h"

namespace {

constexpr int KT = 256;  // threads per workgroup (4 waves)

struct MetaOut {
  uint32_t *xmask;
  uint32_t epoch;
  uint32_t *act_list;
  uint64_t *chunks;
  uint32_t *ctr;        // this call's counters: [0] N_nzblk, [1] push chunks, [2] error flags
  uint32_t *ctr_next;   // next call's counters, cleared here
  const uint32_t *cb_ptr;
  int32_t n, nb;
  int64_t max_chunks;   // capacity of `chunks`; act_list holds nb entries
  // y clearing: head bytes, 16-B body, tail bytes
  uint8_t *y;
  int64_t y_head, y_body, y_tail;
};

// Registers the leaders (first lane of each nonzero vector block) of one
// 256-thread round: compacted list + push chunk reservation, one global
// atomic per workgroup for each.
DBS_DEV void register_blocks(const MetaOut &o, bool leader, uint32_t b) {
  __shared__ uint32_t s_cnt[KT / DBS_WAVE], s_ch[KT / DBS_WAVE];
  __shared__ uint32_t s_base_cnt, s_base_ch;
  const int lane = __lane_id(), w = threadIdx.x / DBS_WAVE;
  uint32_t nch = 0;
  if (leader) {
    const uint32_t cnt = o.cb_ptr[b + 1] - o.cb_ptr[b];
    nch = (cnt + 63u) >> 6;
  }
  const uint64_t bal = __ballot(leader);
  const uint32_t rank = (uint32_t)__popcll(bal & __lanemask_lt());
  const uint32_t chinc = group_incl_scan_u32<64>(nch);
  if (lane == 63) {
    s_cnt[w] = (uint32_t)__popcll(bal);
    s_ch[w] = chinc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tc = 0, th = 0;
    for (int i = 0; i < KT / DBS_WAVE; ++i) {
      tc += s_cnt[i];
      th += s_ch[i];
    }
    s_base_cnt = tc ? atomicAdd(&o.ctr[0], tc) : 0u;
    s_base_ch = th ? atomicAdd(&o.ctr[1], th) : 0u;
  }
  __syncthreads();
  if (leader) {
    uint32_t pc = s_base_cnt, ph = s_base_ch;
    for (int i = 0; i < w; ++i) {
      pc += s_cnt[i];
      ph += s_ch[i];
    }
    // an unsorted x_idx (invalid input) can name a block more than once:
    // never write past the lists
    if (pc + rank < (uint32_t)o.nb) o.act_list[pc + rank] = b;
    const uint32_t first = ph + chinc - nch;
    for (uint32_t k = 0; k < nch && (int64_t)first + k < o.max_chunks; ++k)
      o.chunks[first + k] = (uint64_t)b | ((uint64_t)k << 32);
  }
  __syncthreads();
}

DBS_DEV void clear_y(const MetaOut &o) {
  const int64_t gt = (int64_t)blockIdx.x * KT + threadIdx.x, gs = (int64_t)gridDim.x * KT;
  if (gt < o.y_head) o.y[gt] = 0;
  uint4 *body = (uint4 *)(o.y + o.y_head);
  for (int64_t k = gt; k < o.y_body; k += gs) body[k] = make_uint4(0, 0, 0, 0);
  if (gt < o.y_tail) o.y[o.y_head + 16 * o.y_body + gt] = 0;
}

// Sparse x: sorted x_idx.  The first entry of each vector block (the leader)
// gathers the block's mask from the following entries.
template <int VK>
__global__ __launch_bounds__(KT) void k_xmeta_sparse(MetaOut o, int32_t nnz_x, const int32_t *x_idx,
                                                     const void *x_val, void *xd, int check) {
  if (blockIdx.x == 0 && threadIdx.x < 8) o.ctr_next[threadIdx.x] = 0;
  clear_y(o);
  const int64_t gs = (int64_t)gridDim.x * KT;
  for (int64_t base = (int64_t)blockIdx.x * KT; base < nnz_x; base += gs) {
    const int64_t i = base + threadIdx.x;
    const bool valid = i < nnz_x;
    const int32_t idx = valid ? x_idx[i] : -1;
    const bool inb = valid && idx >= 0 && idx < o.n;
    const int32_t b = idx >> 4;
    if (inb && VK != VK_PAT && x_val) {
      if (VK == VK_F32) ((float *)xd)[idx] = ((const float *)x_val)[i];
      else ((uint16_t *)xd)[idx] = ((const uint16_t *)x_val)[i];
    }
    const int32_t prev = (valid && i > 0) ? x_idx[i - 1] : -1;
    if (check && valid && i > 0 && idx <= prev) atomicOr(&o.ctr[2], 1u);
    const bool leader = inb && (i == 0 || (prev >> 4) != b);
    if (leader) {
      uint32_t mk = 0;
      int64_t j = i;
      for (; j < nnz_x && j < i + 16; ++j) {
        const int32_t v = x_idx[j];
        if ((v >> 4) != b || v >= o.n) break;
        mk |= 1u << (v & 15);
      }
      if (check && j == i + 16 && j < nnz_x && (x_idx[j] >> 4) == b) atomicOr(&o.ctr[2], 1u);
      o.xmask[b] = (o.epoch << 16) | mk;
    }
    register_blocks(o, leader, (uint32_t)b);
  }
}

// Dense x (decode, section 4.1): one ballot per wave gives the nonzero
// pattern of 64 consecutive entries, i.e. the masks of four vector blocks.
template <int VK>
__global__ __launch_bounds__(KT) void k_xmeta_dense(MetaOut o, const void *x) {
  if (blockIdx.x == 0 && threadIdx.x < 8) o.ctr_next[threadIdx.x] = 0;
  clear_y(o);
  const int lane = __lane_id();
  const int64_t gs = (int64_t)gridDim.x * KT;
  const int64_t npad = (int64_t)o.nb * 16;
  for (int64_t base = (int64_t)blockIdx.x * KT; base < npad; base += gs) {
    const int64_t j = base + threadIdx.x;
    bool nz = false;
    if (j < o.n) {
      if (VK == VK_BF16) nz = (((const uint16_t *)x)[j] & 0x7FFFu) != 0u;
      else nz = (__float_as_uint(((const float *)x)[j]) & 0x7FFFFFFFu) != 0u;
    }
    const uint64_t bal = __ballot(nz);
    const uint32_t mk = (uint32_t)(bal >> (lane & 48)) & 0xFFFFu;
    const bool head = (lane & 15) == 0 && j < npad;
    const uint32_t b = (uint32_t)(j >> 4);
    if (head) o.xmask[b] = (o.epoch << 16) | mk;
    register_blocks(o, head && mk != 0u, b);
  }
}

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

struct SpmvParams {
  const uint32_t *t_cb;
  const uint64_t *t_meta;
  const uint32_t *cb_ptr;
  const uint32_t *csc_rb;
  const uint32_t *csc2csr;
  const uint8_t *payload;
  uint64_t dense_mask_off;
  const uint32_t *segs;
  int64_t nseg;
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
  const bool act = k < kend;
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
      const uint32_t f = coo_or(base, nnz, m);
      for (uint32_t ff = f; ff; ff &= ff - 1u) {
        const uint32_t row = rb * 16u + (uint32_t)(__ffs(ff) - 1);
        ((uint8_t *)P.y)[row] = 1;
      }
    } else {
      constexpr int VS = VK == VK_F32 ? 4 : 2;
      const uint8_t *vals = base + coo_val_off(nnz);
      for (uint32_t e = 0; e < nnz; ++e) {
        const uint32_t rc = base[e];
        const uint32_t c = rc & 15u;
        if ((m >> c) & 1u)
          unsafeAtomicAdd((float *)P.y + rb * 16u + (rc >> 4), load_a<VK>(vals + e * VS) * sx[c]);
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
// ---------------------------------------------------------------------------
template <int VK, int SR>
DBS_DEV void pull_segment(const SpmvParams &P, int64_t s, float *sx, float *spart, int lane) {
  const uint4 seg = ((const uint4 *)P.segs)[s];
  const uint32_t rb = seg.x & ~SEG_SPLIT;
  const bool split = (seg.x & SEG_SPLIT) != 0u;
  const uint32_t t = seg.y + (uint32_t)lane;
  bool act = t < seg.z;
  uint32_t cb = 0, m = 0;
  uint64_t meta = 0;
  if (act) {
    cb = P.t_cb[t];
    const uint32_t w = P.xmask[cb];
    m = (w >> 16) == P.epoch ? (w & 0xFFFFu) : 0u;
    act = m != 0u;
    if (act) meta = P.t_meta[t];
  }
  const uint32_t type = meta_type(meta);
  const int64_t row0 = (int64_t)rb * 16;
  if (SR == DBS_OR_AND) {
    uint32_t f = 0;
    if (act && type == DBS_TILE_COO) f = coo_or(P.payload + meta_vp(meta), meta_nnz(meta), m);
    f = group_or_u32<64>(f);
    uint64_t todo = __ballot(act && type != DBS_TILE_COO);
    while (todo) {
      const int src = __ffsll((unsigned long long)todo) - 1;
      todo &= todo - 1;
      const uint64_t tm = __shfl(meta, src);
      const uint32_t tmask = (uint32_t)__shfl((int)m, src);
      f |= tile_or<VK>(P.payload + meta_vp(tm), dense_mask_ptr<VK>(P, meta_vp(tm)), meta_type(tm), tmask,
                       lane);
    }
    if (lane < 16 && row0 + lane < P.m) {
      const uint8_t bit = (uint8_t)((f >> lane) & 1u);
      if (!split) ((uint8_t *)P.y)[row0 + lane] = bit;
      else if (bit) ((uint8_t *)P.y)[row0 + lane] = 1;
    }
  } else {
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
    if (act && type == DBS_TILE_COO)
      coo_plus<VK>(P.payload + meta_vp(meta), meta_nnz(meta), m, P.xd, (int64_t)cb * 16, acc);
    float rowsum = wave_rows_reduce(acc, lane);
    uint64_t todo = __ballot(act && type != DBS_TILE_COO);
    while (todo) {
      const int src = __ffsll((unsigned long long)todo) - 1;
      todo &= todo - 1;
      const uint64_t tm = __shfl(meta, src);
      const uint32_t tmask = (uint32_t)__shfl((int)m, src);
      const uint32_t tcb = (uint32_t)__shfl((int)cb, src);
      stage_x<VK>(sx, P.xd, tcb, tmask, lane);
      rowsum += tile_plus<VK>(P.payload + meta_vp(tm), meta_type(tm), meta_nnz(tm), tmask, sx, spart,
                              P.local_cutoff, lane);
      __syncwarp();
    }
    if (lane < 16 && row0 + lane < P.m) {
      if (!split) ((float *)P.y)[row0 + lane] = rowsum;
      else if (rowsum != 0.0f) unsafeAtomicAdd((float *)P.y + row0 + lane, rowsum);
    }
  }
}

template <int VK, int SR>
__global__ __launch_bounds__(KT) void k_spmspv(SpmvParams P) {
  __shared__ float s_x[KT / DBS_WAVE][16];
  __shared__ float s_part[KT / DBS_WAVE][64];
  const int lane = __lane_id(), w = threadIdx.x / DBS_WAVE;
  const uint32_t nz = P.ctr[0];
  const bool push = P.force_path == 1 ||
                    (P.force_path == 0 && (int64_t)nz * P.th3_den < (int64_t)P.nb * P.th3_num);
  const int64_t gw = (int64_t)blockIdx.x * (KT / DBS_WAVE) + w;
  const int64_t nw = (int64_t)gridDim.x * (KT / DBS_WAVE);
  if (push) {
    const int64_t nch = (int64_t)P.ctr[1] < P.max_chunks ? (int64_t)P.ctr[1] : P.max_chunks;
    for (int64_t c = gw; c < nch; c += nw) push_chunk<VK, SR>(P, P.chunks[c], s_x[w], s_part[w], lane);
  } else {
    for (int64_t s = gw; s < P.nseg; s += nw) pull_segment<VK, SR>(P, s, s_x[w], s_part[w], lane);
  }
}

inline unsigned grid_for(int64_t waves, unsigned cap) {
  int64_t g = (waves + (KT / DBS_WAVE) - 1) / (KT / DBS_WAVE);
  if (g < 1) g = 1;
  return (unsigned)(g < cap ? g : cap);
}

template <int VK, int SR>
void launch_spmspv(const SpmvParams &P, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((k_spmspv<VK, SR>), dim3(grid), dim3(KT), 0, s, P);
}

}  // namespace

#define SPMV_TRY(expr)                                   \
  do {                                                   \
    if (DBS_NOTE(expr) != hipSuccess) return DBS_ERR_DEVICE;     \
  } while (0)

dbs_status dbs_spmspv_impl(dbs_matrix *A, int32_t nnz_x, const int32_t *x_idx, const void *x_val,
                           const void *x_dense, dbs_semiring sr, void *y, hipStream_t s) {
  const bool timing = A->opt[DBS_OPT_TIMING] != 0;
  // epoch tag of this call's masks; a full clear every 65535 calls
  A->epoch++;
  if (A->epoch > 0xFFFFu) {
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((A->nb + 255) / 256)), dim3(256), 0, s, A->xmask,
                       (int64_t)A->nb, 0u);
    SPMV_TRY(hipGetLastError());
    A->epoch = 1;
  }
  MetaOut o;
  o.xmask = A->xmask;
  o.epoch = A->epoch;
  o.act_list = A->act_list;
  o.chunks = A->chunks;
  o.ctr = A->ctr + 8 * A->cbuf;
  o.ctr_next = A->ctr + 8 * (1 - A->cbuf);
  o.cb_ptr = A->cb_ptr;
  o.n = A->n;
  o.nb = A->nb;
  o.max_chunks = A->max_chunks;
  const int64_t ybytes = (int64_t)A->m * (sr == DBS_OR_AND ? 1 : 4);
  o.y = (uint8_t *)y;
  int64_t head = (int64_t)((16 - ((uintptr_t)y & 15)) & 15);
  if (head > ybytes) head = ybytes;
  o.y_head = head;
  o.y_body = (ybytes - head) / 16;
  o.y_tail = ybytes - head - 16 * o.y_body;

  const bool dense = x_dense != nullptr;
  const int64_t xwork = dense ? (int64_t)A->nb * 16 : (int64_t)nnz_x;
  int64_t mwork = xwork > o.y_body ? xwork : o.y_body;
  unsigned mgrid = (unsigned)((mwork + KT - 1) / KT);
  if (mgrid < 1) mgrid = 1;
  if (mgrid > 2048) mgrid = 2048;

  // metadata uses the value kind of x: the matrix kind, or f32 for a
  // dense x on a pattern matrix
  int xk = A->vk;
  if (xk == VK_PAT) xk = dense ? VK_F32 : VK_PAT;

  if (timing) SPMV_TRY(hipEventRecord(A->ev[0], s));
  if (dense) {
    if (xk == VK_BF16) hipLaunchKernelGGL(k_xmeta_dense<VK_BF16>, dim3(mgrid), dim3(KT), 0, s, o, x_dense);
    else hipLaunchKernelGGL(k_xmeta_dense<VK_F32>, dim3(mgrid), dim3(KT), 0, s, o, x_dense);
  } else {
    const int check = (int)A->opt[DBS_OPT_CHECK];
    const void *xv = sr == DBS_PLUS_TIMES ? x_val : nullptr;
    if (xk == VK_F32)
      hipLaunchKernelGGL(k_xmeta_sparse<VK_F32>, dim3(mgrid), dim3(KT), 0, s, o, nnz_x, x_idx, xv, A->xd, check);
    else if (xk == VK_BF16)
      hipLaunchKernelGGL(k_xmeta_sparse<VK_BF16>, dim3(mgrid), dim3(KT), 0, s, o, nnz_x, x_idx, xv, A->xd, check);
    else
      hipLaunchKernelGGL(k_xmeta_sparse<VK_PAT>, dim3(mgrid), dim3(KT), 0, s, o, nnz_x, x_idx, xv, A->xd, check);
  }
  SPMV_TRY(hipGetLastError());
  if (timing) SPMV_TRY(hipEventRecord(A->ev[1], s));

  SpmvParams P;
  P.t_cb = A->t_cb;
  P.t_meta = A->t_meta;
  P.cb_ptr = A->cb_ptr;
  P.csc_rb = A->csc_rb;
  P.csc2csr = A->csc2csr;
  P.payload = A->payload;
  P.dense_mask_off = A->dense_mask_off;
  P.segs = A->segs;
  P.nseg = A->nseg;
  P.m = A->m;
  P.nb = A->nb;
  P.xmask = A->xmask;
  P.epoch = A->epoch;
  P.xd = dense ? x_dense : A->xd;
  P.chunks = A->chunks;
  P.max_chunks = A->max_chunks;
  P.ctr = o.ctr;
  P.force_path = (int32_t)A->opt[DBS_OPT_PATH];
  P.th3_num = A->opt[DBS_OPT_TH3_NUM];
  P.th3_den = A->opt[DBS_OPT_TH3_DEN];
  P.local_cutoff = (int32_t)A->opt[DBS_OPT_LOCAL_PUSH_CUTOFF];
  P.y = y;
  const int64_t waves = A->nseg > A->max_chunks ? A->nseg : A->max_chunks;
  const unsigned grid = grid_for(waves, 2048);
  const int vk = A->vk;
  if (sr == DBS_OR_AND) {
    if (vk == VK_F32) launch_spmspv<VK_F32, DBS_OR_AND>(P, grid, s);
    else if (vk == VK_BF16) launch_spmspv<VK_BF16, DBS_OR_AND>(P, grid, s);
    else launch_spmspv<VK_PAT, DBS_OR_AND>(P, grid, s);
  } else {
    if (vk == VK_F32) launch_spmspv<VK_F32, DBS_PLUS_TIMES>(P, grid, s);
    else launch_spmspv<VK_BF16, DBS_PLUS_TIMES>(P, grid, s);
  }
  SPMV_TRY(hipGetLastError());
  if (timing) SPMV_TRY(hipEventRecord(A->ev[2], s));
  A->timing_pending = timing ? 1 : 0;
  A->cbuf ^= 1;
  A->last_stream = s;
  A->st.last_path = -2;  // resolved from the device counters by dbs_get_stats
  return DBS_OK;
}
