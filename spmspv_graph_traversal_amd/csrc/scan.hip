// Device-wide exclusive scans and a stable LSD radix sort, used by the
// format builder (prefix sums of tile counts and payload sizes; the
// block-level CSC view is a stable sort of the tiles by column block).
#include "common.h"

namespace {

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ROUNDS = 8;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_ROUNDS;

// exclusive scan of one value per thread over a 256-thread block; returns the
// block total in `total`.
template <typename T>
__device__ T block_excl_scan(T v, T &total) {
  __shared__ T wsum[SCAN_THREADS / DBS_WAVE];
  const int lane = __lane_id();
  const int w = threadIdx.x / DBS_WAVE;
  T inc = v;
#pragma unroll
  for (int o = 1; o < DBS_WAVE; o <<= 1) {
    T t = __shfl_up(inc, o, DBS_WAVE);
    if (lane >= o) inc += t;
  }
  if (lane == DBS_WAVE - 1) wsum[w] = inc;
  __syncthreads();
  T pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < SCAN_THREADS / DBS_WAVE; ++i) {
    if (i < w) pre += wsum[i];
    tot += wsum[i];
  }
  __syncthreads();
  total = tot;
  return pre + inc - v;
}

template <typename T>
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_reduce(const T *in, int64_t n, T *part) {
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
  T s = 0;
  for (int i = 0; i < SCAN_ROUNDS; ++i) {
    int64_t k = base + (int64_t)i * SCAN_THREADS + threadIdx.x;
    if (k < n) s += in[k];
  }
  T tot;
  (void)block_excl_scan<T>(s, tot);
  if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

// single block: exclusive scan of the per-tile partials, in place
template <typename T>
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_partials(T *part, int64_t nblk) {
  T carry = 0;
  for (int64_t base = 0; base < nblk; base += SCAN_THREADS) {
    int64_t k = base + threadIdx.x;
    T v = k < nblk ? part[k] : (T)0;
    T tot;
    T ex = block_excl_scan<T>(v, tot);
    if (k < nblk) part[k] = carry + ex;
    carry += tot;
  }
}

template <typename T>
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_down(const T *in, T *out, int64_t n,
                                                            const T *part) {
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
  T carry = part[blockIdx.x];
  for (int i = 0; i < SCAN_ROUNDS; ++i) {
    int64_t k = base + (int64_t)i * SCAN_THREADS + threadIdx.x;
    T v = k < n ? in[k] : (T)0;
    T tot;
    T ex = block_excl_scan<T>(v, tot);
    if (k < n) out[k] = carry + ex;
    if (k == n - 1) out[n] = carry + ex + v;
    carry += tot;
  }
}

template <typename T>
__global__ void k_write_zero(T *p) { *p = 0; }

template <typename T>
hipError_t scan_impl(const T *in, T *out, int64_t n, void *tmp, hipStream_t s) {
  if (n <= 0) {
    hipLaunchKernelGGL(k_write_zero<T>, dim3(1), dim3(1), 0, s, out);
    return hipGetLastError();
  }
  const int64_t nblk = (n + SCAN_TILE - 1) / SCAN_TILE;
  T *part = (T *)tmp;
  hipLaunchKernelGGL(k_scan_reduce<T>, dim3((unsigned)nblk), dim3(SCAN_THREADS), 0, s, in, n, part);
  hipLaunchKernelGGL(k_scan_partials<T>, dim3(1), dim3(SCAN_THREADS), 0, s, part, nblk);
  hipLaunchKernelGGL(k_scan_down<T>, dim3((unsigned)nblk), dim3(SCAN_THREADS), 0, s, in, out, n,
                     (const T *)part);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort, 8-bit digits.  A 256-thread block owns 4096
// consecutive keys; ranks inside a block follow input order (wave ballots
// find lanes with equal digits), which keeps every pass stable.
// ---------------------------------------------------------------------------
constexpr int RS_THREADS = 256;
constexpr int RS_ROUNDS = 16;
constexpr int RS_TILE = RS_THREADS * RS_ROUNDS;

__global__ __launch_bounds__(RS_THREADS) void k_rs_hist(const uint32_t *keys, int64_t n, int shift,
                                                        uint32_t *hist, int64_t ntiles) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RS_TILE;
  for (int i = 0; i < RS_ROUNDS; ++i) {
    int64_t k = base + (int64_t)i * RS_THREADS + threadIdx.x;
    if (k < n) atomicAdd(&h[(keys[k] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * ntiles + blockIdx.x] = h[threadIdx.x];
}

__global__ __launch_bounds__(RS_THREADS) void k_rs_scatter(const uint32_t *keys, const uint32_t *vals,
                                                           uint32_t *keys_out, uint32_t *vals_out,
                                                           int64_t n, int shift, const uint32_t *hist,
                                                           int64_t ntiles) {
  __shared__ uint32_t run[256];
  __shared__ uint32_t wcnt[RS_THREADS / DBS_WAVE][256];
  const int t = threadIdx.x;
  const int w = t / DBS_WAVE;
  run[t] = hist[(int64_t)t * ntiles + blockIdx.x];
  const int64_t base = (int64_t)blockIdx.x * RS_TILE;
  const uint64_t lt = __lanemask_lt();
  for (int i = 0; i < RS_ROUNDS; ++i) {
    const int64_t k = base + (int64_t)i * RS_THREADS + t;
    const bool valid = k < n;
    const uint32_t key = valid ? keys[k] : 0u;
    const uint32_t d = (key >> shift) & 255u;
#pragma unroll
    for (int q = 0; q < RS_THREADS / DBS_WAVE; ++q) wcnt[q][t] = 0;
    __syncthreads();
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & lt);
    if (valid && rank == 0) wcnt[w][d] = (uint32_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t off = run[d];
      for (int q = 0; q < w; ++q) off += wcnt[q][d];
      keys_out[off + rank] = key;
      vals_out[off + rank] = vals[k];
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int q = 0; q < RS_THREADS / DBS_WAVE; ++q) add += wcnt[q][t];
    run[t] += add;
    __syncthreads();
  }
}

}  // namespace

size_t dbs_scan_tmp_bytes(int64_t n) {
  return (size_t)(((n + SCAN_TILE - 1) / SCAN_TILE) + 1) * sizeof(uint64_t);
}

hipError_t dbs_scan_u32(const uint32_t *in, uint32_t *out, int64_t n, void *tmp, hipStream_t s) {
  return scan_impl<uint32_t>(in, out, n, tmp, s);
}

hipError_t dbs_scan_u64(const uint64_t *in, uint64_t *out, int64_t n, void *tmp, hipStream_t s) {
  return scan_impl<uint64_t>(in, out, n, tmp, s);
}

size_t dbs_radix_tmp_bytes(int64_t n) {
  const int64_t ntiles = (n + RS_TILE - 1) / RS_TILE;
  const int64_t h = 256 * ntiles;
  return (size_t)(h + 1) * sizeof(uint32_t) + dbs_scan_tmp_bytes(h) + 256;
}

hipError_t dbs_radix_sort_pairs(uint32_t *keys, uint32_t *vals, uint32_t *keys_tmp,
                                uint32_t *vals_tmp, int64_t n, int bits, void *tmp,
                                hipStream_t s) {
  if (n <= 1 || bits <= 0) return hipSuccess;
  const int64_t ntiles = (n + RS_TILE - 1) / RS_TILE;
  const int64_t h = 256 * ntiles;
  uint32_t *hist = (uint32_t *)tmp;
  uint32_t *hscan = hist;  // scanned in place (out[h] lands one past the end)
  void *stmp = (void *)(((uintptr_t)(hist + h + 1) + 255) & ~(uintptr_t)255);
  uint32_t *ki = keys, *vi = vals, *ko = keys_tmp, *vo = vals_tmp;
  const int npass = (bits + 7) / 8;
  for (int p = 0; p < npass; ++p) {
    const int shift = 8 * p;
    hipLaunchKernelGGL(k_rs_hist, dim3((unsigned)ntiles), dim3(RS_THREADS), 0, s, ki, n, shift, hist,
                       ntiles);
    DBS_HIP_TRY(hipGetLastError());
    DBS_HIP_TRY(dbs_scan_u32(hist, hscan, h, stmp, s));
    hipLaunchKernelGGL(k_rs_scatter, dim3((unsigned)ntiles), dim3(RS_THREADS), 0, s, ki, vi, ko, vo,
                       n, shift, hscan, ntiles);
    DBS_HIP_TRY(hipGetLastError());
    uint32_t *t1 = ki, *t2 = vi;
    ki = ko;
    vi = vo;
    ko = t1;
    vo = t2;
  }
  if (ki != keys) {
    DBS_HIP_TRY(hipMemcpyAsync(keys, ki, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    DBS_HIP_TRY(hipMemcpyAsync(vals, vi, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
  }
  return hipSuccess;
}
