// Streaming-read probe: the bandwidth a plain HIP kernel reaches when it
// reads device memory once with 16-byte loads and writes nothing, measured
// beside the published HBM peak (the yardstick for the byte-model roofline
// of the SpMSpV kernels).  Not part of the method.
#include "common.h"

namespace {

// Each thread XORs the 16-byte words i, i + stride, ... of the buffer, four
// loads in flight per iteration; the result is stored only when it equals a
// value the caller's data never folds to (so the loads stay live), in which
// case *sink receives it.
__global__ __launch_bounds__(256) void k_probe_read(const uint4 *__restrict__ p, int64_t n16, uint32_t *sink,
                                                     uint32_t never) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == never) *sink = acc;
}

}  // namespace

extern "C" dbs_status dbs_probe_read(const void *buf, int64_t bytes, uint32_t *sink, uint32_t never, void *stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0) return DBS_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return DBS_ERR_DEVICE;
  const int64_t n16 = bytes / 16;
  int64_t groups = (int64_t)cus * 8;  // eight 256-thread workgroups per CU
  const int64_t need = (n16 + 255) / 256;
  if (groups > need) groups = need;
  hipLaunchKernelGGL(k_probe_read, dim3((unsigned)groups), dim3(256), 0, (hipStream_t)stream, (const uint4 *)buf, n16,
                     sink, never);
  return hipGetLastError() == hipSuccess ? DBS_OK : DBS_ERR_DEVICE;
}
