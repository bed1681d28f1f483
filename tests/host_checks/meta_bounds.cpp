// Host-only check of the arithmetic that keeps the push work lists in bounds
// (the library's meta.h, compiled for the host only; no GPU is used).
//
// Claim: for every vector-block count the registration can produce (at most
// 16 list entries per block when x_idx is not strictly increasing), every
// option setting and every number of vector blocks, the count the kernels use
// (nzblk_clamped) is at most nb, the list's capacity, and a call that pushes
// while enumerating its chunks from the list (push_from_list) has at most
// PUSH_LIST_MAX blocks, the capacity of the LDS prefix array.
#include <stdio.h>

#include "../../spmspv_graph_traversal_amd/csrc/meta.h"

int main() {
  using namespace dbs_meta;
  const int32_t nbs[] = {1, 2, 15, 16, 17, 63, 64, 65, 100, 101, 6143, 6144, 6145, 61440, 614399,
                         614400, 614401, 1 << 20, 134217727};
  const int64_t th3[][2] = {{1, 100}, {0, 1}, {1, 1}, {2, 1}, {3, 2}, {16, 1}, {1, 3}, {99, 100},
                            {(int64_t)1 << 31, 1}, {1, (int64_t)1 << 31}, {7, 1000}};
  long checked = 0, failures = 0;
  for (int32_t nb : nbs) {
    const uint64_t raws[] = {0u, 1u, (uint64_t)nb - 1, (uint64_t)nb, (uint64_t)nb + 1, 2ull * nb,
                             16ull * nb - 1, 16ull * nb, 6143u, 6144u, 6145u, 100000u};
    for (const auto &t : th3) {
      for (int32_t fp = 0; fp <= 2; ++fp) {
        const bool list = push_from_list(nb, fp, t[0], t[1]);
        for (uint64_t raw64 : raws) {
          if (raw64 > 16ull * (uint64_t)nb || raw64 > 0xFFFFFFFFull) continue;
          const uint32_t raw = (uint32_t)raw64;
          const uint32_t nz = nzblk_clamped(raw, nb);
          const bool push = selector_push(nz, nb, fp, t[0], t[1]);
          ++checked;
          if (nz > (uint32_t)nb) {
            ++failures;
            printf("FAIL clamp nb=%d raw=%u nz=%u\n", nb, raw, nz);
          }
          if (nz != (raw < (uint32_t)nb ? raw : (uint32_t)nb)) {
            ++failures;
            printf("FAIL clamp value nb=%d raw=%u nz=%u\n", nb, raw, nz);
          }
          if (push && list && nz > (uint32_t)PUSH_LIST_MAX) {
            ++failures;
            printf("FAIL list nb=%d fp=%d th3=%lld/%lld raw=%u nz=%u\n", nb, fp, (long long)t[0],
                   (long long)t[1], raw, nz);
          }
          // the selector is the strict rule of section 3.3.1
          const bool want = fp == 1 || (fp == 0 && (__int128)nz * t[1] < (__int128)nb * t[0]);
          if (push != want) {
            ++failures;
            printf("FAIL selector nb=%d fp=%d nz=%u\n", nb, fp, nz);
          }
        }
      }
    }
  }
  printf("checked %ld cases, %ld failures\n", checked, failures);
  return failures ? 1 : 0;
}
