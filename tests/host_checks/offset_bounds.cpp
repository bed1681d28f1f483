// Host-only check of the limits that keep the kernels' 32-bit buffer offsets
// in range (the library's common.h, compiled for the host only; no GPU).
//
// Claim: for every format the build accepts (dbs_format_fits_offsets) and
// every x a PLUS_TIMES call accepts (dbs_x_fits_offsets), the largest byte
// offset a kernel computes in 32-bit arithmetic stays below the out-of-range
// marker 0xFFFFFFF0 without wrapping, and the limits are tight: one more
// byte, tile or vector block is refused.
#include <stdio.h>

#include "../../spmspv_graph_traversal_amd/csrc/common.h"

static long failures = 0, checked = 0;
#define CHECK(c, ...)          \
  do {                         \
    ++checked;                 \
    if (!(c)) {                \
      ++failures;              \
      printf("FAIL " __VA_ARGS__); \
      printf("\n");            \
    }                          \
  } while (0)

int main() {
  const uint64_t L = 0xFFFFFFF0ull;
  // x staged block-padded: the largest offset is that of column 15 of the
  // last block, (cb * 16 + c) * vs computed in uint32
  for (uint32_t vs : {2u, 4u}) {
    const uint64_t nb_max = L / (16u * vs);
    for (uint64_t nb : {(uint64_t)1, (uint64_t)2, (uint64_t)1000, nb_max - 1, nb_max, nb_max + 1, (uint64_t)1 << 27}) {
      const bool ok = dbs_x_fits_offsets(nb, vs);
      CHECK(ok == (nb <= nb_max), "x limit nb=%llu vs=%u", (unsigned long long)nb, vs);
      if (ok) {
        const uint32_t cb = (uint32_t)(nb - 1), c = 15u;
        const uint32_t off32 = (cb * 16u + c) * vs;
        const uint64_t off64 = ((uint64_t)cb * 16u + c) * vs;
        CHECK(off32 == off64 && off64 + vs <= L, "x offset nb=%llu vs=%u", (unsigned long long)nb, vs);
      }
    }
  }
  // the format: the payload is read up to its slack (wide row loads that
  // start in the last tile), metadata at 8 * tile in uint32
  const uint64_t p_max = L - DBS_PAYLOAD_SLACK, t_max = L / 8u;
  for (uint64_t p : {(uint64_t)0, (uint64_t)1000, p_max - 1, p_max, p_max + 1, (uint64_t)1 << 32, (uint64_t)1 << 40})
    for (uint64_t t : {(uint64_t)0, (uint64_t)1, t_max - 1, t_max, t_max + 1}) {
      const bool ok = dbs_format_fits_offsets(p, t);
      CHECK(ok == (p <= p_max && t <= t_max), "format limit p=%llu t=%llu", (unsigned long long)p,
            (unsigned long long)t);
      if (ok) {
        CHECK(p + DBS_PAYLOAD_SLACK <= L, "payload end p=%llu", (unsigned long long)p);
        if (t > 0) {
          const uint32_t m32 = (uint32_t)(t - 1) * 8u;
          CHECK((uint64_t)m32 == (t - 1) * 8u && (t - 1) * 8u + 8u <= L, "meta offset t=%llu",
                (unsigned long long)t);
        }
      }
    }
  printf("%ld checks, %ld failures\n", checked, failures);
  return failures != 0;
}
