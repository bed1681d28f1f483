/*
 * All-core CPU baseline of the Boolean (OR-AND) pull: the same loop as
 * orc_or_and_pull in oracle.c (y_i = 1 iff row i holds an entry in an active
 * column; the plain definition of the product under the Boolean semiring,
 * "DB-SpMSpV" section 2.1, the pull form of Algorithm 1), with its rows split
 * over OpenMP threads.  Test and measurement infrastructure: only the
 * CPU-baseline leg of bench.py loads it; the library never does.  It shares
 * no code with the GPU path.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* threads an OpenMP parallel region uses here */
int orc_omp_threads(void) { return omp_get_max_threads(); }

int orc_or_and_pull_omp(int32_t m, int32_t n, const int32_t *row_ptr, const int32_t *col_idx, int32_t nnz_x,
                        const int32_t *x_idx, uint8_t *y) {
  unsigned char *act = (unsigned char *)calloc((size_t)n + 1, 1);
  if (!act) return -1;
  for (int32_t q = 0; q < nnz_x; ++q)
    if (x_idx[q] >= 0 && x_idx[q] < n) act[x_idx[q]] = 1;
#pragma omp parallel for schedule(dynamic, 4096)
  for (int32_t i = 0; i < m; ++i) {
    uint8_t f = 0;
    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1] && !f; ++k) f = act[col_idx[k]];
    y[i] = f;
  }
  free(act);
  return 0;
}
