// Host build of the library's exact-sum accumulator (dit_amd/csrc/exact_sum.h) for the CPU
// tests: sums n fp64 values exactly and rounds once, normalising every 2^20 additions.
#include "exact_sum.h"

extern "C" double exact_sum_host(const double* x, int64_t n) {
  int64_t lim[fixedm::kLimbs] = {0};
  for (int64_t i = 0; i < n; ++i) {
    fixedm::exact_add(lim, x[i]);
    if ((i & ((1 << 20) - 1)) == (1 << 20) - 1) fixedm::exact_normalize(lim);
  }
  return fixedm::exact_round(lim);
}
