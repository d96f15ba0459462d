// The grid-tail split plan of the bf16 attention launch (host code; no HIP dependency, so the
// CPU tests build it with the host compiler).
#pragma once
#include <stdint.h>

namespace fixedm {

constexpr int kMaxParts = 8;             // key-range parts of a split tail tile (bf16 kernel)
constexpr int kMaxSplitTail = 255;       // most tail tiles that are split

// Grid-tail split of the bf16 attention launch.  The tiles fill whole rounds of one
// workgroup per compute unit; the remaining `tail` tiles would leave most CUs idle for a
// whole round, so each is cut into `parts` key ranges run by separate workgroups, whose
// partial sums the finalize merges.  parts minimises the expected end of the launch past
// its whole rounds, in tiles:
//   eps rounds + max(rounds / parts, tail / cus + min(drift, 1 / (2 parts)))
// with rounds = ceil(tail parts / cus), the parts a CU runs; eps the fixed cost of a work item
// (taking it, its set-up, the ring fill, the state store: ~24 key-tile steps, measured) over
// the tile's key tiles; and drift the spread of the CUs' finishing times after the whole
// rounds (the XCDs' clocks differ under load: ~2% of the elapsed rounds, measured), which the
// dynamic taking of the parts evens out down to about half a part.  Depends on the tile
// count, the run's key count and the CU count only, so every launch of a run and its finalize
// agree.
struct SplitPlan {
  int32_t n_whole, parts;
};
inline SplitPlan split_plan(int64_t tiles, int cus, int64_t key_tiles) {
  SplitPlan sp{(int32_t)tiles, 1};
  if (cus <= 0) return sp;
  const int64_t tail = tiles % cus;
  if (tail == 0 || tail > kMaxSplitTail) return sp;
  const double w = (double)tail / cus;
  const double drift = 0.02 * (double)(tiles / cus);
  const double eps = 24.0 / (double)(key_tiles > 1 ? key_tiles : 1);
  double best = 0.0;
  for (int p = 1; p <= kMaxParts; ++p) {
    const int64_t rounds = (tail * p + cus - 1) / cus;
    const double spread = drift < 0.5 / p ? drift : 0.5 / p;
    const double end = (double)rounds / p > w + spread ? (double)rounds / p : w + spread;
    const double cost = eps * (double)rounds + end;
    if (p == 1 || cost < best - 1e-9) { best = cost; sp.parts = p; }
  }
  if (sp.parts > 1) sp.n_whole = (int32_t)(tiles - tail);
  return sp;
}

}  // namespace fixedm
