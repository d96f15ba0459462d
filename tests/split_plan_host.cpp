// Host build of the bf16 attention launch's grid-tail split plan (dit_amd/csrc/split_plan.h)
// for the CPU tests.
#include "split_plan.h"

extern "C" void split_plan_host(int64_t tiles, int cus, int64_t key_tiles, int32_t* n_whole, int32_t* parts) {
  const fixedm::SplitPlan sp = fixedm::split_plan(tiles, cus, key_tiles);
  *n_whole = sp.n_whole;
  *parts = sp.parts;
}

extern "C" int split_plan_max_parts() { return fixedm::kMaxParts; }
extern "C" int split_plan_max_tail() { return fixedm::kMaxSplitTail; }
