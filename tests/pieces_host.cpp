// Host build of the bf16 kernel's piece-list builder (dit_amd/csrc/pieces.h) for the CPU tests.
#include "pieces.h"

extern "C" int build_piece_list_host(uint32_t* out, const uint64_t* kb, const uint64_t* vb, const int64_t* k_ss,
                                     const int64_t* v_ss, const int64_t* len, int n, int64_t v0, int64_t v1,
                                     uint32_t extra) {
  fixedm::PieceSrc src[64];
  if (n > 64) return -1;
  for (int c = 0; c < n; ++c) src[c] = fixedm::PieceSrc{kb[c], vb[c], k_ss[c], v_ss[c], len[c]};
  return fixedm::build_piece_list(out, [&](int c) { return src[c]; }, n, v0, v1, extra);
}
