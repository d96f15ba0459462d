// Chunk-piece descriptor lists of the bf16 attention kernel: the 32-key tiles a work item
// visits, chunk by chunk, in the form the assembly loop reads with scalar loads.  Plain C++
// (host and device), so the CPU tests can build lists and run the loop's scalar code on them.
//
// A list is one descriptor per chunk its tile range touches, then a terminator, each of
// kPieceDescWords dwords:
//   0-1 K address of the piece's first tile     2-3 V address of it
//   4-5 K bytes between tiles                   6-7 V bytes between tiles
//   8-9 K address of the piece's last tile     10-11 V address of it
//   12  tiles to load                           13, 14  K, V row strides in bytes
//   15  rows the lane rows shift down (32 - len for a chunk shorter than a tile, else 0)
//   16  tiles to score                          17  first real row of the last tile
//   18  first real row of the other tiles       19  `extra`, the same in every descriptor
//   20-31 zero
// (The online-softmax loop takes its rescale slack, fp32 bits, from word 19.)
// Tile j of a chunk of len >= 32 keys holds the 32 keys from min(32 j, len - 32): the partial
// last tile is loaded as the chunk's last 32-key window, and its rows before 32 - rem (keys
// of the previous tile) are masked.  A chunk shorter than a tile is loaded with its keys in
// the tile's last len rows (the rows before them repeat its first key) and rows before
// 32 - len masked.  The terminator repeats the last tile's window for ever (the loads run
// ahead of the scores) with every key masked.  Every load stays inside its chunk.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define FIXEDM_PHD __host__ __device__
#else
#define FIXEDM_PHD
#endif

namespace fixedm {

constexpr int kPieceDescWords = 32;
constexpr uint32_t kPieceForever = 0x7fffffffu;

// One chunk as the list builder sees it: byte addresses of key row 0 of this (b, h) in K and
// V, row strides in elements (bf16), real keys.
struct PieceSrc {
  uint64_t kb, vb;
  int64_t k_ss, v_ss, len;
};

FIXEDM_PHD inline void piece_put_u64(uint32_t* d, int i, uint64_t x) {
  d[i] = (uint32_t)x;
  d[i + 1] = (uint32_t)(x >> 32);
}

// Writes the list of the tiles [v0, v1) of the chunks' tile sequence (the concatenation of
// each chunk's ceil(len / 32) tiles) to `out`; returns the number of pieces (0: an empty
// range, nothing written).  chunk(c) gives chunk c as a PieceSrc.
template <class ChunkAt>
FIXEDM_PHD inline int build_piece_list(uint32_t* out, ChunkAt chunk, int n_chunks, int64_t v0, int64_t v1,
                                       uint32_t extra) {
  constexpr int64_t kT = 32;
  int np = 0;
  int64_t vbase = 0;
  uint32_t d[kPieceDescWords];
  for (int c = 0; c < n_chunks; ++c) {
    const PieceSrc s = chunk(c);
    const int64_t nt = (s.len + kT - 1) / kT;
    const int64_t j0 = v0 - vbase > 0 ? v0 - vbase : 0;
    const int64_t j1 = v1 - vbase < nt ? v1 - vbase : nt;
    vbase += nt;
    if (j1 <= j0) continue;
    const uint64_t kss = (uint64_t)(2 * s.k_ss), vss = (uint64_t)(2 * s.v_ss);
    const int64_t r0 = s.len >= kT ? (j0 * kT < s.len - kT ? j0 * kT : s.len - kT) : 0;
    const int64_t r1 = s.len >= kT ? ((j1 - 1) * kT < s.len - kT ? (j1 - 1) * kT : s.len - kT) : 0;
    const int64_t n_full = s.len / kT, rem = s.len - n_full * kT;
    for (int i = 0; i < kPieceDescWords; ++i) d[i] = 0;
    piece_put_u64(d, 0, s.kb + (uint64_t)r0 * kss);
    piece_put_u64(d, 2, s.vb + (uint64_t)r0 * vss);
    piece_put_u64(d, 4, (uint64_t)kT * kss);
    piece_put_u64(d, 6, (uint64_t)kT * vss);
    piece_put_u64(d, 8, s.kb + (uint64_t)r1 * kss);
    piece_put_u64(d, 10, s.vb + (uint64_t)r1 * vss);
    d[12] = (uint32_t)(j1 - j0);
    d[13] = (uint32_t)kss;
    d[14] = (uint32_t)vss;
    d[15] = s.len < kT ? (uint32_t)(kT - s.len) : 0u;
    d[16] = (uint32_t)(j1 - j0);
    d[17] = j1 - 1 == n_full && rem > 0 ? (uint32_t)(kT - rem) : 0u;
    d[18] = 0;
    d[19] = extra;
    for (int i = 0; i < kPieceDescWords; ++i) out[np * kPieceDescWords + i] = d[i];
    ++np;
  }
  if (np == 0) return 0;
  // the terminator: the last tile's window again, never advancing, every key masked
  d[0] = d[8];
  d[1] = d[9];
  d[2] = d[10];
  d[3] = d[11];
  for (int i = 4; i < 8; ++i) d[i] = 0;
  d[12] = kPieceForever;
  d[16] = kPieceForever;
  d[17] = (uint32_t)kT;
  d[18] = (uint32_t)kT;
  for (int i = 0; i < kPieceDescWords; ++i) out[np * kPieceDescWords + i] = d[i];
  return np;
}

}  // namespace fixedm
