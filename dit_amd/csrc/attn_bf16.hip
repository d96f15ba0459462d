// Fixed-m attention forward, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// Sources (page title, section):
//   [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention":
//        "Dropping the online max buys a better layout" (K-stationary scores, no P
//        transpose), "A static bound makes the ring reduction pure addition",
//        "Accumulate, then normalize once" (fp32 accumulator, init-or-add per ring step).
//   [FM] "feat(attention): fixed-m splash attention kernel with dynamic bounds and safety
//        fallbacks", Summary (subtract the precomputed shift m and accumulate numerator and
//        denominator directly in fp32; virtual K-centring through the per-row projection
//        q.k_mean; ragged KV tail without padding).
//   [UR] "feat(attention): 2D Ulysses+Ring attention with Global Virtual K-Centering",
//        Summary (ineligible blocks take online softmax for the whole ring).
//
// Design (MI355X):
//   * Workgroup = 4 waves x 64 query rows = 256 rows of one (b, h).  Each wave keeps its 64
//     query rows resident in VGPRs as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16).
//   * In the 32x32 accumulator layout each lane owns ONE query column and 16 keys, so the
//     fixed-m exponent e = alpha*S - (m + c_i) is one FMA with a per-lane constant, the
//     row sum is a per-lane running fp32 sum of the fp32 probabilities, and the exp2'd
//     scores, packed to bf16, are
//     already the B operand of O^T += V^T P^T with no transpose (the K-stationary layout of
//     [CM]).  The matching key order on the V^T operand comes from the gfx950 LDS transpose
//     read ds_read_b64_tr_b16.
//   * K/V tiles of 32 keys stream through an 8-stage LDS ring (K ring in the first 64 KB,
//     V ring in the next 64 KB) with direct global->LDS loads (global_load_lds_dwordx4)
//     issued six tiles ahead; no VGPR staging.  Tiles are XOR-swizzled so both the K row
//     reads and the V transpose reads are bank-conflict free.  The main loop is unrolled
//     over the 8 stages, so every LDS address is a per-lane base plus an immediate.
//   * Fixed-m body, software-pipelined per 32-key tile t: the MFMAs of O += V(t-1) P(t-1)
//     are independent of the VALU work exp2(alpha S(t) - shift), so the matrix cores and
//     the vector ALUs overlap within one wave.
//   * The body is chosen per wave from its q-block's eligibility byte and bound U: the
//     fixed-m assembly loop on bf16(alpha q) (U <= kR17MaxU), the fixed-m assembly loop that
//     applies alpha in fp32 (eligible, U above it), or online softmax (ineligible).  A
//     wave-uniform branch.
//   * One launch folds one K/V chunk (one ring step) into the workspace.
//   * Ragged KV tails: rows past a chunk's end are clamped to its last row on load and
//     their probabilities forced to zero; no padding copies.  Query rows past Sq are
//     clamped on load and land in padded workspace rows that finalize never reads.
//   * Persistent workgroups (one per compute unit) take query tiles from per-XCD queues:
//     each XCD works through consecutive tiles of the same heads (sharing the K/V stream in
//     its L2) and, once its queue is empty, takes work from the back of the others.
#include <math.h>

#include "fixedm_internal.h"

namespace fixedm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kD = 128;
constexpr int kKT = 32;                        // keys per pipeline tile
constexpr int kRowBytes = kD * 2;              // 256 bytes per key row
constexpr int kTileBytes = kKT * kRowBytes;    // 8 KB: K (or V) of one tile
constexpr int kStages = 8;                     // LDS ring depth in tiles
constexpr int kAhead = kStages - 2;            // tiles in flight ahead of the current one
constexpr int kLoadsPerTile = 4;               // global->LDS instructions per wave per tile
constexpr int kVRing = kStages * kTileBytes;   // the V ring starts after the K ring
constexpr int kLdsBytes = 2 * kStages * kTileBytes;   // 128 KB
// Largest block bound U for which the fixed-m body takes its logits from bf16(alpha q).  The
// rounding (relative <= 2^-8 per element) moves a base-2 logit by at most 2^-8 sum_d
// |alpha q_d k_d| <= 2^-8 U; in practice the moves are random and far smaller, and up to
// U = 20 they add about 1e-3 at most to the output error of the bf16 probabilities (sharp
// rows over 64 keys), while above it they grow with U.  Blocks above it apply alpha in fp32.
constexpr double kR17MaxU = 20.0;

// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence __syncthreads() adds: the ring's prefetch
// loads must stay in flight across it.  LDS visibility is ensured by the explicit vmcnt
// wait that precedes every barrier.
__device__ inline void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One 16-byte-per-lane global->LDS load of a tile row's chunk: lane L's 16 bytes come from
// sbase + max(row - rsh, 0) * stride + chunk and land at LDS byte lds + 16 L.  Written as
// inline asm so the compiler's wait-count pass does not treat every later LDS read as
// aliasing an in-flight load (it would insert vmcnt(0) and drain the ring); the ring's vmcnt
// waits are explicit instead.  The lane offset is formed inside the block from loop-invariant
// inputs: the compiler takes a register an asm load reads as busy until the load completes,
// so rewriting a register that holds an offset would make it wait on the vector memory
// counter (which also counts the ring's loads) and drain the ring.  The destination is passed
// as an LDS pointer (with a memory clobber) so the compiler knows the asm writes the shared
// buffer.  M0 carries the wave-uniform LDS address; no compiler-generated instruction here
// reads M0.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ inline void dma16_row(uint32_t row, uint32_t chunk, uint32_t rsh, uint32_t stride, uint64_t sbase,
                                 lds_u8* lds) {
  uint32_t off;
  asm volatile(
      "v_subrev_u32 %0, %3, %1\n\t"
      "v_max_i32 %0, 0, %0\n\t"
      "v_mul_lo_u32 %0, %0, %4\n\t"
      "v_add_u32 %0, %0, %2\n\t"
      "s_mov_b32 m0, %5\n\t"
      "global_load_lds_dwordx4 %0, %6"
      : "=&v"(off)
      : "v"(row), "v"(chunk), "s"(rsh), "s"(stride), "s"(lds), "s"(sbase)
      : "memory");
}

__device__ inline uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// LDS read offsets of this lane in stage 0: the K fragment rows of k-steps 0..7 and the V^T
// transpose reads of dim tiles 0..3 (XOR-swizzled like the DMA placement below).
struct LdsOff {
  uint32_t koff[8];
  uint32_t voff[4];
};
__device__ inline LdsOff lds_offsets(int lane) {
  LdsOff g;
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, j = lane & 15, dhalf = grp & 1;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) g.koff[kk] = (uint32_t)(lq * kRowBytes + (((2 * kk + hh) ^ (lq & 15)) << 4));
  const int r0 = 4 * hh + (j >> 2);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int chunk = 4 * m + 2 * dhalf + ((j & 3) >> 1);
    g.voff[m] = (uint32_t)(kVRing + r0 * kRowBytes + ((chunk ^ ((r0 & 3) << 2)) << 4) + (j & 1) * 8);
  }
  return g;
}

// This lane's part of a tile load: lane L of DMA instruction i (0, 1) of wave w writes row
// 4 (2 w + i) + L / 16 of the tile at physical 16-byte chunk L % 16, and fetches the logical
// chunk the swizzle puts there (K: phys ^ (row & 15), V: phys ^ ((row & 3) << 2)).  ck / cv
// are those chunks' byte offsets in the row.
struct DmaLane {
  uint32_t row[2], ck[2], cv[2];
};
__device__ inline DmaLane dma_lane(int wave, int lane) {
  DmaLane d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 4 * (2 * wave + i) + (lane >> 4), phys = lane & 15;
    d.row[i] = (uint32_t)row;
    d.ck[i] = (uint32_t)(16 * (phys ^ (row & 15)));
    d.cv[i] = (uint32_t)(16 * (phys ^ ((row & 3) << 2)));
  }
  return d;
}

// The key tiles of one work item are the 32-key tiles of its chunk pieces in order, read
// from a piece descriptor list (pieces.h) that the prep kernel writes before each launch.
// The lists are read through the constant address space, so the reads are scalar loads:
// a vector load here would make the compiler wait on the vector memory counter, which also
// counts the ring's loads in flight, and drain the ring.
typedef __attribute__((address_space(4))) const uint32_t desc_word;
__device__ inline uint32_t desc_at(const uint32_t* d, int i) { return ((const desc_word*)d)[i]; }
__device__ inline uint64_t desc_u64(const uint32_t* d, int i) {
  return ((uint64_t)desc_at(d, i + 1) << 32) | desc_at(d, i);
}

// Load side of the ring as the compiled body runs it (the assembly loop keeps the same
// cursor in SGPRs): the next tile's addresses, the tiles left in the piece, this lane's
// offsets into the piece's rows.
struct DmaCursor {
  const uint32_t* d;
  uint64_t kt, vt, ktile, vtile, klast, vlast;
  uint32_t rem, kss, vss, rsh;
};
__device__ inline void dma_load(DmaCursor& c) {
  const uint32_t* d = c.d;
  c.kt = desc_u64(d, 0);
  c.vt = desc_u64(d, 2);
  c.ktile = desc_u64(d, 4);
  c.vtile = desc_u64(d, 6);
  c.klast = desc_u64(d, 8);
  c.vlast = desc_u64(d, 10);
  c.rem = desc_at(d, 12);
  c.kss = desc_at(d, 13);
  c.vss = desc_at(d, 14);
  c.rsh = desc_at(d, 15);
}
// Issues this wave's share of the next tile (2 KB of K rows, 2 KB of V rows) into LDS stage
// `stage`, then advances: the piece's last tile is its last window, and past the piece's
// end the cursor moves to the next descriptor.
__device__ __attribute__((always_inline)) void dma_next(uint8_t* smem, DmaCursor& c, const DmaLane& ln, int wave,
                                                        int stage) {
  lds_u8* kl = (lds_u8*)(smem + stage * kTileBytes);
  lds_u8* vl = (lds_u8*)(smem + kVRing + stage * kTileBytes);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = __builtin_amdgcn_readfirstlane(1024 * (2 * wave + i));
    dma16_row(ln.row[i], ln.ck[i], c.rsh, c.kss, c.kt, kl + blk);
    dma16_row(ln.row[i], ln.cv[i], c.rsh, c.vss, c.vt, vl + blk);
  }
  c.kt += c.ktile;
  c.vt += c.vtile;
  if (--c.rem == 1) {
    c.kt = c.klast;
    c.vt = c.vlast;
  } else if (c.rem == 0) {
    c.d += kPieceWords;
    dma_load(c);
  }
}

// Score side: the first real row of each tile in turn.
struct MaskCursor {
  const uint32_t* d;
  uint32_t rem, lo_last, lo_base;
};
__device__ inline void mask_load(MaskCursor& m) {
  m.rem = desc_at(m.d, 16);
  m.lo_last = desc_at(m.d, 17);
  m.lo_base = desc_at(m.d, 18);
}
__device__ inline int mask_next(MaskCursor& m) {
  const int lo = (int)(m.rem == 1 ? m.lo_last : m.lo_base);
  if (--m.rem == 0) {
    m.d += kPieceWords;
    mask_load(m);
  }
  return lo;
}

// Key index within the tile held by accumulator register r of this lane.
__device__ inline int tile_key(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// S^T(tile) = K(tile) Q^T for one 32-key tile and two 32-query tiles: 16 MFMAs.  Rows of the
// tile before `lo` (keys that are not real) start from -inf (p = 0), the others from 0.
__device__ __attribute__((always_inline)) void compute_s(const uint8_t* smem, const LdsOff& g, int stage,
                                                         const bf16x8 (&qf)[2][8], f32x16 (&s)[2], int lo,
                                                         int hh) {
  const uint8_t* ks = smem + stage * kTileBytes;
  bf16x8 kf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(ks + g.koff[kk]);
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = tile_key(r, hh) >= lo ? 0.0f : -INFINITY;
  s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0][0], c, 0, 0, 0);
  s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[1][0], c, 0, 0, 0);
#pragma unroll
  for (int kk = 1; kk < 8; ++kk) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[0][kk], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[1][kk], s[1], 0, 0, 0);
  }
}

// O^T += V(tile)^T P(tile)^T: four 32-dim tiles x two 16-key steps x two query tiles.  For
// each 16-key step st and 32-dim tile m a lane holds one dim and 8 keys in the P register
// order, from two LDS transpose reads (each 4 keys x 16 dims to a 16-lane group).
__device__ __attribute__((always_inline)) void compute_pv(const uint8_t* smem, const LdsOff& g, int stage,
                                                          const bf16x8 (&p)[2][2], f32x16 (&o)[2][4]) {
  const uint8_t* vs = smem + stage * kTileBytes;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint8_t* a0 = vs + g.voff[m] + 4096 * st;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 2048));
      const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[0][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[0][st], o[0][m], 0, 0, 0);
      o[1][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[1][st], o[1][m], 0, 0, 0);
    }
  }
}

// The fixed-m pass of a work item, written out instruction by instruction (generated).
#include "fixed_loop.inc"

// Packs 8 probabilities to bf16 (round to nearest even; the B operand of the PV product)
// and adds the fp32 probabilities to the row sum, key by key.
__device__ __attribute__((always_inline)) bf16x8 pack8_sum(const f32x16& e, int base, float& lsum) {
  bf16x2 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = __builtin_convertvector((f32x2){e[base + 2 * i], e[base + 2 * i + 1]}, bf16x2);
    lsum += e[base + 2 * i];
    lsum += e[base + 2 * i + 1];
  }
  bf16x8 r;
  __builtin_memcpy(&r, w, 16);
  return r;
}

// Online-softmax probabilities of one tile (the fallback body).  The running reference r of
// each query row (base 2) is raised to the row's max only when some row of the wave's query
// tile exceeds its r by more than kRescaleSlack; the accumulator and the row sum are then
// rescaled by 2^(r_old - r_new) (one wave-uniform branch).  Between raises the probabilities
// 2^(alpha s - r) stay below 2^kRescaleSlack, well inside the bf16 and fp32 ranges, and O / l
// does not depend on which r was used, so most tiles skip the 64 accumulator multiplies.
// Masked rows arrive as -inf scores (every tile this body visits has at least one real key).
constexpr float kRescaleSlack = 8.0f;
__device__ __attribute__((always_inline)) void softmax_online(const f32x16 (&s)[2], bf16x8 (&p)[2][2],
                                                              float (&lsum)[2], float (&rmax)[2],
                                                              f32x16 (&o)[2][4], float alpha) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[n][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float am = alpha * mx;
    if (__builtin_amdgcn_ballot_w64(am > rmax[n] + kRescaleSlack) != 0) {
      const float rn = fmaxf(rmax[n], am);
      const float f = __builtin_amdgcn_exp2f(rmax[n] - rn);
      rmax[n] = rn;
      lsum[n] *= f;
#pragma unroll
      for (int m = 0; m < 4; ++m) o[n][m] *= f;
    }
    f32x16 e;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(alpha, s[n][r], -rmax[n]));
    p[n][0] = pack8_sum(e, 0, lsum[n]);
    p[n][1] = pack8_sum(e, 8, lsum[n]);
  }
}

// The online-softmax pass of a work item (the fallback body), on the same ring as the
// assembly loop: the prologue's six tile loads and barrier, then per tile t a barrier
// (tile t+1 landed, stage t-2 free), the load of tile t+6, and the tile's scores,
// probabilities and PV product; then one more barrier and load for the assembly loop's
// step t = n_tiles.  The waves of a workgroup thus meet at the same barriers and load the
// same tiles whichever body each runs.
__device__ __attribute__((always_inline)) void run_online(const AttnArgs& a, uint8_t* smem, const uint32_t* pieces,
                                                          int n_tiles, const bf16x8 (&qf)[2][8], f32x16 (&o)[2][4],
                                                          float (&lsum)[2], float (&rmax)[2], int wave, int lane) {
  const int hh = lane >> 5;
  const LdsOff g = lds_offsets(lane);
  const DmaLane ln = dma_lane(wave, lane);
  // The compiler does not count the ring's loads (inline asm): a vector memory access of its
  // own still in flight when the loop starts (a spill reload, say) would make it wait on the
  // counter inside the loop, every iteration, and drain the ring.  Waiting here, before the
  // first ring load, leaves it nothing to wait for.
  wait_vmcnt<0>();
  DmaCursor dc;
  dc.d = pieces;
  dma_load(dc);
  MaskCursor mc;
  mc.d = pieces;
  mask_load(mc);
#pragma unroll 1
  for (int t = 0; t < kAhead; ++t) dma_next(smem, dc, ln, wave, t);
  wait_vmcnt<(kAhead - 1) * kLoadsPerTile>();   // tile 0 has landed (this wave's part)
  barrier();
#pragma unroll 1
  for (int t = 0; t <= n_tiles; ++t) {
    wait_vmcnt<(kAhead - 2) * kLoadsPerTile>();
    barrier();
    dma_next(smem, dc, ln, wave, (t + kAhead) % kStages);
    if (t == n_tiles) break;
    const int stage = t % kStages;
    f32x16 s[2];
    bf16x8 p[2][2];
    compute_s(smem, g, stage, qf, s, mask_next(mc), hh);
    softmax_online(s, p, lsum, rmax, o, a.alpha);
    compute_pv(smem, g, stage, p, o);
  }
}

// The fixed-m pass of a work item: the assembly loop, with bf16(alpha q) fragments (r17) or
// with the logit factor applied in fp32.
__device__ __attribute__((always_inline)) void run_fixed(const AttnArgs& a, uint8_t* smem, const uint32_t* pieces,
                                                         int n_tiles, const bf16x8 (&qf)[2][8], f32x16 (&o)[2][4],
                                                         float (&lsum)[2], const float (&shift)[2], bool r17,
                                                         int wave, int lane) {
  // The lane's offsets are formed from an id the compiler cannot hoist above the assembly
  // block, so they are not kept live (and spilled) around it.
  int tid = wave * 64 + lane;
  asm volatile("" : "+v"(tid));
  const int w = tid >> 6, l = tid & 63;
  const LdsOff g = lds_offsets(l);
  const DmaLane ln = dma_lane(w, l);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_u8*)smem;
  uint32_t koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = lds0 + g.koff[kk];
#pragma unroll
  for (int m = 0; m < 4; ++m) voff[m] = lds0 + g.voff[m];
  const uint32_t lane6[6] = {ln.row[0], ln.row[1], ln.ck[0], ln.ck[1], ln.cv[0], ln.cv[1]};
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds0 + 2048 * w);
  const float nshift[2] = {-shift[0], -shift[1]};
  const uint64_t list = uniform_u64((uint64_t)(uintptr_t)pieces);
  const uint32_t nt = __builtin_amdgcn_readfirstlane((uint32_t)n_tiles);
  if (r17)
    fixed_loop_asm(o, qf, lsum, nshift, koff, voff, lane6, (uint32_t)(4 * (l >> 5)), list, nt, lds_wave);
  else
    fixed_loop_fp32a_asm(o, qf, lsum, nshift, koff, voff, lane6, (uint32_t)(4 * (l >> 5)), list, nt, lds_wave,
                         a.alpha);
}

// One work item: a whole query tile (all tiles of the launch's chunks), or part p of a split
// tail tile: the launch's key tiles [T p / parts, T (p + 1) / parts) (T tiles in all).
__device__ __attribute__((always_inline)) void process_item(const AttnArgs& a, uint8_t* smem, int tile,
                                                            int part) {
  const bool split = a.parts > 1 && tile >= a.n_whole;
  const int64_t T = a.call_tiles;
  const int n_tiles = split ? (int)(T * (part + 1) / a.parts - T * part / a.parts) : (int)T;
  const int qt = tile % a.n_qtiles;
  const int bh = tile / a.n_qtiles;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hh = lane >> 5;
  const int q0 = qt * kQTile + wave * 64;
  const int qlast = q0 < a.Sq ? q0 : a.Sq - 1;
  const int beta = qlast / a.q_block;
  const int64_t bq = (int64_t)bh * a.nqb + beta;
  // The body is chosen per wave: make the choice visibly wave-uniform (a scalar branch), so
  // no wave steps through the other body's code with an empty exec mask (that code holds
  // barriers and assembly that keeps its state in fixed registers).
  const bool fixed = __builtin_amdgcn_readfirstlane((int)a.elig[bq]) != 0;
  const int mshift = __builtin_amdgcn_readfirstlane(a.m[bq]);
  // Eligible blocks with a bound above kR17MaxU take the fixed-m body with the logit factor
  // applied in fp32: the rounding of bf16(alpha q) moves a base-2 logit by up to 2^-8 U.
  const bool r17 = fixed && __builtin_amdgcn_readfirstlane((int)(a.u[bq] <= kR17MaxU)) != 0;

  // resident query fragments (B operand of S^T = K Q^T) and the centring term q . k_mean.
  // The fixed-m assembly body takes its logits in base 2 straight from the MFMA: its query
  // fragments are bf16(alpha q) (fp32 product, one rounding: the base-2 rescale of Q that the
  // TPU path folds into Q's producer, [FM] Summary "Relayout optimization", bit-identical
  // there by the [UR] review thread) and c_i = (alpha q_i) . k_mean.  The other two bodies
  // keep q and scale their scores by alpha in fp32 (c_i = alpha (q_i . k_mean)).
  bf16x8 qf[2][8];
  float cdot[2];
  const float* km = a.k_mean + (int64_t)bh * kD;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    int row = q0 + 32 * n + lq;
    if (row >= a.Sq) row = a.Sq - 1;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + b * a.q_sb + (int64_t)row * a.q_ss + h * a.q_sh;
    float dot = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * kk + 8 * hh);
      uint32_t u[4] = {w.x, w.y, w.z, w.w};
      if (r17) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2 x = {__uint_as_float(u[i] << 16) * a.alpha, __uint_as_float(u[i] & 0xffff0000u) * a.alpha};
          const bf16x2 y = __builtin_convertvector(x, bf16x2);
          __builtin_memcpy(&u[i], &y, 4);
        }
      }
      __builtin_memcpy(&qf[n][kk], u, 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dot = __builtin_fmaf(__uint_as_float(u[i] << 16), km[16 * kk + 8 * hh + 2 * i], dot);
        dot = __builtin_fmaf(__uint_as_float(u[i] & 0xffff0000u), km[16 * kk + 8 * hh + 2 * i + 1], dot);
      }
    }
    // q . k_mean: this half's dims plus the other half's, low half first on both lanes; the
    // assembly body's fragments already carry alpha, the fp32-factor body applies it here
    const float other = __shfl_xor(dot, 32, 64);
    cdot[n] = hh == 0 ? dot + other : other + dot;
    if (!r17) cdot[n] *= a.alpha;
  }
  // The query fragments are read only as MFMA B operands, which may sit in accumulation
  // registers: pin them there so the 256 architectural VGPRs hold S, P and the K/V
  // fragments of the pipeline.
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+a"(qf[n][kk]));

  f32x16 o[2][4];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) o[n][m] = f32x16{};
  float lsum[2] = {0.0f, 0.0f};
  float shift[2];
  if (fixed) {
    // the fixed shift: the q-block's m, or (per-row shifts) each query row's own m
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      int mm = mshift;
      if (a.m_row != nullptr) {
        const int row = q0 + 32 * n + lq < a.Sq ? q0 + 32 * n + lq : a.Sq - 1;
        mm = a.m_row[(int64_t)bh * a.Sq + row];
      }
      shift[n] = (float)mm + cdot[n];
    }
  } else {
    shift[0] = shift[1] = -INFINITY;
  }
  if (n_tiles > 0) {
    const uint32_t* pieces = a.ptable + ((int64_t)bh * kPieceLists + (split ? 1 + part : 0)) * kPieceSlots * kPieceWords;
    if (fixed) run_fixed(a, smem, pieces, n_tiles, qf, o, lsum, shift, r17, wave, lane);
    else run_online(a, smem, pieces, n_tiles, qf, o, lsum, shift, wave, lane);
    wait_vmcnt<0>();   // the ring's trailing loads land before the workgroup's LDS is reused
    barrier();
  }

  if (a.final_out && !split) {
    // The run ends with this launch: merge the workspace's earlier keys (if any), normalise
    // once ([CM] "Accumulate, then normalize once") and write O, and lse, straight from the
    // accumulator registers.  The arithmetic is the finalize kernel's: O = acc / l (IEEE
    // division), bf16 by round-to-nearest-even, lse = ln 2 (r + log2 l).
    const int64_t tb = (int64_t)tile * (kQTile * kD);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const float other = __shfl_xor(lsum[n], 32, 64);
      const float ltot = hh == 0 ? lsum[n] + other : other + lsum[n];
      const int64_t rowi = (int64_t)bh * a.sq_pad + q0 + 32 * n + lq;
      float lnew = ltot, rnew = shift[n], fw = 0.0f, fo = 1.0f;
      if (a.accumulate) {
        const float lp = a.l[rowi], rp = a.r[rowi];
        if (fixed) {
          lnew = lp + ltot;
          fw = 1.0f;
        } else {
          rnew = fmaxf(rp, shift[n]);
          fw = rp == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(rp - rnew);
          fo = shift[n] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(shift[n] - rnew);
          lnew = lp * fw + ltot * fo;
        }
      }
      const int q = q0 + 32 * n + lq;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x4 v = {o[n][m][4 * jj], o[n][m][4 * jj + 1], o[n][m][4 * jj + 2], o[n][m][4 * jj + 3]};
          if (a.accumulate) {
            const f32x4 prev =
                *reinterpret_cast<const f32x4*>(a.acc + tb + ((((wave * 2 + n) * 4 + m) * 4 + jj) * 64 + lane) * 4);
            if (fixed) v = prev + v;
            else v = prev * fw + v * fo;
          }
          if (q < a.Sq) {
            const int64_t off = b * a.o_sb + (int64_t)q * a.o_ss + h * a.o_sh + 32 * m + 8 * jj + 4 * hh;
            const float x0 = __fdiv_rn(v[0], lnew), x1 = __fdiv_rn(v[1], lnew);
            const float x2 = __fdiv_rn(v[2], lnew), x3 = __fdiv_rn(v[3], lnew);
            if (a.out_dtype == FIXEDM_F32) {
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + off) = f32x4{x0, x1, x2, x3};
            } else {
              uint2 w;
              w.x = bf16_rne(x0) | (bf16_rne(x1) << 16);
              w.y = bf16_rne(x2) | (bf16_rne(x3) << 16);
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + off) = w;
            }
          }
        }
      }
      if (a.lse != nullptr && hh == 0 && q < a.Sq) a.lse[(int64_t)bh * a.Sq + q] = lse_of(rnew, lnew);
    }
    return;
  }

  // ---- fold into the workspace: acc in register order (one 1 KB coalesced float4 store
  // per (wave, n, m, j)), l and r per padded query row (parts 1.. of a split tile: their own
  // slots).  The first visit of a run writes; later visits add (fixed-m: pure addition) or
  // rescale-merge (online softmax; a part that has seen no key yet holds r = -inf, l = 0).
  float* acc_t = a.acc;
  float* l_t = a.l;
  float* r_t = a.r;
  int64_t tb = (int64_t)tile * (kQTile * kD);
  int64_t row0 = (int64_t)bh * a.sq_pad + q0;
  if (part > 0) {
    const int64_t u = (int64_t)(tile - a.n_whole) * (a.parts - 1) + part - 1;
    acc_t = a.acc_x;
    l_t = a.l_x;
    r_t = a.r_x;
    tb = u * (kQTile * kD);
    row0 = u * kQTile + wave * 64;
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const float other = __shfl_xor(lsum[n], 32, 64);
    const float ltot = hh == 0 ? lsum[n] + other : other + lsum[n];
    const int64_t rowi = row0 + 32 * n + lq;
    float lnew = ltot, rnew = shift[n], fw = 0.0f, fo = 1.0f;
    if (a.accumulate) {
      const float lp = l_t[rowi], rp = r_t[rowi];
      if (fixed) {
        lnew = lp + ltot;
        fw = 1.0f;
      } else {
        rnew = fmaxf(rp, shift[n]);
        fw = rp == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(rp - rnew);
        fo = shift[n] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(shift[n] - rnew);
        lnew = lp * fw + ltot * fo;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4* dst = reinterpret_cast<f32x4*>(acc_t + tb + ((((wave * 2 + n) * 4 + m) * 4 + jj) * 64 + lane) * 4);
        f32x4 v = {o[n][m][4 * jj], o[n][m][4 * jj + 1], o[n][m][4 * jj + 2], o[n][m][4 * jj + 3]};
        if (a.accumulate) {
          const f32x4 prev = *dst;
          if (fixed) v = prev + v;
          else v = prev * fw + v * fo;
        }
        *dst = v;
      }
    }
    if (hh == 0) {
      l_t[rowi] = lnew;
      r_t[rowi] = rnew;
    }
  }
}

// Work items: the n_whole whole tiles, then the split parts (tile n_whole + u / parts, part
// u % parts).  They are dealt to kQueues queues, one per XCD: queue x holds whole tiles
// [x W / 8, (x + 1) W / 8) followed by parts [x P / 8, (x + 1) P / 8), so each XCD works
// through consecutive tiles of the same heads and shares their K/V stream in its L2.  A
// queue is one counter of items taken from its front, by its own XCD and, once their own
// queues are empty, by the others.  It only grows and every take returns the count before
// its own increment, so exactly `size` takes succeed: each item is processed once.  The
// XCDs run at different clocks under load, and a few slow tiles hold some compute units
// for a long time, so stealing keeps every XCD busy to the end; stealing from the front
// (the largest items left) rather than the back leaves the split parts, the smallest items,
// for last everywhere (taking parts from the back measured a 1.1 ms spread of XCD end times
// against 0.4 ms with 1% of the tiles on the online body).
constexpr int kQueues = 8;

struct QueueRange {
  int64_t w0, nw, p0, size;
};
__device__ inline QueueRange queue_range(const AttnArgs& a, int q) {
  const int64_t W = a.n_whole, P = (int64_t)(a.B * a.H * a.n_qtiles - a.n_whole) * a.parts;
  QueueRange r;
  r.w0 = W * q / kQueues;
  r.nw = W * (q + 1) / kQueues - r.w0;
  r.p0 = P * q / kQueues;
  r.size = r.nw + P * (q + 1) / kQueues - r.p0;
  return r;
}

// Whole tiles with a wave on the online-softmax body (an ineligible q-block) take ~3x as long
// as fixed-m ones at the same clock; taken late, one of them would end the launch well after
// the rest.  They are therefore taken first: the prep kernel lists them (queue[kSlowCount]
// entries in slow_list), every workgroup drains that list before its queues (queue[kSlowTaken]
// counts takes), and queue takes skip them.
constexpr int kSlowCount = kQueues, kSlowTaken = kQueues + 1;

__device__ inline bool tile_is_slow(const AttnArgs& a, int64_t tile) {
  const int64_t bh = tile / a.n_qtiles;
  const int qt = (int)(tile % a.n_qtiles);
  for (int w = 0; w < 4; ++w) {
    const int q0 = qt * kQTile + 64 * w;
    const int beta = (q0 < a.Sq ? q0 : a.Sq - 1) / a.q_block;
    if (a.elig[bh * a.nqb + beta] == 0) return true;
  }
  return false;
}

// Takes the next item for a workgroup on XCD `xcc` (one thread calls it): a listed slow tile,
// else the front of its own queue, else the front of the others in turn.  `dead` marks
// queues seen empty (bit kQueues: the slow list).  -1: none left.
__device__ inline int64_t take_item(const AttnArgs& a, int xcc, uint32_t& dead) {
  if (!((dead >> kQueues) & 1u)) {
    const unsigned long long n_slow = __hip_atomic_load(a.queue + kSlowCount, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long i = n_slow > 0 ? atomicAdd(a.queue + kSlowTaken, 1ull) : n_slow;
    if (i < n_slow) return a.slow_list[i];
    dead |= 1u << kQueues;
  }
  for (int k = 0; k < kQueues; ++k) {
    const int q = (xcc + k) % kQueues;
    if ((dead >> q) & 1u) continue;
    const QueueRange r = queue_range(a, q);
    const int64_t j = (int64_t)atomicAdd(a.queue + q, 1ull);
    if (j >= r.size) {
      dead |= 1u << q;
      continue;
    }
    if (j < r.nw && tile_is_slow(a, r.w0 + j)) {   // listed: taken from the slow list
      --k;                                          // this queue again
      continue;
    }
    return j < r.nw ? r.w0 + j : a.n_whole + r.p0 + (j - r.nw);
  }
  return -1;
}

// Persistent: one workgroup per compute unit, each taking items until every queue is empty.
__global__ __launch_bounds__(256, 1) void attn_bf16_d128_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  __shared__ int64_t next_item;
  const int xcc = (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) % kQueues);   // HW_REG_XCC_ID
  uint32_t dead = 0;
  for (;;) {
    if (threadIdx.x == 0) next_item = take_item(a, xcc, dead);
    __syncthreads();
    const int64_t item = next_item;
    __syncthreads();   // read by every thread before thread 0 takes the next one
    if (item < 0) break;
    const int64_t u = item < a.n_whole ? 0 : item - a.n_whole;
    const int tile = item < a.n_whole ? (int)item : (int)(a.n_whole + u / a.parts);
    process_item(a, smem, tile, item < a.n_whole ? 0 : (int)(u % a.parts));
  }
}

// The piece descriptor list of (b, h) = bh for list 0 (every tile of the launch's chunks) or
// list 1 + p (part p of a split tile: tiles [T p / parts, T (p + 1) / parts) of the T).
__device__ void write_piece_list(const AttnArgs& a, int64_t bh, int list) {
  const int64_t T = a.call_tiles;
  const int64_t v0 = list > 0 ? T * (list - 1) / a.parts : 0;
  const int64_t v1 = list > 0 ? T * list / a.parts : T;
  const int64_t b = bh / a.H, h = bh % a.H;
  const auto chunk = [&](int c) {
    const ChunkDesc& ch = a.ch[c];
    return PieceSrc{(uint64_t)(uintptr_t)ch.k + (uint64_t)(2 * (b * ch.k_sb + h * ch.k_sh)),
                    (uint64_t)(uintptr_t)ch.v + (uint64_t)(2 * (b * ch.v_sb + h * ch.v_sh)), ch.k_ss, ch.v_ss,
                    ch.len};
  };
  build_piece_list(a.ptable + (bh * kPieceLists + list) * kPieceSlots * kPieceWords, chunk, a.n_chunks, v0, v1);
}

// Before each launch.  Block 0 clears the queue counters and lists the slow whole tiles (in
// no particular order: each tile's result does not depend on when it runs); the other
// blocks write the piece descriptor lists, one per thread.
__global__ __launch_bounds__(256) void prep_kernel(AttnArgs a, int64_t lists) {
  if (blockIdx.x == 0) {
    __shared__ unsigned int n_slow;
    if (threadIdx.x == 0) n_slow = 0;
    if (threadIdx.x <= kSlowTaken) a.queue[threadIdx.x] = 0ull;
    __syncthreads();
    for (int64_t t = threadIdx.x; t < a.n_whole; t += blockDim.x)
      if (tile_is_slow(a, t)) a.slow_list[atomicAdd(&n_slow, 1u)] = (int32_t)t;
    __syncthreads();
    if (threadIdx.x == 0) a.queue[kSlowCount] = n_slow;
    return;
  }
  const int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x;
  if (i >= lists) return;
  const int per_bh = a.parts > 1 ? 1 + a.parts : 1;
  write_piece_list(a, i / per_bh, (int)(i % per_bh));
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)a.B * a.H * a.n_qtiles;
  const int64_t items = a.n_whole + (tiles - a.n_whole) * a.parts;
  const int cus = device_cus();
  const int64_t grid = items < cus || cus <= 0 ? items : cus;
  const int64_t lists = (int64_t)a.B * a.H * (a.parts > 1 ? 1 + a.parts : 1);
  prep_kernel<<<(unsigned)(1 + (lists + 255) / 256), 256, 0, s>>>(a, lists);
  attn_bf16_d128_kernel<<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fixedm
