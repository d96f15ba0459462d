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
//     query rows resident (in AGPRs) as the B operand of S^T = K Q^T
//     (v_mfma_f32_32x32x16_bf16).
//   * In the 32x32 accumulator layout each lane owns ONE query column and 16 keys, so the
//     per-query shift is a per-lane constant, the row sum is a per-lane running fp32 sum of
//     the fp32 probabilities, and the exp2'd scores, packed to bf16, are already the B operand
//     of O^T += V^T P^T with no transpose (the K-stationary layout of [CM]).  The matching key
//     order on the V^T operand comes from the gfx950 LDS transpose read ds_read_b64_tr_b16.
//   * K/V tiles of 32 keys stream through an 8-stage LDS ring (K ring in the first 64 KB,
//     V ring in the next 64 KB) with direct global->LDS loads (global_load_lds_dwordx4)
//     issued six tiles ahead; no VGPR staging.  Tiles are XOR-swizzled so both the K row
//     reads and the V transpose reads are bank-conflict free.
//   * A work item (a query tile, or part of a split one) runs all the 32-key tiles of its
//     chunk pieces as one pipeline, in one generated assembly block: the matrix cores and
//     the vector ALUs overlap within one wave, and the ring, its barriers and the
//     accumulators continue across chunk boundaries.
//   * The body is chosen per wave from its q-block's eligibility byte and bound U: the
//     fixed-m loop on bf16(alpha q) (U <= kR17MaxU), the fixed-m loop that applies alpha in
//     fp32 (eligible, U above it), or the online-softmax loop (ineligible).  All three take
//     the same loads and barriers, so the waves of a workgroup may run different bodies.
//   * Ragged KV tails: a chunk's partial last tile is loaded as its last 32-key window and
//     the keys already counted are masked; no padding copies.  Query rows past Sq are
//     clamped on load and land in padded workspace rows that finalize never reads.
//   * Persistent workgroups (one per compute unit) take work items from per-XCD queues:
//     each XCD works through consecutive tiles of the same heads (sharing the K/V stream in
//     its L2) and, once its queue is empty, takes work from the others.
//   * A call that continues a run starts each work item from the state the previous call
//     saved in the workspace (the loop loads it straight into its accumulation registers);
//     the run's last call writes O itself, each wave staging its rows through the idle ring
//     so that every store instruction writes whole rows.
#include <math.h>

#include <type_traits>

#include "fixedm_internal.h"

namespace fixedm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kKT = 32;                        // keys per pipeline tile
constexpr int kRowBytes = kD * 2;              // 256 bytes per key row
constexpr int kTileBytes = kKT * kRowBytes;    // 8 KB: K (or V) of one tile
constexpr int kStages = 8;                     // LDS ring depth in tiles
constexpr int kAhead = kStages - 2;            // tiles in flight ahead of the current one
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

typedef __attribute__((address_space(3))) uint8_t lds_u8;

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

// The three passes of a work item over its key tiles, written out instruction by instruction
// (generated): fixed_loop_asm, fixed_loop_fp32a_asm and online_loop_asm.
#include "fixed_loop.inc"

// How far (base 2) the online body lets a row's maximum run ahead of its reference before it
// raises the reference (word 19 of every piece descriptor): s = clamp(127 - ceil(log2 N) -
// ceil(log2 max|v|), 0, kMaxSlack), so that N 2^s max|v| <= 2^127 and the accumulators stay
// finite wherever those of exact online softmax (s = 0) do.  The larger s, the rarer the
// raises (each rescales the row sums and, out of line, the accumulators), but the further a
// sharp row's dominant keys sit above the reference: their probabilities 2^x, x fractional,
// lose bits to the bf16 rounding of P that the fp32 row sum does not see, where a reference at
// the row's maximum gives the top key exactly 1.  kMaxSlack = 8 keeps that small.  max|v| is
// 256 when the V check passed, else the largest |v| it recorded (non-finite: s = 0; the output
// is then not finite anyway).
constexpr int kMaxSlack = 8;
__device__ inline float online_slack(const AttnArgs& a) {
  const uint32_t vb = (uint32_t)__builtin_amdgcn_readfirstlane(*a.v_bad);
  if (vb >= 0x7f800000u) return 0.0f;
  const int log2_v = vb == 0 ? 8 : (int)(vb >> 23) - 127 + ((vb & 0x7fffffu) != 0 ? 1 : 0);
  const int s = 127 - a.log2_n - log2_v;
  return (float)(s < 0 ? 0 : s > kMaxSlack ? kMaxSlack : s);
}

// Sets a work item's accumulators in the registers the assembly passes keep O in, o[n][m] in
// a[16 (4 n + m) .. + 15]: zero when `load` is 0, else the state saved in the workspace (its
// register order: 16 bytes per lane at ((n 4 + m) 4 + j) KB + 16 lane from the wave's 32 KB),
// loaded straight into those registers and waited for inside the block.
__device__ __attribute__((always_inline)) inline void init_acc(f32x16 (&o)[2][4], const float* wave_base, int lane,
                                                               uint32_t load) {
  const uint64_t s0 = uniform_u64((uint64_t)(uintptr_t)wave_base);
  const uint64_t s1 = s0 + 16384;
  const uint32_t v0 = 16u * (uint32_t)lane, v1 = v0 + 4096u, v2 = v0 + 8192u, v3 = v0 + 12288u;
  const uint32_t ld = __builtin_amdgcn_readfirstlane(load);
  asm volatile(
      "s_cmp_eq_u32 %[ld], 0\n"
      "s_cbranch_scc1 L_init_acc_zero_%=\n"
      "global_load_dwordx4 a[0:3], %[v0], %[s0] offset:0\n"
      "global_load_dwordx4 a[4:7], %[v0], %[s0] offset:1024\n"
      "global_load_dwordx4 a[8:11], %[v0], %[s0] offset:2048\n"
      "global_load_dwordx4 a[12:15], %[v0], %[s0] offset:3072\n"
      "global_load_dwordx4 a[16:19], %[v1], %[s0] offset:0\n"
      "global_load_dwordx4 a[20:23], %[v1], %[s0] offset:1024\n"
      "global_load_dwordx4 a[24:27], %[v1], %[s0] offset:2048\n"
      "global_load_dwordx4 a[28:31], %[v1], %[s0] offset:3072\n"
      "global_load_dwordx4 a[32:35], %[v2], %[s0] offset:0\n"
      "global_load_dwordx4 a[36:39], %[v2], %[s0] offset:1024\n"
      "global_load_dwordx4 a[40:43], %[v2], %[s0] offset:2048\n"
      "global_load_dwordx4 a[44:47], %[v2], %[s0] offset:3072\n"
      "global_load_dwordx4 a[48:51], %[v3], %[s0] offset:0\n"
      "global_load_dwordx4 a[52:55], %[v3], %[s0] offset:1024\n"
      "global_load_dwordx4 a[56:59], %[v3], %[s0] offset:2048\n"
      "global_load_dwordx4 a[60:63], %[v3], %[s0] offset:3072\n"
      "global_load_dwordx4 a[64:67], %[v0], %[s1] offset:0\n"
      "global_load_dwordx4 a[68:71], %[v0], %[s1] offset:1024\n"
      "global_load_dwordx4 a[72:75], %[v0], %[s1] offset:2048\n"
      "global_load_dwordx4 a[76:79], %[v0], %[s1] offset:3072\n"
      "global_load_dwordx4 a[80:83], %[v1], %[s1] offset:0\n"
      "global_load_dwordx4 a[84:87], %[v1], %[s1] offset:1024\n"
      "global_load_dwordx4 a[88:91], %[v1], %[s1] offset:2048\n"
      "global_load_dwordx4 a[92:95], %[v1], %[s1] offset:3072\n"
      "global_load_dwordx4 a[96:99], %[v2], %[s1] offset:0\n"
      "global_load_dwordx4 a[100:103], %[v2], %[s1] offset:1024\n"
      "global_load_dwordx4 a[104:107], %[v2], %[s1] offset:2048\n"
      "global_load_dwordx4 a[108:111], %[v2], %[s1] offset:3072\n"
      "global_load_dwordx4 a[112:115], %[v3], %[s1] offset:0\n"
      "global_load_dwordx4 a[116:119], %[v3], %[s1] offset:1024\n"
      "global_load_dwordx4 a[120:123], %[v3], %[s1] offset:2048\n"
      "global_load_dwordx4 a[124:127], %[v3], %[s1] offset:3072\n"
      "s_waitcnt vmcnt(0)\n"
      "s_branch L_init_acc_done_%=\n"
      "L_init_acc_zero_%=:\n"
      "v_accvgpr_write_b32 a0, 0\n"
      "v_accvgpr_write_b32 a1, 0\n"
      "v_accvgpr_write_b32 a2, 0\n"
      "v_accvgpr_write_b32 a3, 0\n"
      "v_accvgpr_write_b32 a4, 0\n"
      "v_accvgpr_write_b32 a5, 0\n"
      "v_accvgpr_write_b32 a6, 0\n"
      "v_accvgpr_write_b32 a7, 0\n"
      "v_accvgpr_write_b32 a8, 0\n"
      "v_accvgpr_write_b32 a9, 0\n"
      "v_accvgpr_write_b32 a10, 0\n"
      "v_accvgpr_write_b32 a11, 0\n"
      "v_accvgpr_write_b32 a12, 0\n"
      "v_accvgpr_write_b32 a13, 0\n"
      "v_accvgpr_write_b32 a14, 0\n"
      "v_accvgpr_write_b32 a15, 0\n"
      "v_accvgpr_write_b32 a16, 0\n"
      "v_accvgpr_write_b32 a17, 0\n"
      "v_accvgpr_write_b32 a18, 0\n"
      "v_accvgpr_write_b32 a19, 0\n"
      "v_accvgpr_write_b32 a20, 0\n"
      "v_accvgpr_write_b32 a21, 0\n"
      "v_accvgpr_write_b32 a22, 0\n"
      "v_accvgpr_write_b32 a23, 0\n"
      "v_accvgpr_write_b32 a24, 0\n"
      "v_accvgpr_write_b32 a25, 0\n"
      "v_accvgpr_write_b32 a26, 0\n"
      "v_accvgpr_write_b32 a27, 0\n"
      "v_accvgpr_write_b32 a28, 0\n"
      "v_accvgpr_write_b32 a29, 0\n"
      "v_accvgpr_write_b32 a30, 0\n"
      "v_accvgpr_write_b32 a31, 0\n"
      "v_accvgpr_write_b32 a32, 0\n"
      "v_accvgpr_write_b32 a33, 0\n"
      "v_accvgpr_write_b32 a34, 0\n"
      "v_accvgpr_write_b32 a35, 0\n"
      "v_accvgpr_write_b32 a36, 0\n"
      "v_accvgpr_write_b32 a37, 0\n"
      "v_accvgpr_write_b32 a38, 0\n"
      "v_accvgpr_write_b32 a39, 0\n"
      "v_accvgpr_write_b32 a40, 0\n"
      "v_accvgpr_write_b32 a41, 0\n"
      "v_accvgpr_write_b32 a42, 0\n"
      "v_accvgpr_write_b32 a43, 0\n"
      "v_accvgpr_write_b32 a44, 0\n"
      "v_accvgpr_write_b32 a45, 0\n"
      "v_accvgpr_write_b32 a46, 0\n"
      "v_accvgpr_write_b32 a47, 0\n"
      "v_accvgpr_write_b32 a48, 0\n"
      "v_accvgpr_write_b32 a49, 0\n"
      "v_accvgpr_write_b32 a50, 0\n"
      "v_accvgpr_write_b32 a51, 0\n"
      "v_accvgpr_write_b32 a52, 0\n"
      "v_accvgpr_write_b32 a53, 0\n"
      "v_accvgpr_write_b32 a54, 0\n"
      "v_accvgpr_write_b32 a55, 0\n"
      "v_accvgpr_write_b32 a56, 0\n"
      "v_accvgpr_write_b32 a57, 0\n"
      "v_accvgpr_write_b32 a58, 0\n"
      "v_accvgpr_write_b32 a59, 0\n"
      "v_accvgpr_write_b32 a60, 0\n"
      "v_accvgpr_write_b32 a61, 0\n"
      "v_accvgpr_write_b32 a62, 0\n"
      "v_accvgpr_write_b32 a63, 0\n"
      "v_accvgpr_write_b32 a64, 0\n"
      "v_accvgpr_write_b32 a65, 0\n"
      "v_accvgpr_write_b32 a66, 0\n"
      "v_accvgpr_write_b32 a67, 0\n"
      "v_accvgpr_write_b32 a68, 0\n"
      "v_accvgpr_write_b32 a69, 0\n"
      "v_accvgpr_write_b32 a70, 0\n"
      "v_accvgpr_write_b32 a71, 0\n"
      "v_accvgpr_write_b32 a72, 0\n"
      "v_accvgpr_write_b32 a73, 0\n"
      "v_accvgpr_write_b32 a74, 0\n"
      "v_accvgpr_write_b32 a75, 0\n"
      "v_accvgpr_write_b32 a76, 0\n"
      "v_accvgpr_write_b32 a77, 0\n"
      "v_accvgpr_write_b32 a78, 0\n"
      "v_accvgpr_write_b32 a79, 0\n"
      "v_accvgpr_write_b32 a80, 0\n"
      "v_accvgpr_write_b32 a81, 0\n"
      "v_accvgpr_write_b32 a82, 0\n"
      "v_accvgpr_write_b32 a83, 0\n"
      "v_accvgpr_write_b32 a84, 0\n"
      "v_accvgpr_write_b32 a85, 0\n"
      "v_accvgpr_write_b32 a86, 0\n"
      "v_accvgpr_write_b32 a87, 0\n"
      "v_accvgpr_write_b32 a88, 0\n"
      "v_accvgpr_write_b32 a89, 0\n"
      "v_accvgpr_write_b32 a90, 0\n"
      "v_accvgpr_write_b32 a91, 0\n"
      "v_accvgpr_write_b32 a92, 0\n"
      "v_accvgpr_write_b32 a93, 0\n"
      "v_accvgpr_write_b32 a94, 0\n"
      "v_accvgpr_write_b32 a95, 0\n"
      "v_accvgpr_write_b32 a96, 0\n"
      "v_accvgpr_write_b32 a97, 0\n"
      "v_accvgpr_write_b32 a98, 0\n"
      "v_accvgpr_write_b32 a99, 0\n"
      "v_accvgpr_write_b32 a100, 0\n"
      "v_accvgpr_write_b32 a101, 0\n"
      "v_accvgpr_write_b32 a102, 0\n"
      "v_accvgpr_write_b32 a103, 0\n"
      "v_accvgpr_write_b32 a104, 0\n"
      "v_accvgpr_write_b32 a105, 0\n"
      "v_accvgpr_write_b32 a106, 0\n"
      "v_accvgpr_write_b32 a107, 0\n"
      "v_accvgpr_write_b32 a108, 0\n"
      "v_accvgpr_write_b32 a109, 0\n"
      "v_accvgpr_write_b32 a110, 0\n"
      "v_accvgpr_write_b32 a111, 0\n"
      "v_accvgpr_write_b32 a112, 0\n"
      "v_accvgpr_write_b32 a113, 0\n"
      "v_accvgpr_write_b32 a114, 0\n"
      "v_accvgpr_write_b32 a115, 0\n"
      "v_accvgpr_write_b32 a116, 0\n"
      "v_accvgpr_write_b32 a117, 0\n"
      "v_accvgpr_write_b32 a118, 0\n"
      "v_accvgpr_write_b32 a119, 0\n"
      "v_accvgpr_write_b32 a120, 0\n"
      "v_accvgpr_write_b32 a121, 0\n"
      "v_accvgpr_write_b32 a122, 0\n"
      "v_accvgpr_write_b32 a123, 0\n"
      "v_accvgpr_write_b32 a124, 0\n"
      "v_accvgpr_write_b32 a125, 0\n"
      "v_accvgpr_write_b32 a126, 0\n"
      "v_accvgpr_write_b32 a127, 0\n"
      "L_init_acc_done_%=:\n"
      : "={a[0:15]}"(o[0][0]), "={a[16:31]}"(o[0][1]), "={a[32:47]}"(o[0][2]), "={a[48:63]}"(o[0][3]),
        "={a[64:79]}"(o[1][0]), "={a[80:95]}"(o[1][1]), "={a[96:111]}"(o[1][2]), "={a[112:127]}"(o[1][3])
      : [s0] "s"(s0), [s1] "s"(s1), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [v3] "v"(v3), [ld] "s"(ld)
      : "scc", "memory");
}

// A work item's pass over its key tiles, in the assembly block of its body: fixed-m with
// bf16(alpha q) fragments (kFixedR17), fixed-m with the logit factor applied in fp32
// (kFixedF32), or online softmax (kOnline; shift[] returns each query row's reference r,
// -inf before the first key).  Every body takes the same loads and barriers.
enum Body { kFixedR17, kFixedF32, kOnline };

__device__ __attribute__((always_inline)) void run_pass(const AttnArgs& a, uint8_t* smem, const uint32_t* pieces,
                                                        int n_tiles, const bf16x8 (&qf)[2][8], f32x16 (&o)[2][4],
                                                        float (&lsum)[2], float (&shift)[2], Body body, int wave,
                                                        int lane, const float* saved) {
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
  const uint64_t list = uniform_u64((uint64_t)(uintptr_t)pieces);
  const uint32_t nt = __builtin_amdgcn_readfirstlane((uint32_t)n_tiles);
  const uint32_t kb4 = (uint32_t)(4 * (l >> 5));
  // O starts from the state a previous call saved (its address), or from zero (0)
  const uint64_t accp = uniform_u64((uint64_t)(uintptr_t)saved);
  const uint32_t accv = 16u * (uint32_t)l;
  if (body == kOnline) {
    float nshift[2] = {-shift[0], -shift[1]};
    online_loop_asm(o, qf, lsum, nshift, koff, voff, lane6, kb4, list, nt, lds_wave, a.alpha, accp, accv);
    shift[0] = -nshift[0];
    shift[1] = -nshift[1];
    return;
  }
  const float nshift[2] = {-shift[0], -shift[1]};
  if (body == kFixedR17)
    fixed_loop_asm(o, qf, lsum, nshift, koff, voff, lane6, kb4, list, nt, lds_wave, accp, accv);
  else
    fixed_loop_fp32a_asm(o, qf, lsum, nshift, koff, voff, lane6, kb4, list, nt, lds_wave, a.alpha, accp, accv);
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
  // The item's workspace slot: acc in register order (one 1 KB coalesced float4 per (wave,
  // n, m, j)), l and r per padded query row; parts 1.. of a split tile have their own slots.
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
  // Every load of the set-up is issued before any of its results is used (the item's
  // set-up then costs one memory round trip): the block's flags, shift and bound, the query
  // rows and k_mean.
  // The pass starts by reading the item's first chunk-piece descriptor with scalar loads: its
  // two cache lines are requested here, beside the set-up's loads, so that read hits the scalar
  // cache instead of adding a memory round trip of its own.
  const uint32_t* pieces = a.ptable + ((int64_t)bh * kPieceLists + (split ? 1 + part : 0)) * kPieceSlots * kPieceWords;
  // (every list of the table is written before the launch, so this read is in bounds also for
  // an item without tiles; the table does not change during the launch)
  typedef const __attribute__((address_space(4))) uint32_t* const_u32;
  const const_u32 pieces_u = reinterpret_cast<const_u32>(uniform_u64((uint64_t)(uintptr_t)pieces));
  const uint32_t prefetched = pieces_u[0] ^ pieces_u[16];
  const uint32_t elig_raw = a.elig[bq];
  const int m_raw = a.m[bq];
  const double u_raw = a.u[bq];
  const float* km = a.k_mean + (int64_t)bh * kD;
  uint4 qw[2][8];
  f32x4 kmv[8][2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    int row = q0 + 32 * n + lq;
    if (row >= a.Sq) row = a.Sq - 1;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + b * a.q_sb + (int64_t)row * a.q_ss + h * a.q_sh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qw[n][kk] = *reinterpret_cast<const uint4*>(qp + 16 * kk + 8 * hh);
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int i = 0; i < 2; ++i) kmv[kk][i] = *reinterpret_cast<const f32x4*>(km + 16 * kk + 8 * hh + 4 * i);
  // (the descriptor lines are taken here, after every set-up load has been issued: their wait
  // overlaps the set-up's own)
  asm volatile("" ::"s"(prefetched));
  // The body is chosen per wave: make the choice visibly wave-uniform (a scalar branch), so
  // no wave steps through the other body's code with an empty exec mask (that code holds
  // barriers and assembly that keeps its state in fixed registers).
  const bool fixed = __builtin_amdgcn_readfirstlane((int)elig_raw) != 0;
  const int mshift = __builtin_amdgcn_readfirstlane(m_raw);
  // Eligible blocks with a bound above kR17MaxU take the fixed-m body with the logit factor
  // applied in fp32: the rounding of bf16(alpha q) moves a base-2 logit by up to 2^-8 U.
  // (a branch-free test: the bound's load then stays beside the other set-up loads instead of
  // being issued, and waited for, only after the eligibility flag has arrived)
  const bool r17 = __builtin_amdgcn_readfirstlane((int)((elig_raw != 0) & (u_raw <= kR17MaxU))) != 0;

  // resident query fragments (B operand of S^T = K Q^T) and the centring term q . k_mean.
  // The fixed-m assembly body takes its logits in base 2 straight from the MFMA: its query
  // fragments are bf16(alpha q) (fp32 product, one rounding: the base-2 rescale of Q that the
  // TPU path folds into Q's producer, [FM] Summary "Relayout optimization", bit-identical
  // there by the [UR] review thread) and c_i = (alpha q_i) . k_mean.  The other two bodies
  // keep q and scale their scores by alpha in fp32 (c_i = alpha (q_i . k_mean)).  The
  // scaling is a select, not a branch, so no load waits behind the choice.
  bf16x8 qf[2][8];
  float cdot[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    float dot = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 w = qw[n][kk];
      uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 x = {__uint_as_float(u[i] << 16) * a.alpha, __uint_as_float(u[i] & 0xffff0000u) * a.alpha};
        const bf16x2 y = __builtin_convertvector(x, bf16x2);
        uint32_t sc;
        __builtin_memcpy(&sc, &y, 4);
        u[i] = r17 ? sc : u[i];
      }
      __builtin_memcpy(&qf[n][kk], u, 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 kv = kmv[kk][i >> 1];
        dot = __builtin_fmaf(__uint_as_float(u[i] << 16), kv[2 * (i & 1)], dot);
        dot = __builtin_fmaf(__uint_as_float(u[i] & 0xffff0000u), kv[2 * (i & 1) + 1], dot);
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
  // (pinned to the exact registers the passes read them from, a[128 + 32 n + 4 kk .. + 3], so
  // that they never sit where the accumulators are loaded)
  asm volatile("" : "+{a[128:131]}"(qf[0][0]), "+{a[132:135]}"(qf[0][1]), "+{a[136:139]}"(qf[0][2]),
                    "+{a[140:143]}"(qf[0][3]), "+{a[144:147]}"(qf[0][4]), "+{a[148:151]}"(qf[0][5]),
                    "+{a[152:155]}"(qf[0][6]), "+{a[156:159]}"(qf[0][7]), "+{a[160:163]}"(qf[1][0]),
                    "+{a[164:167]}"(qf[1][1]), "+{a[168:171]}"(qf[1][2]), "+{a[172:175]}"(qf[1][3]),
                    "+{a[176:179]}"(qf[1][4]), "+{a[180:183]}"(qf[1][5]), "+{a[184:187]}"(qf[1][6]),
                    "+{a[188:191]}"(qf[1][7]));

  // A run that continues picks up its state where the previous call left it ([CM]
  // "Accumulate, then normalize once": the accumulators carry across ring steps): O and the
  // row sum from the workspace (the row sum in the low-half lanes only: the two halves'
  // sums are added at the end), and on the online body the running reference r (a fixed-m
  // row's shift is the same in every call).  The pass then just continues the sums.
  f32x16 o[2][4];
  float lsum[2] = {0.0f, 0.0f};
  float rprev[2] = {-INFINITY, -INFINITY};
  if (a.accumulate) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int64_t rowi = row0 + 32 * n + lq;
      const float lp = l_t[rowi];
      rprev[n] = r_t[rowi];
      lsum[n] = hh == 0 ? lp : 0.0f;
    }
  }
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
    shift[0] = rprev[0];
    shift[1] = rprev[1];
  }
  // The pass sets the accumulators itself (zero, or the saved state), so no start value is
  // kept in registers across it; an item without tiles only takes the saved state.
  const float* saved = a.accumulate ? acc_t + tb + wave * 8192 : nullptr;
  if (n_tiles > 0) {
    run_pass(a, smem, pieces, n_tiles, qf, o, lsum, shift, fixed ? (r17 ? kFixedR17 : kFixedF32) : kOnline, wave,
             lane, saved);
    wait_vmcnt<0>();   // the ring's trailing loads land before the workgroup's LDS is reused
    barrier();
  } else {
    init_acc(o, saved, lane, saved != nullptr ? 1u : 0u);
  }

  if (a.final_out && !split) {
    // The run ends with this launch (the accumulators already hold any earlier calls' keys):
    // normalise once ([CM] "Accumulate, then normalize once") and write O, and lse, from the accumulator
    // registers.  The arithmetic is the finalize kernel's: O = acc times the correctly rounded
    // 1 / l, bf16 by round-to-nearest-even, lse = ln 2 (r + log2 l).  A lane holds pieces of 4 elements of one
    // query row, rows 10 KB apart across a wave in the usual layout: stored directly, each
    // instruction would touch 64 rows.  So each wave stages its 64 rows in its own 32 KB of the
    // (now idle) ring, 32 pieces a row at piece p ^ (row mod 32), and stores whole rows: lane L
    // of instruction i writes piece L mod 32 of row 2 i + L / 32 (8 bytes bf16, 16 bytes fp32).
    const int64_t tb = (int64_t)tile * (kQTile * kD);
    // staging offsets from an id the compiler cannot hoist above the assembly block
    int sid = threadIdx.x;
    asm volatile("" : "+v"(sid));
    const int s_lane = sid & 63, s_lq = s_lane & 31, s_hh = s_lane >> 5;
    uint8_t* stage = smem + (sid >> 6) * 32768;
    // one code path per output type (no test of the type inside the loops)
    const auto write_out = [&](auto f32tag) {
      constexpr bool f32out = decltype(f32tag)::value;
      constexpr uint32_t pbytes = f32out ? 16u : 8u;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const float other = __shfl_xor(lsum[n], 32, 64);
        const float ltot = hh == 0 ? lsum[n] + other : other + lsum[n];
        const float lnew = ltot, rnew = shift[n], rl = row_recip(lnew);
        const int q = q0 + 32 * n + lq;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float x0 = o[n][m][4 * jj] * rl, x1 = o[n][m][4 * jj + 1] * rl;
            const float x2 = o[n][m][4 * jj + 2] * rl, x3 = o[n][m][4 * jj + 3] * rl;
            const int r = 32 * n + s_lq, pc = 8 * m + 2 * jj + s_hh;
            uint8_t* dst = stage + (uint32_t)(r * 32 + (pc ^ (r & 31))) * pbytes;
            if constexpr (f32out)
              *reinterpret_cast<f32x4*>(dst) = f32x4{x0, x1, x2, x3};
            else
              *reinterpret_cast<uint2*>(dst) = uint2{bf16x2_rne(x0, x1), bf16x2_rne(x2, x3)};
          }
        }
        if (a.lse != nullptr && hh == 0 && q < a.Sq) a.lse[(int64_t)bh * a.Sq + q] = lse_of(rnew, lnew);
      }
      // the wave's own rows only: its LDS writes complete before its reads of them
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 8
      for (int i = 0; i < 32; ++i) {
        const int r = 2 * i + s_hh, pc = s_lq, q = q0 + r;
        const uint8_t* src = stage + (uint32_t)(r * 32 + (pc ^ (r & 31))) * pbytes;
        if (q < a.Sq) {
          const int64_t off = b * a.o_sb + (int64_t)q * a.o_ss + h * a.o_sh + 4 * pc;
          if constexpr (f32out)
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + off) = *reinterpret_cast<const f32x4*>(src);
          else
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + off) = *reinterpret_cast<const uint2*>(src);
        }
      }
    };
    if (a.out_dtype == FIXEDM_F32)
      write_out(std::true_type{});
    else
      write_out(std::false_type{});
    return;
  }

  // ---- store the state into the item's workspace slot for the next call or the finalize:
  // acc, l (the sum of both halves' row sums) and r (the shift, or the online reference; a
  // part that has seen no key yet holds r = -inf, l = 0).
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const float other = __shfl_xor(lsum[n], 32, 64);
    const float ltot = hh == 0 ? lsum[n] + other : other + lsum[n];
    const int64_t rowi = row0 + 32 * n + lq;
    const float lnew = ltot, rnew = shift[n];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4* dst = reinterpret_cast<f32x4*>(acc_t + tb + ((((wave * 2 + n) * 4 + m) * 4 + jj) * 64 + lane) * 4);
        *dst = f32x4{o[n][m][4 * jj], o[n][m][4 * jj + 1], o[n][m][4 * jj + 2], o[n][m][4 * jj + 3]};
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
// Items taken so far (every successful take adds one): a workgroup whose own queue is empty
// reads it once and, when every item is taken, stops without trying the other queues one
// after another (a device-wide round trip each).
constexpr int kTakenTotal = kQueues + 2;

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
// queues seen empty (bit kQueues: the slow list; bit kQueues + 1: the launch has no slow
// tile, so a queue take needs no look at the tile's blocks).  -1: none left.
__device__ inline int64_t take_item(const AttnArgs& a, int xcc, uint32_t& dead) {
  if (!((dead >> kQueues) & 1u)) {
    const unsigned long long n_slow = __hip_atomic_load(a.queue + kSlowCount, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
    if (n_slow == 0) {
      dead |= 3u << kQueues;
    } else {
      const unsigned long long i = atomicAdd(a.queue + kSlowTaken, 1ull);
      if (i < n_slow) {
        atomicAdd(a.queue + kTakenTotal, 1ull);
        return a.slow_list[i];
      }
      dead |= 1u << kQueues;
    }
  }
  const bool any_slow = !((dead >> (kQueues + 1)) & 1u);
  bool checked = false;
  for (int k = 0; k < kQueues; ++k) {
    const int q = (xcc + k) % kQueues;
    if ((dead >> q) & 1u) continue;
    if (q != xcc && !checked) {
      checked = true;
      const int64_t n_items = a.n_whole + (int64_t)(a.B * a.H * a.n_qtiles - a.n_whole) * a.parts;
      if ((int64_t)__hip_atomic_load(a.queue + kTakenTotal, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_items)
        return -1;
    }
    const QueueRange r = queue_range(a, q);
    const int64_t j = (int64_t)atomicAdd(a.queue + q, 1ull);
    if (j >= r.size) {
      dead |= 1u << q;
      continue;
    }
    if (any_slow && j < r.nw && tile_is_slow(a, r.w0 + j)) {   // listed: taken from the slow list
      --k;                                          // this queue again
      continue;
    }
    atomicAdd(a.queue + kTakenTotal, 1ull);
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
  build_piece_list(a.ptable + (bh * kPieceLists + list) * kPieceSlots * kPieceWords, chunk, a.n_chunks, v0, v1,
                   __float_as_uint(online_slack(a)));
}

// Before each launch.  Block 0 clears the queue counters and lists the slow whole tiles (in
// no particular order: each tile's result does not depend on when it runs); the other
// blocks write the piece descriptor lists, one per thread.
__global__ __launch_bounds__(256) void prep_kernel(AttnArgs a, int64_t lists) {
  if (blockIdx.x == 0) {
    __shared__ unsigned int n_slow;
    if (threadIdx.x == 0) n_slow = 0;
    if (threadIdx.x <= kTakenTotal) a.queue[threadIdx.x] = 0ull;
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
