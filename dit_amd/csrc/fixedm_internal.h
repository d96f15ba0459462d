// Internal declarations shared by the HIP translation units of libfixedm (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fixedm.h"
#include "pieces.h"
#include "split_plan.h"

namespace fixedm {

constexpr int kMaxChunksPerLaunch = 8;   // K/V chunks folded by one attention launch
constexpr int kMaxBoundsChunks = 32;     // chunks one fixedm_bounds call accepts
constexpr int kBoundsHeads = 64;         // heads one bounds workgroup covers (LDS staging)
constexpr int kQTile = 256;              // query rows per attention workgroup (4 waves x 64)
constexpr int kPieceWords = kPieceDescWords;   // dwords of one chunk-piece descriptor (bf16 kernel)
constexpr int kPieceSlots = kMaxChunksPerLaunch + 1;   // descriptors of a list, terminator included
constexpr int kPieceLists = 1 + kMaxParts;            // lists per (b, h): whole tiles, then each part
constexpr int64_t kMaxKeys = (int64_t)1 << 38;   // most keys of a problem (and of a chunk)
constexpr int64_t kMaxKeysBf16 = (int64_t)1 << 35;   // most keys of a bf16 problem
constexpr int64_t kMaxRowStrideBf16 = (int64_t)1 << 26;   // largest sequence stride of a bf16 tensor

// Key slabs of the k_mean reduction: about 256 workgroups of B x head groups (with 640-thread
// workgroups that fills the chip; more slabs only lengthen the final reduction), at most one
// slab per 16 keys, and at most max_slabs.  The key sum is
// exact, so the slab count changes the speed only, never a bit of the result.
inline int kmean_slabs(int64_t B, int64_t H, int64_t N, int64_t max_slabs = 1 << 30) {
  const int64_t groups = B * ((H + kBoundsHeads - 1) / kBoundsHeads);
  int64_t s = (256 + groups - 1) / groups;
  if (s > N / 16) s = N / 16;
  if (s > max_slabs) s = max_slabs;
  if (s < 1) s = 1;
  return (int)s;
}

// Scratch of one bounds call in COMPUTE centring: the key-mean partial sums
// [slabs][B*H][D] fp64, then their exactness flags [slabs][B*H][D] uint8 (byte offsets from the
// scratch base, 256-byte aligned).  Empty for the other centring modes.
struct BoundsScratch {
  int32_t slabs;
  size_t kpart, kflag, total;
};
inline BoundsScratch bounds_scratch(const fixedm_problem& p, int64_t max_slabs = 1 << 30) {
  BoundsScratch s{0, 0, 0, 0};
  if (p.center != FIXEDM_CENTER_COMPUTE) return s;
  const size_t el = (size_t)(p.batch * p.heads) * (size_t)p.head_dim;
  s.slabs = kmean_slabs(p.batch, p.heads, p.sk_total, max_slabs);
  s.kflag = ((size_t)s.slabs * el * 8 + 255) & ~(size_t)255;
  s.total = (s.kflag + (size_t)s.slabs * el + 255) & ~(size_t)255;
  return s;
}

// The no-allocation variant of fixedm_bounds keeps its scratch in one static device array
// of this many bytes per GPU (defined in bounds.hip).
constexpr size_t kStaticScratchBytes = (size_t)24 << 20;
// Device address of that array on the current device (looked up once per device), or null
// if the lookup fails.
void* static_scratch();

struct ChunkDesc {
  const void* k;
  const void* v;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t len;    // real keys in this chunk
  int64_t start;  // index of its first key: over all chunks (bounds kernels), or within the
                  // launch's chunk sequence (attention kernels)
};

// Device buffer layout of the bounds descriptor (byte offsets, 256-byte aligned).
struct BoundsLayout {
  size_t m, elig, u, q2, k2, k_mean, v_bad, m_row, q2_row, u_row, scratch, total;
};
bool bounds_layout(const fixedm_problem& p, BoundsLayout* out);

// Workspace: acc fp32, then row sum l and row shift r, per padded query row; for the bf16
// kernel also the same three for parts 1.. of split tail tiles ([kMaxParts - 1] per tile,
// room for kMaxSplitTail tiles), and the work-queue counters of its launches.
struct WorkspaceLayout {
  int64_t n_qtiles, sq_pad;
  size_t acc, l, r, acc_x, l_x, r_x, queue, slow_list, ptable, total;
};
bool workspace_layout(const fixedm_problem& p, WorkspaceLayout* out);

struct BoundsArgs {
  const void* q;
  int64_t q_sb, q_ss, q_sh;
  ChunkDesc ch[kMaxBoundsChunks];
  int32_t n_chunks;
  int32_t dtype;
  int32_t B, H, D;
  int64_t Sq, N, q_block, nqb;
  int32_t center;
  const float* k_mean_in;
  double alpha64;
  int32_t C, gate;
  // outputs (device)
  int32_t* m;
  uint8_t* elig;
  double* u;
  unsigned long long* q2;   // fp64 bit patterns (non-negative: integer order = value order)
  unsigned long long* k2;
  float* k_mean;
  int32_t* v_bad;
  double* kpart;            // [kslabs][B*H][D] partial key sums
  uint8_t* kflag;           // [kslabs][B*H][D]: 1 when that slab's partial sum of the element
                            // may not be exact (or a key is not finite)
  int32_t kslabs;
  // per-row shifts (shift == FIXEDM_SHIFT_ROW; null otherwise): [B, H, Sq]
  int32_t* m_row;
  double* q2_row;
  double* u_row;
};
hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;
  int64_t q_sb, q_ss, q_sh;
  ChunkDesc ch[kMaxChunksPerLaunch];
  int32_t n_chunks;
  int64_t call_len;    // keys of all chunks of this launch
  int64_t call_tiles;  // their 32-key tiles (the sum over chunks of ceil(len / 32))
  int32_t B, H, D;
  int32_t Sq, n_qtiles, sq_pad;
  int32_t q_block, nqb;
  const int32_t* m;
  const int32_t* m_row;   // per-row shifts [B, H, Sq], or null for one shift per q-block
  const uint8_t* elig;
  const double* u;        // per-block bound U [B, H, nQB]
  const float* k_mean;
  const int32_t* v_bad;   // 0, or the fp32 bits of the largest |v| when some |v| > 256
  int32_t log2_n;         // ceil(log2 N), N the keys of the whole run
  float alpha;       // fp32(scale * log2 e)
  double alpha64;    // fp64 scale * log2 e (fp32 path)
  float* acc;
  float* l;
  float* r;
  int32_t accumulate;  // 0: these keys open the run (initialise); 1: merge into workspace
  int32_t n_whole, parts;      // split plan (bf16 kernel)
  unsigned long long* queue;   // bf16 kernel: 8 work-queue counters, the slow-list length and
                               // take counter, the count of items taken (set up before each
                               // launch; 16 slots)
  int32_t* slow_list;          // bf16 kernel: whole tiles taken first (room for every tile)
  uint32_t* ptable;            // bf16 kernel: chunk-piece descriptor lists [B*H][kPieceLists]
                               // [kPieceSlots][kPieceWords] (written before each launch)
  float* acc_x;                // parts 1.. of split tiles: [(tile - n_whole) * (parts - 1) + part - 1]
  float* l_x;
  float* r_x;
  // Fused finalize (bf16 kernel): when set, this launch completes the run and the whole
  // tiles write O = acc / l (and lse) straight from registers; split tiles still fold
  // into the workspace for a finalize over those tiles only.
  int32_t final_out;
  int32_t out_dtype;
  void* out;
  int64_t o_sb, o_ss, o_sh;
  float* lse;
};
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

struct FinalizeArgs {
  const float* acc;
  const float* l;
  const float* r;
  void* out;
  int64_t o_sb, o_ss, o_sh;
  int32_t out_dtype;
  float* lse;
  int32_t B, H, D, Sq, n_qtiles, sq_pad;
  int32_t reg_layout;  // 1: acc in the bf16 kernel's register order; 0: row-major [bh][q][d]
  int32_t n_whole, parts;      // split plan of the bf16 launches (reg_layout only)
  int64_t tile_begin;          // reg_layout: first query tile finalized (the rest follow)
  const float* acc_x;
  const float* l_x;
  const float* r_x;
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);

int device_cus();   // compute units of the current device (cached per device)

// Two fp32 values to a packed bf16 pair (lo in bits 0..15) by the hardware conversion
// (v_cvt_pk_bf16_f32): round-to-nearest-even for every value that is not a NaN (subnormals, ties
// and the overflow to infinity included; checked against the bit formula on 2^20 values), and a
// NaN stays a quiet NaN of the same sign.  The output cast of both the finalize kernel and the
// fused finalize of the bf16 attention kernel.
__device__ inline uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t x = {lo, hi};
  const bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
  uint32_t w;
  __builtin_memcpy(&w, &y, 4);
  return w;
}

// The output row is acc times the correctly rounded reciprocal of its row sum l: within 1.5
// ulp of the fp32 quotient acc / l, one multiply an element instead of a division each (the
// reciprocal is formed once a row).  The fused epilogue of the bf16 attention kernel and the
// finalize kernels all form it this way, so every output path gives the same bits.
__device__ inline float row_recip(float l) { return __fdiv_rn(1.0f, l); }

// Natural-log log-sum-exp of a row from its base-2 shift r and its row sum l under r.
__device__ inline float lse_of(float r, float l) {
  return 0.69314718055994531f * (r + log2f(l));
}

}  // namespace fixedm
