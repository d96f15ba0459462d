// Internal declarations shared by the HIP translation units of libfixedm (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fixedm.h"

namespace fixedm {

constexpr int kMaxChunksPerLaunch = 1;   // K/V chunks folded by one attention launch
constexpr int kMaxBoundsChunks = 32;     // chunks one fixedm_bounds call accepts
constexpr int kKmeanSlabs = 64;          // key slabs of the deterministic k_mean reduction
constexpr int kQTile = 256;              // query rows per attention workgroup (4 waves x 64)

struct ChunkDesc {
  const void* k;
  const void* v;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t len;    // real keys in this chunk
  int64_t start;  // global index of its first key (bounds kernels)
};

// Device buffer layout of the bounds descriptor (byte offsets, 256-byte aligned).
struct BoundsLayout {
  size_t m, elig, u, q2, k2, k_mean, v_bad, scratch, total;
};
bool bounds_layout(const fixedm_problem& p, BoundsLayout* out);

// Workspace: acc fp32, then row sum l and row shift r, per padded query row.
struct WorkspaceLayout {
  int64_t n_qtiles, sq_pad;
  size_t acc, l, r, total;
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
  double* kpart;            // [kKmeanSlabs][B*H][D] partial key sums
};
hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;
  int64_t q_sb, q_ss, q_sh;
  ChunkDesc ch[kMaxChunksPerLaunch];
  int32_t n_chunks;
  int32_t B, H, D;
  int32_t Sq, n_qtiles, sq_pad;
  int32_t q_block, nqb;
  const int32_t* m;
  const uint8_t* elig;
  const float* k_mean;
  float alpha;       // fp32(scale * log2 e)
  double alpha64;    // fp64 scale * log2 e (fp32 path)
  float* acc;
  float* l;
  float* r;
  int32_t accumulate;  // 0: these keys open the run (initialise); 1: merge into workspace
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
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);

}  // namespace fixedm
