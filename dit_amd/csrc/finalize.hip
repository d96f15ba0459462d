// Finalize: O = acc / l once at the end (acc times the correctly rounded 1 / l), cast to the
// output dtype, optional log-sum-exp.
//
// Sources (page title, section):
//   [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention",
//        "Accumulate, then normalize once" (a single division at the end) and the Interface
//        table (lse = c_i + log(sum_exp) when training).
//
// The row sum is positive on every real row: under the gate every shifted exponent is at
// least -125, so each term is a normal fp32 and l >= N * 2^-125; on fallback rows the
// largest term is 2^0.  The page's 1e-37 clamp therefore never binds and is not applied.
// lse is returned in natural-log units: ln 2 * (r + log2 l), where r is the row's shift
// (m + alpha q.k_mean for fixed-m rows, the running max for fallback rows).
#include <math.h>

#include "fixedm_internal.h"

namespace fixedm {
namespace {

__device__ inline void store4(const FinalizeArgs& a, int b, int q, int h, int d0, float4 v) {
  if (a.out_dtype == FIXEDM_F32) {
    float* o = reinterpret_cast<float*>(a.out) + b * a.o_sb + (int64_t)q * a.o_ss + h * a.o_sh + d0;
    *reinterpret_cast<float4*>(o) = v;
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + b * a.o_sb + (int64_t)q * a.o_ss + h * a.o_sh + d0;
    uint2 w;
    w.x = bf16x2_rne(v.x, v.y);
    w.y = bf16x2_rne(v.z, v.w);
    *reinterpret_cast<uint2*>(o) = w;
  }
}

// acc in the bf16 kernel's register order: [tile][wave 4][n 2][m 4][j 4][lane 64][4].
// Tiles tile_begin.. are finalized (all of them, or only the split tail tiles after a
// launch that wrote the whole tiles' output itself).
__global__ void finalize_reg_kernel(FinalizeArgs a) {
  const int64_t total = (int64_t)a.B * a.H * a.n_qtiles * 8192;
  const int64_t idx = a.tile_begin * 8192 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t tile = idx / 8192;
  const int rem = (int)(idx % 8192);
  const int lane = rem & 63, jj = (rem >> 6) & 3, m = (rem >> 8) & 3, n = (rem >> 10) & 1, wave = rem >> 11;
  const int bh = (int)(tile / a.n_qtiles), qt = (int)(tile % a.n_qtiles);
  const int q = qt * kQTile + wave * 64 + n * 32 + (lane & 31);
  if (q >= a.Sq) return;
  const int d0 = 32 * m + 8 * jj + 4 * (lane >> 5);
  const int64_t rowi = (int64_t)bh * a.sq_pad + q;
  float l = a.l[rowi], r = a.r[rowi];
  float4 acc = reinterpret_cast<const float4*>(a.acc)[idx];
  if (a.parts > 1 && tile >= a.n_whole) {
    // a split tail tile: merge its parts (same shift on fixed-m rows, so every factor is 1
    // there and the merge is a plain sum; online rows rescale to the largest running max;
    // a part that saw no key has r = -inf and l = 0)
    const int64_t u0 = (tile - a.n_whole) * (a.parts - 1);
    const int rin = wave * 64 + n * 32 + (lane & 31);
    float rm = r;
    for (int p = 1; p < a.parts; ++p) rm = fmaxf(rm, a.r_x[(u0 + p - 1) * kQTile + rin]);
    const float f0 = r == rm ? 1.0f : (r == -INFINITY ? 0.0f : exp2f(r - rm));
    acc = make_float4(acc.x * f0, acc.y * f0, acc.z * f0, acc.w * f0);
    l = l * f0;
    for (int p = 1; p < a.parts; ++p) {
      const int64_t u = u0 + p - 1;
      const float rp = a.r_x[u * kQTile + rin];
      const float f = rp == rm ? 1.0f : (rp == -INFINITY ? 0.0f : exp2f(rp - rm));
      const float4 x = reinterpret_cast<const float4*>(a.acc_x)[u * 8192 + rem];
      acc = make_float4(acc.x + f * x.x, acc.y + f * x.y, acc.z + f * x.z, acc.w + f * x.w);
      l = l + f * a.l_x[u * kQTile + rin];
    }
    r = rm;
  }
  const float rl = row_recip(l);
  store4(a, bh / a.H, q, bh % a.H, d0, make_float4(acc.x * rl, acc.y * rl, acc.z * rl, acc.w * rl));
  if (a.lse != nullptr && m == 0 && jj == 0 && lane < 32)
    a.lse[(int64_t)bh * a.Sq + q] = lse_of(r, l);
}

// acc row-major: [bh][sq_pad][D].
__global__ void finalize_row_kernel(FinalizeArgs a) {
  const int per_row = a.D / 4;
  const int64_t total = (int64_t)a.B * a.H * a.Sq * per_row;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c4 = (int)(idx % per_row);
  const int64_t rq = idx / per_row;
  const int q = (int)(rq % a.Sq);
  const int bh = (int)(rq / a.Sq);
  const int64_t rowi = (int64_t)bh * a.sq_pad + q;
  const float l = a.l[rowi];
  const float4 acc = reinterpret_cast<const float4*>(a.acc + rowi * a.D)[c4];
  const float rl = row_recip(l);
  store4(a, bh / a.H, q, bh % a.H, 4 * c4, make_float4(acc.x * rl, acc.y * rl, acc.z * rl, acc.w * rl));
  if (a.lse != nullptr && c4 == 0) a.lse[(int64_t)bh * a.Sq + q] = lse_of(a.r[rowi], l);
}

}  // namespace

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  if (a.reg_layout) {
    const int64_t total = ((int64_t)a.B * a.H * a.n_qtiles - a.tile_begin) * 8192;
    if (total <= 0) return hipSuccess;
    finalize_reg_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
  } else {
    const int64_t total = (int64_t)a.B * a.H * a.Sq * (a.D / 4);
    finalize_row_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace fixedm
