// Fixed-m attention forward, fp32 inputs (head_dim 64 or 128): the precision path.
//
// Sources (page title, section):
//   [FM] "feat(attention): fixed-m splash attention kernel with dynamic bounds and safety
//        fallbacks", Summary (shift by the precomputed m; numerator and denominator
//        accumulate directly in fp32).
//   [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention",
//        "Assembling the bound" note (the exponent needs absolute precision) and
//        "Accumulate, then normalize once" (fp32 accumulator).
//   [UR] "feat(attention): 2D Ulysses+Ring attention with Global Virtual K-Centering",
//        Summary (online-softmax fallback).
//
// Peaked rows put base-2 exponents near 100, where an fp32 exponent would carry ~1e-5
// absolute error.  This path therefore forms each logit q.k and each exponent in fp64
// (products of fp32 values are exact in fp64) and evaluates 2^e in fp64; the probability
// is then rounded once to fp32 and, as the method prescribes, accumulated in fp32.
// One wave per workgroup, one query row per lane; keys are staged through LDS 32 at a time,
// and the launch's chunks are folded one after the other into the same registers.
#include <math.h>

#include "fixedm_internal.h"

namespace fixedm {
namespace {

constexpr int kKB = 32;

template <int D, bool kFixed>
__device__ void run(const AttnArgs& a, float (&qv)[D], float (&acc)[D], float& l, float& r,
                    int b, int h, float (*ks)[D], float (*vs)[D]) {
  const int lane = threadIdx.x;
  double shift = (double)r;
  for (int c = 0; c < a.n_chunks; ++c) {
    const ChunkDesc& cd = a.ch[c];
    const float* kb = reinterpret_cast<const float*>(cd.k) + b * cd.k_sb + h * cd.k_sh;
    const float* vb = reinterpret_cast<const float*>(cd.v) + b * cd.v_sb + h * cd.v_sh;
    for (int64_t key0 = 0; key0 < cd.len; key0 += kKB) {
      const int valid = (int)((cd.len - key0) < kKB ? (cd.len - key0) : kKB);
      __syncthreads();
      for (int i = lane; i < kKB * D / 4; i += 64) {
        const int row = i / (D / 4), c4 = i % (D / 4);
        const int64_t key = key0 + (row < valid ? row : valid - 1);
        reinterpret_cast<float4*>(ks[row])[c4] = *reinterpret_cast<const float4*>(kb + key * cd.k_ss + 4 * c4);
        reinterpret_cast<float4*>(vs[row])[c4] = *reinterpret_cast<const float4*>(vb + key * cd.v_ss + 4 * c4);
      }
      __syncthreads();
      if (!kFixed) {
        // online softmax: block max first (logits recomputed in the second pass)
        double zmax = -INFINITY;
        for (int j = 0; j < valid; ++j) {
          double s = 0.0;
#pragma unroll
          for (int d = 0; d < D; ++d) s = fma((double)qv[d], (double)ks[j][d], s);
          zmax = fmax(zmax, a.alpha64 * s);
        }
        const float rn = fmaxf(r, (float)zmax);
        const float f = (float)exp2((double)r - (double)rn);
        r = rn;
        shift = (double)rn;
        l *= f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= f;
      }
      for (int j = 0; j < valid; ++j) {
        double s = 0.0;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fma((double)qv[d], (double)ks[j][d], s);
        const float p = (float)exp2(a.alpha64 * s - shift);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vs[j][d], acc[d]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float ks[kKB][D];
  __shared__ __attribute__((aligned(16))) float vs[kKB][D];
  const int nq64 = (a.Sq + 63) / 64;
  const int bh = blockIdx.x / nq64, qt = blockIdx.x % nq64;
  const int b = bh / a.H, h = bh % a.H;
  const int lane = threadIdx.x;
  const int row = qt * 64 + lane;
  const int rowc = row < a.Sq ? row : a.Sq - 1;
  const int beta = (qt * 64) / a.q_block;
  const int64_t bq = (int64_t)bh * a.nqb + beta;
  const bool fixed = a.elig[bq] != 0;

  float qv[D], acc[D];
  const float* qp = reinterpret_cast<const float*>(a.q) + b * a.q_sb + (int64_t)rowc * a.q_ss + h * a.q_sh;
  const float* km = a.k_mean + (int64_t)bh * D;
  double dot = 0.0;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qp[d];
    acc[d] = 0.0f;
    dot = fma((double)qv[d], (double)km[d], dot);
  }
  float l = 0.0f, r;
  if (fixed) {
    const int32_t mm = a.m_row != nullptr ? a.m_row[(int64_t)bh * a.Sq + rowc] : a.m[bq];
    r = (float)((double)mm + a.alpha64 * dot);
    run<D, true>(a, qv, acc, l, r, b, h, ks, vs);
  } else {
    r = -INFINITY;
    run<D, false>(a, qv, acc, l, r, b, h, ks, vs);
  }

  // fold into the row-major workspace
  const int64_t rowi = (int64_t)bh * a.sq_pad + row;
  float fw = 0.0f, fo = 1.0f, lnew = l, rnew = r;
  if (a.accumulate) {
    const float lp = a.l[rowi], rp = a.r[rowi];
    if (fixed) {
      fw = 1.0f;
      lnew = lp + l;
    } else {
      rnew = fmaxf(rp, r);
      fw = (float)exp2((double)rp - (double)rnew);
      fo = (float)exp2((double)r - (double)rnew);
      lnew = lp * fw + l * fo;
    }
  }
  float* dst = a.acc + rowi * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    float v = acc[d];
    if (a.accumulate) v = fixed ? dst[d] + v : dst[d] * fw + v * fo;
    dst[d] = v;
  }
  a.l[rowi] = lnew;
  a.r[rowi] = rnew;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const int nb = a.B * a.H * ((a.Sq + 63) / 64);
  if (a.D == 64) attn_f32_kernel<64><<<nb, 64, 0, s>>>(a);
  else attn_f32_kernel<128><<<nb, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fixedm
