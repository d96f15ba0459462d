// Bounds and gate kernels: k_mean, per-row norms and their maxima, the V-magnitude check,
// and the integer shift m with the eligibility mask.
//
// Sources (page title, section):
//   [FM] "feat(attention): fixed-m splash attention kernel with dynamic bounds and safety
//        fallbacks", Summary (C(N), W(N), gate, m = ceil(U) - C(N), virtual K-centring),
//        review thread on the V check (|V| <= 256), commit message (dtype and v_ok contracts).
//   [UR] "feat(attention): 2D Ulysses+Ring attention with Global Virtual K-Centering",
//        Summary (key mean over real keys shared by every ring step; one merged reduction
//        of the Q, K and V norms).
//   [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention",
//        "Transpose prologue with fused norms" (Q keeps per-row sums of squares, K folds
//        into a running max), "Assembling the bound" (square roots deferred to the end).
//
// Arithmetic contract: every sum of squares runs over d in index order in fp64, without
// contraction (this file is built with -ffp-contract=off); products of bf16/fp32 values
// are exact in fp64.  Maxima are order-free.  The k_mean sum is a fixed-order tree in
// fp64; for bf16/fp32 keys of ordinary magnitude every partial sum is exact, so the result
// equals the in-order sum.  U = alpha64 * sqrt(Q2 * K2) in exactly that order.
#include <math.h>

#include "fixedm_internal.h"

namespace fixedm {
namespace {

__device__ inline float load_elem(const uint16_t* p) {
  return __uint_as_float(((uint32_t)(*p)) << 16);
}
__device__ inline float load_elem(const float* p) { return *p; }

// 8 consecutive elements as floats (16-byte aligned for bf16, 2x16 bytes for fp32).
__device__ inline void load8(const uint16_t* p, float* f) {
  uint4 w = *reinterpret_cast<const uint4*>(p);
  uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ inline void load8(const float* p, float* f) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ inline int find_chunk(const BoundsArgs& a, int64_t j) {
  int c = 0;
  while (c + 1 < a.n_chunks && j >= a.ch[c + 1].start) ++c;
  return c;
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    unsigned long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Clears the reduction targets and fills k_mean for the NONE / SUPPLIED modes.
__global__ void bounds_init_kernel(BoundsArgs a) {
  const int64_t nqb_all = (int64_t)a.B * a.H * a.nqb;
  const int64_t nkm = (int64_t)a.B * a.H * a.D;
  const int64_t total = nqb_all > nkm ? nqb_all : nkm;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < nqb_all) a.q2[i] = 0ull;
    if (i < (int64_t)a.B * a.H) a.k2[i] = 0ull;
    if (i < nkm) {
      if (a.center == FIXEDM_CENTER_NONE) a.k_mean[i] = 0.0f;
      else if (a.center == FIXEDM_CENTER_SUPPLIED) a.k_mean[i] = a.k_mean_in[i];
    }
    if (i == 0) *a.v_bad = 0;
  }
}

// Partial key sums for the COMPUTE centring mode: slab s of the global key range, one
// (b, h) per blockIdx.y.  Thread (rg, c) sums keys rg, rg + nrg, ... of the slab for the
// 8 dims of column chunk c; the row groups are then added in rg order.
template <typename T>
__global__ __launch_bounds__(256) void kmean_partial_kernel(BoundsArgs a) {
  __shared__ double red[256][8];
  const int nch = a.D / 8, nrg = 256 / nch;
  const int rg = threadIdx.x / nch, c = threadIdx.x % nch;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t s0 = a.N * blockIdx.x / kKmeanSlabs, s1 = a.N * (blockIdx.x + 1) / kKmeanSlabs;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (rg < nrg) {
    int ci = 0;
    for (int64_t j = s0 + rg; j < s1; j += nrg) {
      while (ci + 1 < a.n_chunks && j >= a.ch[ci + 1].start) ++ci;
      const ChunkDesc& cd = a.ch[ci];
      const T* row = reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + (j - cd.start) * cd.k_ss +
                     h * cd.k_sh + 8 * c;
      float f[8];
      load8(row, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = acc[i] + (double)f[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[threadIdx.x][i] = acc[i];
  __syncthreads();
  if (threadIdx.x < nch) {
    double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int g = 0; g < nrg; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = s[i] + red[g * nch + threadIdx.x][i];
    double* dst = a.kpart + ((int64_t)blockIdx.x * a.B * a.H + bh) * a.D + 8 * threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = s[i];
  }
}

// k_mean[b,h,d] = fp32(sum over slabs in order / N).
__global__ void kmean_final_kernel(BoundsArgs a) {
  const int64_t n = (int64_t)a.B * a.H * a.D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    double s = 0.0;
    for (int sl = 0; sl < kKmeanSlabs; ++sl) s = s + a.kpart[(int64_t)sl * n + i];
    a.k_mean[i] = (float)(s / (double)a.N);
  }
}

// One key per thread: K2 = max over keys of sum_d (k_d - k_mean_d)^2 (fp64, d in order),
// and the V-magnitude check on the same key's value row.
template <typename T>
__global__ __launch_bounds__(256) void knorm_vcheck_kernel(BoundsArgs a) {
  __shared__ unsigned long long wmax[4];
  __shared__ int wbad[4];
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  unsigned long long best = 0ull;
  int bad = 0;
  if (j < a.N) {
    const int ci = find_chunk(a, j);
    const ChunkDesc& cd = a.ch[ci];
    const int64_t jj = j - cd.start;
    const T* krow = reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + jj * cd.k_ss + h * cd.k_sh;
    const T* vrow = reinterpret_cast<const T*>(cd.v) + b * cd.v_sb + jj * cd.v_ss + h * cd.v_sh;
    const float* km = a.k_mean + (int64_t)bh * a.D;
    double s = 0.0;
    for (int d0 = 0; d0 < a.D; d0 += 8) {
      float f[8], g[8];
      load8(krow + d0, f);
      load8(vrow + d0, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double t = (double)f[i] - (double)km[d0 + i];
        s = s + t * t;
        bad |= !(fabsf(g[i]) <= 256.0f);
      }
    }
    best = (unsigned long long)__double_as_longlong(s);
  }
  best = wave_max_u64(best);
  const int any_bad = __any(bad) ? 1 : 0;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { wmax[w] = best; wbad[w] = any_bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = wmax[0];
    int vb = wbad[0];
    for (int i = 1; i < 4; ++i) { m = wmax[i] > m ? wmax[i] : m; vb |= wbad[i]; }
    atomicMax(a.k2 + bh, m);
    if (vb) atomicOr(a.v_bad, 1);
  }
}

// One query row per thread: Q2[b,h,beta] = max over the block's real rows of sum_d q_d^2.
template <typename T>
__global__ __launch_bounds__(256) void qnorm_kernel(BoundsArgs a) {
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t i0 = (int64_t)blockIdx.x * 256 + (threadIdx.x & ~63);  // wave's first row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i0 >= a.Sq) return;  // whole wave past the end
  unsigned long long v = 0ull;
  if (i < a.Sq) {
    const T* row = reinterpret_cast<const T*>(a.q) + b * a.q_sb + i * a.q_ss + h * a.q_sh;
    double s = 0.0;
    for (int d0 = 0; d0 < a.D; d0 += 8) {
      float f[8];
      load8(row + d0, f);
#pragma unroll
      for (int k = 0; k < 8; ++k) s = s + (double)f[k] * (double)f[k];
    }
    v = (unsigned long long)__double_as_longlong(s);
  }
  v = wave_max_u64(v);
  if ((threadIdx.x & 63) == 0) atomicMax(a.q2 + (int64_t)bh * a.nqb + i0 / a.q_block, v);
}

// U = alpha64 * sqrt(Q2 * K2); m = ceil(U) - C; elig = v_ok && U <= gate && U finite.
__global__ void gate_kernel(BoundsArgs a) {
  const int64_t n = (int64_t)a.B * a.H * a.nqb;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t bh = i / a.nqb;
  const double q2 = __longlong_as_double((long long)a.q2[i]);
  const double k2 = __longlong_as_double((long long)a.k2[bh]);
  const double u = __dmul_rn(a.alpha64, __dsqrt_rn(__dmul_rn(q2, k2)));
  const bool finite = isfinite(u);
  int32_t m = INT32_MAX;
  if (finite) {
    const double mc = ceil(u) - (double)a.C;
    if (mc >= -2147483648.0 && mc <= 2147483647.0) m = (int32_t)mc;
  }
  a.u[i] = u;
  a.m[i] = m;
  a.elig[i] = (uint8_t)((*a.v_bad == 0) && finite && (u <= (double)a.gate));
}

template <typename T>
void launch_typed(const BoundsArgs& a, hipStream_t s) {
  const int bh = a.B * a.H;
  if (a.center == FIXEDM_CENTER_COMPUTE) {
    kmean_partial_kernel<T><<<dim3(kKmeanSlabs, bh), 256, 0, s>>>(a);
    const int64_t n = (int64_t)bh * a.D;
    kmean_final_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  }
  knorm_vcheck_kernel<T><<<dim3((unsigned)((a.N + 255) / 256), bh), 256, 0, s>>>(a);
  qnorm_kernel<T><<<dim3((unsigned)((a.Sq + 255) / 256), bh), 256, 0, s>>>(a);
}

}  // namespace

hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s) {
  const int64_t nqb_all = (int64_t)a.B * a.H * a.nqb;
  const int64_t nkm = (int64_t)a.B * a.H * a.D;
  const int64_t init_n = nqb_all > nkm ? nqb_all : nkm;
  const unsigned init_blocks = (unsigned)((init_n + 255) / 256 < 4096 ? (init_n + 255) / 256 : 4096);
  bounds_init_kernel<<<init_blocks, 256, 0, s>>>(a);
  if (a.dtype == FIXEDM_BF16) launch_typed<uint16_t>(a, s);
  else launch_typed<float>(a, s);
  gate_kernel<<<(unsigned)((nqb_all + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fixedm
