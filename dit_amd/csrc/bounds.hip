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

// Row j of the global key order (chunk by chunk) for this (b, h), in K or in V.
template <typename T>
__device__ inline const T* key_row(const BoundsArgs& a, int b, int h, int64_t j, bool v) {
  const ChunkDesc& cd = a.ch[find_chunk(a, j)];
  return v ? reinterpret_cast<const T*>(cd.v) + b * cd.v_sb + (j - cd.start) * cd.v_ss + h * cd.v_sh
           : reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + (j - cd.start) * cd.k_ss + h * cd.k_sh;
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
  // eight rows in flight per thread; they are added in increasing key order
  for (int64_t j = s0 + rg; j < s1; j += 8 * nrg) {
    float f[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t jj = j + (int64_t)u * nrg;
      if (jj < s1) load8(key_row<T>(a, b, h, jj, false) + 8 * c, f[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j + (int64_t)u * nrg < s1)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + (double)f[u][i];
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

// One row per thread in the norm kernels: every 16-byte piece of the row is loaded before
// any arithmetic, so a wave keeps 16 loads per lane in flight; the row is then summed in
// index order.  Loads a row of D elements (D = 64 or 128; 128 or 256 bytes for bf16, 256 or 512 for fp32)
// as 16-byte pieces into registers.
template <typename T>
struct RowRegs {
  static constexpr int kPieces = 128 * (int)sizeof(T) / 16;   // for D = 128
  uint4 p[kPieces];
  __device__ inline void load(const T* row, int D) {
    const int n = D * (int)sizeof(T) / 16;
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (i < n) p[i] = reinterpret_cast<const uint4*>(row)[i];
  }
  __device__ inline float elem(int d) const {   // d in [0, D)
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
    if (sizeof(T) == 2) {
      const uint32_t u = w[d >> 1];
      return __uint_as_float((d & 1) ? (u & 0xffff0000u) : (u << 16));
    }
    return __uint_as_float(w[d]);
  }
};

// fp64 sum over d in index order of (x_d - c_d)^2.
template <typename T>
__device__ inline double row_sumsq(const RowRegs<T>& r, const float* c, int D) {
  double s = 0.0;
#pragma unroll
  for (int d = 0; d < 128; ++d) {
    if (d < D) {
      const double t = (double)r.elem(d) - (double)c[d];
      s = s + t * t;
    }
  }
  return s;
}

// 256 keys of one (b, h) per workgroup: K2 = max over keys of sum_d (k_d - k_mean_d)^2
// (fp64, d in order), and the V-magnitude check on the same keys' value rows.
template <typename T>
__global__ __launch_bounds__(256) void knorm_vcheck_kernel(BoundsArgs a) {
  __shared__ float km[128];
  __shared__ unsigned long long wmax[4];
  __shared__ int wbad[4];
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * 256 + tid;
  if (tid < a.D) km[tid] = a.k_mean[(int64_t)bh * a.D + tid];
  __syncthreads();
  unsigned long long best = 0ull;
  int bad = 0;
  if (j < a.N) {
    RowRegs<T> kr, vr;
    kr.load(key_row<T>(a, b, h, j, false), a.D);
    vr.load(key_row<T>(a, b, h, j, true), a.D);
    best = (unsigned long long)__double_as_longlong(row_sumsq<T>(kr, km, a.D));
#pragma unroll
    for (int d = 0; d < 128; ++d)
      if (d < a.D) bad |= !(fabsf(vr.elem(d)) <= 256.0f);
  }
  best = wave_max_u64(best);
  const int any_bad = __any(bad) ? 1 : 0;
  const int w = tid >> 6;
  if ((tid & 63) == 0) { wmax[w] = best; wbad[w] = any_bad; }
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = wmax[0];
    int vb = wbad[0];
    for (int i = 1; i < 4; ++i) { m = wmax[i] > m ? wmax[i] : m; vb |= wbad[i]; }
    atomicMax(a.k2 + bh, m);
    if (vb) atomicOr(a.v_bad, 1);
  }
}

// One query row per thread: Q2[b,h,beta] = max over the block's real rows of sum_d q_d^2.
// Each wave's 64 rows lie in one q-block (q_block is a multiple of 64).
template <typename T>
__global__ __launch_bounds__(256) void qnorm_kernel(BoundsArgs a) {
  __shared__ float zero[128];
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  if (tid < 128) zero[tid] = 0.0f;
  __syncthreads();
  const int64_t iw = (int64_t)blockIdx.x * 256 + (tid & ~63);   // the wave's first row
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  if (iw >= a.Sq) return;
  unsigned long long v = 0ull;
  if (i < a.Sq) {
    RowRegs<T> qr;
    qr.load(reinterpret_cast<const T*>(a.q) + b * a.q_sb + i * a.q_ss + h * a.q_sh, a.D);
    v = (unsigned long long)__double_as_longlong(row_sumsq<T>(qr, zero, a.D));
  }
  v = wave_max_u64(v);
  if ((tid & 63) == 0) atomicMax(a.q2 + (int64_t)bh * a.nqb + iw / a.q_block, v);
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
