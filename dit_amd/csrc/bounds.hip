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

// Partial key sums for the COMPUTE centring mode.  Workgroup (slab, b, head group): thread
// (hl, c) owns dims 8c..8c+7 of head h0 + hl and adds the keys of the slab in key order.
// A key's rows of the whole head group are adjacent in memory, so each key is one
// contiguous read of the workgroup (10 KB for 40 heads of 128 bf16 dims).
template <typename T>
__global__ __launch_bounds__(1024) void kmean_partial_kernel(BoundsArgs a) {
  const int per = a.D / 8;
  const int hl = threadIdx.x / per, c = threadIdx.x % per;
  const int b = blockIdx.y, h = blockIdx.z * kBoundsHeads + hl;
  if (h >= a.H) return;
  const int64_t s0 = a.N * blockIdx.x / a.kslabs, s1 = a.N * (blockIdx.x + 1) / a.kslabs;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int ci = 0;                                    // chunk of the current key (uniform)
  for (int64_t j = s0; j < s1; j += 8) {
    float f[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t jj = j + u;
      if (jj < s1) {
        while (ci + 1 < a.n_chunks && jj >= a.ch[ci + 1].start) ++ci;
        const ChunkDesc& cd = a.ch[ci];
        load8(reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + (jj - cd.start) * cd.k_ss + h * cd.k_sh + 8 * c,
              f[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j + u < s1)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + (double)f[u][i];
  }
  double* dst = a.kpart + ((int64_t)blockIdx.x * a.B * a.H + (int64_t)b * a.H + h) * a.D + 8 * c;
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = acc[i];
}

// k_mean[b,h,d] = fp32(sum over slabs in order / N).
__global__ void kmean_final_kernel(BoundsArgs a) {
  const int64_t n = (int64_t)a.B * a.H * a.D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    double s = 0.0;
    for (int sl = 0; sl < a.kslabs; ++sl) s = s + a.kpart[(int64_t)sl * n + i];
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

// fp64 sum over d in index order of x_d^2.
template <typename T>
__device__ inline double row_sumsq(const RowRegs<T>& r, int D) {
  double s = 0.0;
#pragma unroll
  for (int d = 0; d < 128; ++d) {
    if (d < D) {
      const double t = (double)r.elem(d);
      s = s + t * t;
    }
  }
  return s;
}

// Row r of a norm workgroup's block: kBoundsKeys positions x the head group's heads, in
// memory order (heads of one position adjacent).  One row per thread and pass, so a wave
// reads 64 consecutive 256-byte rows: every cache line it touches is used whole.
struct RowBlock {
  int64_t p0;      // first position of the block
  int h0, hg;      // head group: first head, heads
  int rows;        // positions in the block x hg
};

__device__ inline RowBlock row_block(int64_t block, int64_t n_pos, int H) {
  RowBlock rb;
  rb.p0 = block * kBoundsKeys;
  rb.h0 = blockIdx.z * kBoundsHeads;
  rb.hg = H - rb.h0 < kBoundsHeads ? H - rb.h0 : kBoundsHeads;
  const int64_t np = n_pos - rb.p0 < kBoundsKeys ? n_pos - rb.p0 : kBoundsKeys;
  rb.rows = (int)np * rb.hg;
  return rb;
}

// K2[b,h] = max over keys of sum_d (k_d - k_mean_d)^2 (fp64, d in order), and the
// V-magnitude check on the same rows of V.  Workgroup (key block, b, head group); the head
// group's k_mean sits in LDS with a padded row stride (lanes of a wave read different heads).
template <typename T>
__global__ __launch_bounds__(256) void knorm_vcheck_kernel(BoundsArgs a) {
  __shared__ float km[kBoundsHeads * 129];
  __shared__ unsigned long long hmax[kBoundsHeads];
  const int b = blockIdx.y, tid = threadIdx.x, D = a.D, DP = D + 1;
  const int h0 = blockIdx.z * kBoundsHeads;
  const int hg = a.H - h0 < kBoundsHeads ? a.H - h0 : kBoundsHeads;
  for (int i = tid; i < hg * D; i += 256)
    km[(i / D) * DP + i % D] = a.k_mean[((int64_t)b * a.H + h0) * D + i];
  for (int i = tid; i < hg; i += 256) hmax[i] = 0ull;
  __syncthreads();
  const int64_t n_blocks = (a.N + kBoundsKeys - 1) / kBoundsKeys;
  int bad = 0;
  for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
    const RowBlock rb = row_block(blk, a.N, a.H);
    for (int r = tid; r < rb.rows; r += 256) {
      const int hl = r % rb.hg;
      const int64_t j = rb.p0 + r / rb.hg;
      const int h = h0 + hl;
      const ChunkDesc& cd = a.ch[find_chunk(a, j)];
      const int64_t jl = j - cd.start;
      RowRegs<T> kr;
      kr.load(reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + jl * cd.k_ss + h * cd.k_sh, D);
      if (sizeof(T) == 2) {
        RowRegs<T> vr;
        vr.load(reinterpret_cast<const T*>(cd.v) + b * cd.v_sb + jl * cd.v_ss + h * cd.v_sh, D);
        atomicMax(&hmax[hl], (unsigned long long)__double_as_longlong(row_sumsq<T>(kr, km + hl * DP, D)));
#pragma unroll
        for (int d = 0; d < 128; ++d)
          if (d < D) bad |= !(fabsf(vr.elem(d)) <= 256.0f);
      } else {
        atomicMax(&hmax[hl], (unsigned long long)__double_as_longlong(row_sumsq<T>(kr, km + hl * DP, D)));
        RowRegs<T> vr;     // fp32 rows are 512 bytes: one row in registers at a time
        vr.load(reinterpret_cast<const T*>(cd.v) + b * cd.v_sb + jl * cd.v_ss + h * cd.v_sh, D);
#pragma unroll
        for (int d = 0; d < 128; ++d)
          if (d < D) bad |= !(fabsf(vr.elem(d)) <= 256.0f);
      }
    }
  }
  const int any_bad = __any(bad) ? 1 : 0;
  __syncthreads();
  for (int i = tid; i < hg; i += 256)
    if (hmax[i] != 0ull) atomicMax(a.k2 + (int64_t)b * a.H + h0 + i, hmax[i]);
  if (any_bad && (tid & 63) == 0) atomicOr(a.v_bad, 1);
}

// Q2[b,h,beta] = max over the block's real rows of sum_d q_d^2.  Workgroup (position
// block, b, head group): its kBoundsKeys positions lie in one q-block (q_block is a
// multiple of 64), so each head has one maximum per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void qnorm_kernel(BoundsArgs a) {
  __shared__ unsigned long long hmax[kBoundsHeads];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int h0 = blockIdx.z * kBoundsHeads;
  const int hg = a.H - h0 < kBoundsHeads ? a.H - h0 : kBoundsHeads;
  const int64_t n_blocks = (a.Sq + kBoundsKeys - 1) / kBoundsKeys;
  for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
    if (tid < hg) hmax[tid] = 0ull;
    __syncthreads();
    const RowBlock rb = row_block(blk, a.Sq, a.H);
    for (int r = tid; r < rb.rows; r += 256) {
      const int hl = r % rb.hg;
      const int64_t i = rb.p0 + r / rb.hg;
      RowRegs<T> qr;
      qr.load(reinterpret_cast<const T*>(a.q) + b * a.q_sb + i * a.q_ss + (h0 + hl) * a.q_sh, a.D);
      atomicMax(&hmax[hl], (unsigned long long)__double_as_longlong(row_sumsq<T>(qr, a.D)));
    }
    __syncthreads();
    const int64_t beta = rb.p0 / a.q_block;
    if (tid < hg && hmax[tid] != 0ull) atomicMax(a.q2 + ((int64_t)b * a.H + h0 + tid) * a.nqb + beta, hmax[tid]);
    __syncthreads();
  }
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
  const unsigned groups = (unsigned)((a.H + kBoundsHeads - 1) / kBoundsHeads);
  if (a.center == FIXEDM_CENTER_COMPUTE) {
    const int hpg = a.H < kBoundsHeads ? a.H : kBoundsHeads;
    kmean_partial_kernel<T><<<dim3((unsigned)a.kslabs, (unsigned)a.B, groups), hpg * (a.D / 8), 0, s>>>(a);
    const int64_t n = (int64_t)a.B * a.H * a.D;
    kmean_final_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  }
  const int64_t kb = (a.N + kBoundsKeys - 1) / kBoundsKeys, qb = (a.Sq + kBoundsKeys - 1) / kBoundsKeys;
  const int64_t cap = (int64_t)1 << 20;    // grid-stride loops beyond this many blocks
  knorm_vcheck_kernel<T><<<dim3((unsigned)(kb < cap ? kb : cap), (unsigned)a.B, groups), 256, 0, s>>>(a);
  qnorm_kernel<T><<<dim3((unsigned)(qb < cap ? qb : cap), (unsigned)a.B, groups), 256, 0, s>>>(a);
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
