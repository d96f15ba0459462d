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
// are exact in fp64.  Maxima are order-free.  The key sum behind k_mean is EXACT, rounded
// once to fp64, then divided by N in fp64 and rounded to fp32, so no summation order enters:
// the key-slab partial sums run in fp64 with every addition checked for exactness (TwoSum),
// the exact partials are combined in a fixed-point accumulator, and any element whose
// partial sums were not exact is summed again, key by key, in that accumulator.
// U = alpha64 * sqrt(Q2 * K2) in exactly that order.
#include <math.h>

#include <atomic>

#include "exact_sum.h"
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

// Partial key sums for the COMPUTE centring mode.  Workgroup (w, b, head group) of a grid of
// kslabs: thread (hl, c) owns dims 8c..8c+7 of head h0 + hl and adds, in key order, the keys
// of blocks w, w + kslabs, w + 2 kslabs, ... (8 keys a block).  A key's rows of the head group
// are adjacent in memory, so each key is one contiguous read of the workgroup, and the
// workgroups in flight stream one contiguous window of keys.
//
// Exactness: the thread also keeps, per element, the largest |x| and the smallest nonzero |x|
// of its keys (integer max / min of the magnitude bits, which order like the values; packed
// 16-bit ops for bf16).  Every key is then a multiple of the smallest one's unit in the last
// place, and every partial sum of n keys, in any order, stays below n max|x|; when that is
// below 2^53 such units, every fp64 addition was exact.  Otherwise (keys spanning many
// binades, a NaN or an infinity) the element is flagged for the exact re-summation.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct MagRange;                     // largest and smallest-nonzero magnitude bits per element
template <>
struct MagRange<uint16_t> {
  static constexpr int kMant = 7;    // explicit mantissa bits of bf16
  u16x2 mx[4], mn[4];                // element 2 i + half in word i
  __device__ void init() {
    for (int i = 0; i < 4; ++i) { mx[i] = u16x2{0, 0}; mn[i] = u16x2{0xffff, 0xffff}; }
  }
  __device__ void add(const uint32_t (&w)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u16x2 m = __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu);
      mx[i] = __builtin_elementwise_max(mx[i], m);
      mn[i] = __builtin_elementwise_min(mn[i], (u16x2)(m - (u16x2){1, 1}));   // 0 wraps to 0xffff
    }
  }
  __device__ uint32_t hi(int e) const { return mx[e >> 1][e & 1]; }
  __device__ uint32_t lo1(int e) const { return mn[e >> 1][e & 1]; }   // min nonzero - 1
  static constexpr uint32_t kNone = 0xffffu;
  __device__ static int exp_field(uint32_t m) { return (int)(m >> kMant); }
};
template <>
struct MagRange<float> {
  static constexpr int kMant = 23;
  uint32_t mx[8], mn[8];
  __device__ void init() {
    for (int i = 0; i < 8; ++i) { mx[i] = 0; mn[i] = 0xffffffffu; }
  }
  __device__ void add(const uint32_t (&w)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t m = w[i] & 0x7fffffffu;
      mx[i] = max(mx[i], m);
      mn[i] = min(mn[i], m - 1u);
    }
  }
  __device__ uint32_t hi(int e) const { return mx[e]; }
  __device__ uint32_t lo1(int e) const { return mn[e]; }
  static constexpr uint32_t kNone = 0xffffffffu;
  __device__ static int exp_field(uint32_t m) { return (int)(m >> kMant); }
};

template <typename T>
__global__ __launch_bounds__(1024) void kmean_partial_kernel(BoundsArgs a) {
  // This pass runs first: it clears what the later passes reduce into (the Q and K norm
  // maxima and the V record), so no separate initialising launch is needed.
  {
    const int64_t nth = (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
    const int64_t t0 = (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x +
                       threadIdx.x;
    const int64_t nqb_all = (int64_t)a.B * a.H * a.nqb;
    for (int64_t t = t0; t < nqb_all; t += nth) a.q2[t] = 0ull;
    for (int64_t t = t0; t < (int64_t)a.B * a.H; t += nth) a.k2[t] = 0ull;
    if (t0 == 0) *a.v_bad = 0;
  }
  const int per = a.D / 8;
  const int hl = threadIdx.x / per, c = threadIdx.x % per;
  const int b = blockIdx.y, h = blockIdx.z * kBoundsHeads + hl;
  if (h >= a.H) return;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  MagRange<T> mag;
  mag.init();
  int64_t count = 0;                             // keys this thread adds
  int ci = 0;                                    // chunk of the current key (uniform)
  const int64_t stride = (int64_t)a.kslabs * 8;
  // The workgroup's blocks of 8 keys, software-pipelined: the next block's loads are in flight
  // while the current one is added (raw 16-byte words until then), keys in order.
  constexpr int kW = (int)sizeof(T) / 2;
  const auto load_block = [&](int64_t j, uint4 (&raw)[8][kW]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t jj = j + u;
      if (jj < a.N) {
        while (ci + 1 < a.n_chunks && jj >= a.ch[ci + 1].start) ++ci;
        const ChunkDesc& cd = a.ch[ci];
        const uint4* src = reinterpret_cast<const uint4*>(
            reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + (jj - cd.start) * cd.k_ss + h * cd.k_sh + 8 * c);
#pragma unroll
        for (int w = 0; w < kW; ++w) raw[u][w] = src[w];
      }
    }
  };
  uint4 cur[8][kW], nxt[8][kW];
  int64_t j = (int64_t)blockIdx.x * 8;
  if (j < a.N) load_block(j, cur);
  for (; j < a.N; j += stride) {
    if (j + stride < a.N) load_block(j + stride, nxt);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j + u < a.N) {
        float f[8];
        ++count;
        if constexpr (sizeof(T) == 2) {
          const uint32_t x[4] = {cur[u][0].x, cur[u][0].y, cur[u][0].z, cur[u][0].w};
          mag.add(x);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(x[i] << 16);
            f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
          }
        } else {
          const uint32_t x[8] = {cur[u][0].x, cur[u][0].y, cur[u][0].z, cur[u][0].w,
                                 cur[u][kW - 1].x, cur[u][kW - 1].y, cur[u][kW - 1].z, cur[u][kW - 1].w};
          mag.add(x);
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(x[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + (double)f[i];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int w = 0; w < kW; ++w) cur[u][w] = nxt[u][w];
  }
  // ceil(log2 count): partial sums stay below 2^lc max|x|
  int lc = 0;
  while (((int64_t)1 << lc) < count) ++lc;
  const int64_t el = ((int64_t)b * a.H + h) * a.D + 8 * c;
  const int64_t slab = (int64_t)blockIdx.x * a.B * a.H * a.D;
  double* dst = a.kpart + slab + el;
  uint8_t* flag = a.kflag + slab + el;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dst[i] = acc[i];
    const uint32_t lo1 = mag.lo1(i), hi = mag.hi(i);
    bool inexact = false;                                    // no nonzero key: the sum is 0
    if (lo1 != MagRange<T>::kNone) {
      const int emax = MagRange<T>::exp_field(hi), emin = MagRange<T>::exp_field(lo1 + 1);
      // |x| < 2^(max(emax,1) - 126) and x a multiple of 2^(max(emin,1) - 127 - mant):
      // exact while max(emax,1) - 126 + lc <= max(emin,1) - 127 - mant + 53
      const bool nonfinite = emax == 255;
      const int top = (emax > 1 ? emax : 1) + lc, room = (emin > 1 ? emin : 1) + 52 - MagRange<T>::kMant;
      inexact = nonfinite || top > room;
    }
    flag[i] = inexact ? 1 : 0;
  }
}

// k_mean[b,h,d] = fp32(fl64(exact key sum) / N).  Workgroup of 256 threads = kFinG groups x
// kFinE elements: thread (g, e) adds the partials of slabs g, g + kFinG, ... of element e into its own
// fixed-point accumulator in LDS (exact, so no order enters; a partial whose slab flagged it
// is skipped: it may not be exact, or even finite).  When no slab flagged the element, its
// kFinG accumulators are added and rounded once.  Otherwise (a slab sum that was not exact, or a
// non-finite key) the element's keys are re-summed one by one: thread (g, e) takes the keys
// g, g + kFinG, ... of every chunk (the elements of a workgroup are adjacent dims, so each key
// is one contiguous read).  A NaN, or both infinities, give NaN; otherwise an infinity gives
// itself.
constexpr int kFinG = 16, kFinE = 256 / kFinG;
template <typename T>
__global__ __launch_bounds__(256) void kmean_final_kernel(BoundsArgs a) {
  __shared__ int64_t lim[kFinG][kFinE][kLimbs];
  __shared__ uint32_t st[kFinG][kFinE];
  const int64_t n = (int64_t)a.B * a.H * a.D;
  const int g = threadIdx.x / kFinE, el = threadIdx.x % kFinE;
  const int64_t i = (int64_t)blockIdx.x * kFinE + el;
  const bool valid = i < n;
  int64_t* acc = lim[g][el];
  for (int k = 0; k < kLimbs; ++k) acc[k] = 0;
  uint32_t flagged = 0;
  if (valid) {
    int sl = g;
    for (; sl + 7 * kFinG < a.kslabs; sl += 8 * kFinG) {      // eight partials in flight
      double x[8];
      uint32_t f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[u] = a.kpart[(int64_t)(sl + kFinG * u) * n + i];
        f[u] = a.kflag[(int64_t)(sl + kFinG * u) * n + i];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        flagged |= f[u];
        if (f[u] == 0) exact_add(acc, x[u]);
      }
    }
    for (; sl < a.kslabs; sl += kFinG) {
      const uint32_t f = a.kflag[(int64_t)sl * n + i];
      flagged |= f;
      if (f == 0) exact_add(acc, a.kpart[(int64_t)sl * n + i]);
    }
  }
  st[g][el] = flagged;
  const bool any_in_group = __syncthreads_or(flagged != 0) != 0;
  uint32_t mine = 0;                               // some slab flagged this thread's element
  for (int gg = 0; gg < kFinG; ++gg) mine |= st[gg][el];
  if (g == 0 && valid && mine == 0) {
    int64_t tot[kLimbs];
    for (int k = 0; k < kLimbs; ++k) {
      int64_t t = 0;
      for (int gg = 0; gg < kFinG; ++gg) t += lim[gg][el][k];
      tot[k] = t;
    }
    a.k_mean[i] = (float)(exact_round(tot) / (double)a.N);
  }
  if (!any_in_group) return;                       // the whole workgroup: nothing flagged
  __syncthreads();                                 // every read of st and lim above is done
  uint32_t bits = 0;                               // 1: NaN, 2: +inf, 4: -inf
  if (valid && mine != 0) {
    for (int k = 0; k < kLimbs; ++k) acc[k] = 0;
    const int64_t bh = i / a.D, d = i % a.D, b = bh / a.H, h = bh % a.H;
    int64_t since = 0;
    for (int c = 0; c < a.n_chunks; ++c) {
      const ChunkDesc& cd = a.ch[c];
      const T* col = reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + h * cd.k_sh + d;
      for (int64_t j = g; j < cd.len; j += kFinG) {
        const double x = (double)load_elem(col + j * cd.k_ss);
        if (isnan(x)) bits |= 1u;
        else if (isinf(x)) bits |= x > 0 ? 2u : 4u;
        else exact_add(acc, x);
        if (++since == ((int64_t)1 << 28)) {
          exact_normalize(acc);
          since = 0;
        }
      }
    }
  }
  st[g][el] = bits;
  __syncthreads();
  if (g == 0 && valid && mine != 0) {
    uint32_t all = 0;
    int64_t tot[kLimbs];
    for (int k = 0; k < kLimbs; ++k) tot[k] = 0;
    for (int gg = 0; gg < kFinG; ++gg) {
      all |= st[gg][el];
      exact_normalize(lim[gg][el]);                // each group's limbs into digits first
      for (int k = 0; k < kLimbs; ++k) tot[k] += lim[gg][el][k];
    }
    double sum;
    if ((all & 1u) || (all & 6u) == 6u) sum = __longlong_as_double(0x7ff8000000000000ll);
    else if (all & 2u) sum = __longlong_as_double(0x7ff0000000000000ll);
    else if (all & 4u) sum = -__longlong_as_double(0x7ff0000000000000ll);
    else sum = exact_round(tot);
    a.k_mean[i] = (float)(sum / (double)a.N);
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

// The norm kernels give each wave 64 consecutive rows (keys or query positions) of one
// head.  The wave reads them with coalesced 16-byte loads (P = D sizeof(T) / 16 lanes per
// row), stores them to its LDS area with the piece index XOR-swizzled by the row, and each
// lane then reads back its own row (bank-conflict free both ways) and sums it in index order.
template <typename T>
struct NormGeom {
  static constexpr int kMaxP = 128 * (int)sizeof(T) / 16;   // pieces per row at D = 128
  static constexpr int kWaves = sizeof(T) == 2 ? 4 : 2;       // 64 KB of staging per workgroup
};

// Row pointer of key j, head h, batch b, in K or V, for a key known to lie in chunks c0..c1
// (a wave-uniform range: the chunk is selected without divergent indexing).
template <typename T>
__device__ inline const T* key_row(const BoundsArgs& a, int b, int h, int64_t j, int c0, int c1, bool v) {
  const T* p = nullptr;
  for (int c = c0; c <= c1; ++c) {
    const ChunkDesc& cd = a.ch[c];
    if (j >= cd.start)
      p = v ? reinterpret_cast<const T*>(cd.v) + b * cd.v_sb + (j - cd.start) * cd.v_ss + h * cd.v_sh
            : reinterpret_cast<const T*>(cd.k) + b * cd.k_sb + (j - cd.start) * cd.k_ss + h * cd.k_sh;
  }
  return p;
}

// The largest |x| of a 16-byte piece as fp32 bits: the magnitude bits order finite values by
// size and put inf and NaN above them all.  Branch free (a short-circuit test branches on
// divergent lanes).  Every |x| <= 256 exactly when the result is <= kV256Bits.
constexpr uint32_t kV256Bits = 0x43800000u;   // 256.0f
__device__ inline uint32_t piece_maxabs(uint4 w, const uint16_t*) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = u[i] & 0x7fffu, hi = (u[i] >> 16) & 0x7fffu;
    m = max(m, max(lo, hi));
  }
  return m << 16;
}
__device__ inline uint32_t piece_maxabs(uint4 w, const float*) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, u[i] & 0x7fffffffu);
  return m;
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Records a V magnitude over the bound: v_bad keeps the fp32 bits of the largest |v| seen
// (positive as an int32), so it is nonzero exactly when some |v| > 256 or is not a number.
__device__ inline void note_v_max(const BoundsArgs& a, uint32_t wave_max) {
  if (wave_max > kV256Bits) atomicMax(a.v_bad, (int32_t)wave_max);
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Loads the P pieces lane `lane` owns of the wave's rows: piece lane mod P of rows
// lane / P + i 64 / P.  Rows past nrows repeat row nrows - 1 (every load is in bounds and
// unconditional; those rows are never summed).  row(r) gives a row's pointer.
template <int P, typename RowFn>
__device__ inline void load_pieces(uint4 (&v)[P], int nrows, int lane, RowFn row) {
  const int pc = lane % P;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    int r = lane / P + i * (64 / P);
    r = r < nrows ? r : nrows - 1;
    v[i] = reinterpret_cast<const uint4*>(row(r))[pc];
  }
}

// Stores the pieces to the wave's LDS area (piece pc of row r at slot r P + (pc ^ (r mod P)))
// and reads back row `lane` into out[0..P).
template <int P>
__device__ inline void transpose_rows(const uint4 (&v)[P], uint4* area, int lane, uint4* out) {
  const int pc = lane % P;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int r = lane / P + i * (64 / P);
    area[r * P + (pc ^ (r % P))] = v[i];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int q = 0; q < P; ++q) out[q] = area[lane * P + (q ^ (lane % P))];
}

// 256 keys of one (b, h) per workgroup, one key per thread: K2 = max over keys of
// sum_d (k_d - k_mean_d)^2 (fp64, d in order; k_mean staged in LDS as fp64), and the
// V-magnitude check on the same keys' value rows.  (A coalesced-load variant that
// transposes rows through LDS measured slower: the per-row fp64 work, not the load
// pattern, sets this kernel's pace.)
template <typename T>
__global__ __launch_bounds__(256) void knorm_vcheck_kernel(BoundsArgs a) {
  __shared__ double km[128];
  __shared__ unsigned long long wmax[4];
  __shared__ uint32_t wvmax[4];
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * 256 + tid;
  if (tid < a.D) km[tid] = (double)a.k_mean[(int64_t)bh * a.D + tid];
  __syncthreads();
  unsigned long long best = 0ull;
  uint32_t vmax = 0;
  if (j < a.N) {
    const int c = find_chunk(a, j);
    RowRegs<T> kr, vr;
    kr.load(key_row<T>(a, b, h, j, c, c, false), a.D);
    vr.load(key_row<T>(a, b, h, j, c, c, true), a.D);
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < 128; ++d) {
      if (d < a.D) {
        const double t = (double)kr.elem(d) - km[d];
        s = s + t * t;
      }
    }
    best = (unsigned long long)__double_as_longlong(s);
#pragma unroll
    for (int i = 0; i < RowRegs<T>::kPieces; ++i)
      if (i < a.D * (int)sizeof(T) / 16) vmax = max(vmax, piece_maxabs(vr.p[i], (const T*)nullptr));
  }
  best = wave_max_u64(best);
  vmax = wave_max_u32(vmax);
  const int w = tid >> 6;
  if ((tid & 63) == 0) { wmax[w] = best; wvmax[w] = vmax; }
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = wmax[0];
    uint32_t vm = wvmax[0];
    for (int i = 1; i < 4; ++i) { m = wmax[i] > m ? wmax[i] : m; vm = max(vm, wvmax[i]); }
    atomicMax(a.k2 + bh, m);
    note_v_max(a, vm);
  }
}

// bf16 K2 and V check (D = 128), one persistent workgroup per compute unit.  Each wave takes a
// contiguous range of work items (b, h, block of up to 64 keys of one chunk; ordered by (b, h),
// so a wave keeps its head and its k_mean for many items).  The K rows of an item arrive in
// the wave's LDS stage by direct global->LDS loads, four whole 256-byte rows per instruction
// (lane L of instruction i: row 4 i + L / 16, the 16-byte chunk (L mod 16) ^ (row mod 16) so
// that each lane reads its own row back bank-conflict free); the V rows come the same way
// into registers and are checked where they land.  Two stages per wave: the loads of item k+1
// are issued before the fp64 sums of item k.  (One key per lane reading its own rows from
// HBM was bound by its load pattern: each instruction touched 64 rows a key stride apart.)
__global__ __launch_bounds__(256, 1) void knorm_vcheck_lds_kernel(BoundsArgs a) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) uint4 kst[4][2][64 * 16];
  __shared__ double kmd[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t n_kb = 0;
  for (int c = 0; c < a.n_chunks; ++c) n_kb += (a.ch[c].len + 63) / 64;
  const int64_t n_items = (int64_t)a.B * a.H * n_kb;
  const int64_t G = (int64_t)gridDim.x * 4, g = (int64_t)blockIdx.x * 4 + wave;
  const int64_t i0 = n_items * g / G, i1 = n_items * (g + 1) / G;
  if (i0 >= i1) return;
  // item -> (b, h), chunk, block of the chunk, rows
  struct Item {
    int64_t bh;
    const uint16_t* k0;
    const uint16_t* v0;
    int64_t kss, vss;
    int nrows;
  };
  const auto locate = [&](int64_t item) {
    Item it;
    it.bh = item / n_kb;
    int64_t kb = item % n_kb;
    int c = 0;
    while (kb >= (a.ch[c].len + 63) / 64) {
      kb -= (a.ch[c].len + 63) / 64;
      ++c;
    }
    const ChunkDesc& cd = a.ch[c];
    const int64_t b = it.bh / a.H, h = it.bh % a.H;
    it.k0 = reinterpret_cast<const uint16_t*>(cd.k) + b * cd.k_sb + kb * 64 * cd.k_ss + h * cd.k_sh;
    it.v0 = reinterpret_cast<const uint16_t*>(cd.v) + b * cd.v_sb + kb * 64 * cd.v_ss + h * cd.v_sh;
    it.kss = cd.k_ss;
    it.vss = cd.v_ss;
    it.nrows = cd.len - kb * 64 < 64 ? (int)(cd.len - kb * 64) : 64;
    return it;
  };
  // issues item `it`'s K rows into stage `st` and its V rows into vv (rows past nrows repeat
  // row nrows - 1: every load is in bounds)
  const auto issue = [&](const Item& it, int st, uint4 (&vv)[16]) {
    const int q = lane >> 4, pc = lane & 15;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int r = 4 * i + q;
      r = r < it.nrows ? r : it.nrows - 1;
      const uint16_t* src = it.k0 + r * it.kss + 8 * (pc ^ ((4 * i + q) & 15));
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&kst[wave][st][64 * i], 16, 0,
                                       0);
      vv[i] = *reinterpret_cast<const uint4*>(it.v0 + r * it.vss + 8 * pc);
    }
  };
  uint32_t vmax = 0;
  int64_t cur_bh = -1;
  unsigned long long best = 0ull;
  uint4 vv[16];
  Item it = locate(i0);
  issue(it, 0, vv);
  for (int64_t item = i0; item < i1; ++item) {
    const int st = (int)((item - i0) & 1);
    if (it.bh != cur_bh) {   // a new head: flush the previous head's max, stage this one's k_mean
      if (cur_bh >= 0) {
        const unsigned long long m = wave_max_u64(best);
        if (lane == 0) atomicMax(a.k2 + cur_bh, m);
      }
      best = 0ull;
      cur_bh = it.bh;
      for (int d = lane; d < D; d += 64) kmd[wave][d] = (double)a.k_mean[cur_bh * D + d];
    }
    // this item's loads have landed (the compiler waits for them before the LDS reads below)
#pragma unroll
    for (int i = 0; i < 16; ++i) vmax = max(vmax, piece_maxabs(vv[i], (const uint16_t*)nullptr));
    RowRegs<uint16_t> kr;
#pragma unroll
    for (int p = 0; p < 16; ++p) kr.p[p] = kst[wave][st][lane * 16 + (p ^ (lane & 15))];
    const int nrows = it.nrows;
    if (item + 1 < i1) {       // the next item's loads, in flight during this item's sums
      it = locate(item + 1);
      issue(it, st ^ 1, vv);
    }
    double ss = 0.0;
#pragma unroll
    for (int gq = 0; gq < D / 32; ++gq) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const double t = (double)kr.elem(32 * gq + i) - kmd[wave][32 * gq + i];
        ss = ss + t * t;
      }
    }
    const unsigned long long v = lane < nrows ? (unsigned long long)__double_as_longlong(ss) : 0ull;
    best = v > best ? v : best;
  }
  const unsigned long long m = wave_max_u64(best);
  if (lane == 0) atomicMax(a.k2 + cur_bh, m);
  vmax = wave_max_u32(vmax);
  if (lane == 0) note_v_max(a, vmax);
}

// Q2[b,h,beta] = max over the block's real rows of sum_d q_d^2: work item (block of 64
// positions, head group), as in the K kernel; 64 positions lie in one q-block (q_block is
// a multiple of 64).
template <typename T, int P>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void qnorm_kernel(BoundsArgs a) {
  constexpr int W = NormGeom<T>::kWaves, D = P * 16 / (int)sizeof(T);
  __shared__ uint4 stage[W * 64 * P];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int64_t n_hq = (a.H + W - 1) / W, n_pb = (a.Sq + 63) / 64;
  uint4* area = stage + wave * 64 * P;
  for (int64_t item = blockIdx.x; item < n_pb * n_hq; item += gridDim.x) {
    const int h = (int)(item % n_hq) * W + wave;
    const int64_t i0 = item / n_hq * 64;
    if (h >= a.H) continue;
    const int nrows = a.Sq - i0 < 64 ? (int)(a.Sq - i0) : 64;
    const T* q0 = reinterpret_cast<const T*>(a.q) + b * a.q_sb + i0 * a.q_ss + h * a.q_sh;
    uint4 qv[P];
    load_pieces<P>(qv, nrows, lane, [&](int r) { return q0 + r * a.q_ss; });
    RowRegs<T> qr;
    transpose_rows<P>(qv, area, lane, qr.p);
    const double ss = row_sumsq<T>(qr, D);
    if (a.q2_row != nullptr && lane < nrows) a.q2_row[((int64_t)b * a.H + h) * a.Sq + i0 + lane] = ss;
    unsigned long long best = lane < nrows ? (unsigned long long)__double_as_longlong(ss) : 0ull;
    best = wave_max_u64(best);
    if (lane == 0) atomicMax(a.q2 + ((int64_t)b * a.H + h) * a.nqb + i0 / a.q_block, best);
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

// Per-row shifts: U_i = alpha64 * sqrt(Q2_i * K2); m_i = ceil(U_i) - C (the block formula on
// one row's norm; INT32_MAX when U_i is not finite or m_i leaves int32).
__global__ void gate_row_kernel(BoundsArgs a) {
  const int64_t n = (int64_t)a.B * a.H * a.Sq;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t bh = i / a.Sq;
  const double k2 = __longlong_as_double((long long)a.k2[bh]);
  const double u = __dmul_rn(a.alpha64, __dsqrt_rn(__dmul_rn(a.q2_row[i], k2)));
  int32_t m = INT32_MAX;
  if (isfinite(u)) {
    const double mc = ceil(u) - (double)a.C;
    if (mc >= -2147483648.0 && mc <= 2147483647.0) m = (int32_t)mc;
  }
  a.u_row[i] = u;
  a.m_row[i] = m;
}

template <typename T>
void launch_typed(const BoundsArgs& a, hipStream_t s) {
  const unsigned groups = (unsigned)((a.H + kBoundsHeads - 1) / kBoundsHeads);
  if (a.center == FIXEDM_CENTER_COMPUTE) {
    const int hpg = a.H < kBoundsHeads ? a.H : kBoundsHeads;
    kmean_partial_kernel<T><<<dim3((unsigned)a.kslabs, (unsigned)a.B, groups), hpg * (a.D / 8), 0, s>>>(a);
    const int64_t n = (int64_t)a.B * a.H * a.D;
    kmean_final_kernel<T><<<(unsigned)((n + kFinE - 1) / kFinE), 256, 0, s>>>(a);
  }
  constexpr int W = NormGeom<T>::kWaves;
  const int64_t n_hq = (a.H + W - 1) / W;
  const int64_t qitems = (a.Sq + 63) / 64 * n_hq;
  const int64_t cap = (int64_t)1 << 20;    // grid-stride loops beyond this many workgroups
  const dim3 gq((unsigned)(qitems < cap ? qitems : cap), (unsigned)a.B);
  if constexpr (sizeof(T) == 2) {
    const int cus = device_cus();
    knorm_vcheck_lds_kernel<<<(unsigned)(cus > 0 ? cus : 256), 256, 0, s>>>(a);
  } else {
    knorm_vcheck_kernel<T><<<dim3((unsigned)((a.N + 255) / 256), (unsigned)(a.B * a.H)), 256, 0, s>>>(a);
  }
  if constexpr (sizeof(T) == 4) {            // fp32: D = 64 (16 pieces a row) or 128 (32)
    if (a.D == 128) {
      qnorm_kernel<T, 32><<<gq, 64 * W, 0, s>>>(a);
      return;
    }
  }
  qnorm_kernel<T, 16><<<gq, 64 * W, 0, s>>>(a);   // bf16 D = 128, fp32 D = 64
}

}  // namespace

// Scratch of fixedm_bounds_static (the key-mean partial sums and their flags): one array per
// GPU, held for the life of the process.  In host code `scratch` names a host-side stand-in,
// not the device array: host code uses only the address hipGetSymbolAddress returns on each
// device.  Calls of fixedm_bounds_static that overlap on one GPU share it and race.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

void* static_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s) {
  const int64_t nqb_all = (int64_t)a.B * a.H * a.nqb;
  const int64_t nkm = (int64_t)a.B * a.H * a.D;
  const int64_t init_n = nqb_all > nkm ? nqb_all : nkm;
  const unsigned init_blocks = (unsigned)((init_n + 255) / 256 < 4096 ? (init_n + 255) / 256 : 4096);
  // (with the key mean computed, its first pass does the clearing)
  if (a.center != FIXEDM_CENTER_COMPUTE) bounds_init_kernel<<<init_blocks, 256, 0, s>>>(a);
  if (a.dtype == FIXEDM_BF16) launch_typed<uint16_t>(a, s);
  else launch_typed<float>(a, s);
  gate_kernel<<<(unsigned)((nqb_all + 255) / 256), 256, 0, s>>>(a);
  if (a.m_row != nullptr) {
    const int64_t rows = (int64_t)a.B * a.H * a.Sq;
    gate_row_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace fixedm
