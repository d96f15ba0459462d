// Exact sums of fp32 / bf16 values, rounded once to fp64: the key sum behind the global key
// mean of [UR] Summary ("Global Virtual K-Centering"), made independent of summation order.
//
// A fixed-point accumulator for fp64 values that are integer multiples of 2^-149 (every fp32
// or bf16 value, and every exact sum of them) and below 2^166 in magnitude (at most 2^38
// keys below 2^128 each): kLimbs signed 64-bit limbs, limb i holding a 32-bit digit of
// weight 2^(32 i - 149) plus carries.  An addition touches three consecutive limbs with
// parts below 2^33, so 2^29 additions between normalisations cannot overflow a limb.
// Plain C++ (host and device), so the CPU tests can check it against exact rationals.
#pragma once
#include <math.h>
#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define FIXEDM_HD __host__ __device__
#else
#define FIXEDM_HD
#endif

namespace fixedm {

constexpr int kLimbs = 11;

FIXEDM_HD inline uint64_t f64_bits(double x) {
  uint64_t u;
  __builtin_memcpy(&u, &x, sizeof u);
  return u;
}

// lim += p, exactly.  p must be 0 or a nonzero multiple of 2^-149 below 2^166 in magnitude.
FIXEDM_HD inline void exact_add(int64_t* lim, double p) {
  if (p == 0.0) return;
  const uint64_t bits = f64_bits(p);
  const int e = (int)((bits >> 52) & 0x7ff);
  uint64_t mant = (bits & 0xfffffffffffffull) | (1ull << 52);   // p = mant 2^(e - 1075)
  int sh = e - 1075 + 149;                     // position of mant's lowest bit above 2^-149
  if (sh < 0) {                                // the bits shifted out are zero (p is a
    mant >>= -sh;                              // multiple of 2^-149)
    sh = 0;
  }
  const int L = sh >> 5, r = sh & 31;
  const uint64_t lo = (mant & 0xffffffffull) << r;   // below 2^63
  const uint64_t hi = (mant >> 32) << r;             // below 2^52
  const int64_t d0 = (int64_t)(lo & 0xffffffffull);
  const int64_t d1 = (int64_t)((lo >> 32) + (hi & 0xffffffffull));
  const int64_t d2 = (int64_t)(hi >> 32);
  if (bits >> 63) {
    lim[L] -= d0;
    lim[L + 1] -= d1;
    lim[L + 2] -= d2;
  } else {
    lim[L] += d0;
    lim[L + 1] += d1;
    lim[L + 2] += d2;
  }
}

// Carries each limb's excess into the next: limbs 0 .. kLimbs-2 become digits in [0, 2^32),
// the top limb keeps the sign.  The value is unchanged.
FIXEDM_HD inline void exact_normalize(int64_t* lim) {
  for (int i = 0; i + 1 < kLimbs; ++i) {
    const int64_t c = lim[i] >> 32;            // floor(lim[i] / 2^32)
    lim[i] -= c * 4294967296ll;
    lim[i + 1] += c;
  }
}

// The accumulated value rounded to the nearest fp64, ties to even.  Destroys lim.
FIXEDM_HD inline double exact_round(int64_t* lim) {
  exact_normalize(lim);
  const bool neg = lim[kLimbs - 1] < 0;
  if (neg) {
    for (int i = 0; i < kLimbs; ++i) lim[i] = -lim[i];
    exact_normalize(lim);
  }
  int T = kLimbs - 1;
  while (T >= 0 && lim[T] == 0) --T;
  if (T < 0) return 0.0;
  // 96-bit window of limbs T, T-1, T-2 (missing limbs are 0): bit k of H sits at position
  // 32 (T - 1) + k above 2^-149.  lim[T] is a nonzero digit below 2^32 (the accumulated
  // magnitude stays below 2^166, far under the top limb's weight), so H's leading bit lies
  // in its upper half: lz <= 31.
  const uint64_t top = (uint64_t)lim[T];
  const uint64_t mid = T >= 1 ? (uint64_t)lim[T - 1] : 0ull;
  const uint64_t low = T >= 2 ? (uint64_t)lim[T - 2] : 0ull;
  bool sticky = false;
  for (int i = 0; i + 2 < T; ++i) sticky = sticky || lim[i] != 0;
  uint64_t H = (top << 32) | mid;
  uint64_t Lw = low << 32;
  const int lz = __builtin_clzll(H);
  if (lz > 0) {                                // bring the leading bit to bit 63
    H = (H << lz) | (Lw >> (64 - lz));
    Lw <<= lz;
  }
  const int msb = 32 * T + 31 - lz;            // position of the leading bit above 2^-149
  uint64_t mant = H >> 11;                     // the 53 leading bits
  const bool round = ((H >> 10) & 1ull) != 0;
  sticky = sticky || (H & 0x3ffull) != 0 || Lw != 0;
  if (round && (sticky || (mant & 1ull))) mant += 1;   // a carry to 2^53 stays exact below
  const double v = ldexp((double)mant, msb - 52 - 149);
  return neg ? -v : v;
}

}  // namespace fixedm
