// bf16 GELU(tanh) of the activation passes: the fp32 definition, evaluated
// at compile time for the bf16 inputs where it is not trivial, and the
// branch-free lookup from an LDS copy of that band.
#pragma once

#include <stdint.h>

#include "common.h"

namespace svdq {

// GELU with the tanh approximation in the cancellation-free form
//   GELU(x) = x / (1 + e^z),  z = -2 sqrt(2/pi) (x + 0.044715 x^3)
// (0.5 (1 + tanh y) = 1 / (1 + e^-2y)), every step one IEEE fp32 operation
// with round-to-nearest-even and no fused multiply-add, so that the bf16
// rounding of the result, which decides the 4-bit codes, is reproducible.
// e^z uses Cody and Waite's reduction z = k ln2 + r with ln 2 split as
// 0.693359375 (10 significant bits, so k * 0.693359375 is exact) plus the
// fp32 remainder, a degree-7 Taylor polynomial of e^r in Horner form and
// exact scaling by 2^k; z is clamped to [-104, 104].
//
// The input is bf16, so the function has 65536 arguments: the table below
// holds bf16_RNE(GELU(x)) for every bf16 bit pattern, evaluated by the
// compiler's constant evaluator, whose float arithmetic is IEEE with
// round-to-nearest-even, one rounding per operation.  Constant evaluation
// admits no infinities, so the two places where the fp32 sequence overflows
// take their results directly: x^3 overflows only when |x| > 2^42, where
// z is clamped to -104 (x > 0: e^z = 0 in fp32, GELU = x) or to +104
// (x < 0: e^z = inf, GELU = -0); and p 2^k rounds to inf in fp32 exactly
// when it reaches 2^128 - 2^103, where GELU = x / inf = -0 (z > 0 there, so
// x < 0).  Inf and NaN inputs map to themselves.
namespace gelu_table {

constexpr double kLn2 = 0.69314718055994530942;
constexpr float kA = (float)0.044715;
constexpr float kC1 = 0.693359375f;
constexpr float kC2 = (float)(kLn2 - 0.693359375);
constexpr float kL = (float)(1.0 / kLn2);

constexpr double csqrt(double v) {  // Newton's iteration to the correctly rounded root
  double r = v > 1.0 ? v : 1.0;
  for (int i = 0; i < 200; ++i) r = 0.5 * (r + v / r);
  // the iteration settles within one ulp; step to the root whose square is closest
  for (int i = 0; i < 4; ++i) {
    const double lo = r - r * 0x1p-53, hi = r + r * 0x1p-52;
    const double e0 = r * r - v, el = lo * lo - v, eh = hi * hi - v;
    const double a0 = e0 < 0 ? -e0 : e0, al = el < 0 ? -el : el, ah = eh < 0 ? -eh : eh;
    r = al < a0 ? lo : (ah < a0 ? hi : r);
  }
  return r;
}
constexpr float kB = (float)(-2.0 * csqrt(2.0 / 3.14159265358979323846));

constexpr float rint_even(float v) {  // round to an integer, ties to even (|v| < 2^23)
  const float a = v < 0 ? -v : v;
  const float t = (a + 8388608.0f) - 8388608.0f;
  return v < 0 ? -t : t;
}
constexpr double pow2(int k) {  // 2^k for -1022 <= k <= 1023, from its exponent field
  return __builtin_bit_cast(double, (uint64_t)(k + 1023) << 52);
}
constexpr uint16_t bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
constexpr uint16_t entry(uint32_t xb) {
  if ((xb & 0x7F80u) == 0x7F80u) return (uint16_t)xb;           // inf, NaN
  const float x = __builtin_bit_cast(float, xb << 16);
  const float ax = x < 0 ? -x : x;
  if (ax > 0x1p42f) return x > 0 ? (uint16_t)xb : (uint16_t)0x8000u;
  const float x3 = (x * x) * x;
  const float u = x + kA * x3;
  float z = kB * u;
  z = z < -104.0f ? -104.0f : (z > 104.0f ? 104.0f : z);
  const float k = rint_even(z * kL);
  const float r = (z - k * kC1) - k * kC2;
  float p = (float)(1.0 / 5040.0);
  p = p * r + (float)(1.0 / 720.0);
  p = p * r + (float)(1.0 / 120.0);
  p = p * r + (float)(1.0 / 24.0);
  p = p * r + (float)(1.0 / 6.0);
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const double v = (double)p * pow2((int)k);                  // exact
  if (v >= 0x1p128 - 0x1p103) return (uint16_t)0x8000u;       // e^z = inf, x < 0
  const float e = (float)v;                                   // one rounding
  return bf16_rne(x / (1.0f + e));
}
// Outside a band of exponents the bf16 GELU follows two rules, checked
// against the full definition for all 65536 inputs below: |x| < 2^-10 gives
// bf16_RNE(x / 2) (there e^z = 1 - 1.6 x + ..., so x / (1 + e^z) is within
// 2^-10 of x / 2, inside half a bf16 ulp), and |x| >= 32 gives x for
// positive x and -0 for negative x (inf and NaN map to themselves).  Only the
// 15 binades in between (biased exponents 117..131, both signs: 3840
// entries) are tabulated.
constexpr int kLoExp = 117, kHiExp = 131;
constexpr int kBand = kHiExp - kLoExp + 1;
constexpr int kEntries = 2 * kBand * 128;

constexpr uint16_t half_rule(uint32_t xb) {
  return bf16_rne(__builtin_bit_cast(float, xb << 16) * 0.5f);
}
constexpr uint16_t rule(uint32_t xb) {  // inputs outside the band
  const uint32_t e = (xb >> 7) & 0xFFu;
  if (e < (uint32_t)kLoExp) return half_rule(xb);
  if (e == 0xFFu || (xb & 0x8000u) == 0) return (uint16_t)xb;
  return (uint16_t)0x8000u;
}
constexpr int band_index(uint32_t xb) {
  return (int)((xb >> 15) * kBand + (((xb >> 7) & 0xFFu) - kLoExp)) * 128 + (int)(xb & 0x7Fu);
}
constexpr bool rules_hold() {
  for (uint32_t i = 0; i < 65536; ++i) {
    const uint32_t e = (i >> 7) & 0xFFu;
    if ((e < (uint32_t)kLoExp || e > (uint32_t)kHiExp) && rule(i) != entry(i)) return false;
  }
  return true;
}
static_assert(rules_hold(), "the GELU rules outside the tabulated band");

struct Table {
  uint16_t v[kEntries];
};
constexpr Table make() {
  Table t{};
  for (uint32_t s = 0; s < 2; ++s)
    for (uint32_t e = kLoExp; e <= (uint32_t)kHiExp; ++e)
      for (uint32_t m = 0; m < 128; ++m) {
        const uint32_t xb = (s << 15) | (e << 7) | m;
        t.v[band_index(xb)] = entry(xb);
      }
  return t;
}

// The activation pass's wider band: |x| in [2^-24, 2^14) (biased exponents
// 103..140), where nearly every activation falls, so that the rules above
// are needed only for zeros, tiny or huge values, which the pass handles on
// a rarely taken branch.  Per sign: 38 binades of 128 entries, then one
// sentinel entry, the index that every out-of-band input is clamped to.
constexpr int kWLoExp = 103, kWHiExp = 140;
constexpr int kWBand = kWHiExp - kWLoExp + 1;
constexpr int kWHalf = kWBand * 128 + 1;
constexpr int kWEntries = 2 * kWHalf;
static_assert(kWLoExp <= kLoExp && kWHiExp >= kHiExp, "the rules hold outside the wide band");
struct WideTable {
  uint16_t v[kWEntries];
};
constexpr WideTable make_wide() {
  WideTable t{};
  for (uint32_t s = 0; s < 2; ++s)
    for (uint32_t e = kWLoExp; e <= (uint32_t)kWHiExp; ++e)
      for (uint32_t m = 0; m < 128; ++m) {
        const uint32_t xb = (s << 15) | (e << 7) | m;
        t.v[s * kWHalf + (e - kWLoExp) * 128 + m] = entry(xb);
      }
  return t;
}

}  // namespace gelu_table

__device__ constexpr gelu_table::Table kGeluBand = gelu_table::make();
__device__ constexpr gelu_table::WideTable kGeluWide = gelu_table::make_wide();

// bf16 GELU of one input (low 16 bits of b) from the band table in LDS and
// the two rules.  Branch-free: the table index is clamped into range.
__device__ __forceinline__ uint32_t gelu_one(uint32_t b, const uint16_t* tab) {
  using namespace gelu_table;
  const uint32_t e = (b >> 7) & 0xFFu;
  const bool in_band = e >= (uint32_t)kLoExp && e <= (uint32_t)kHiExp;
  const uint32_t ec = in_band ? e : (uint32_t)kLoExp;
  const uint32_t idx = ((b >> 15) * kBand + (ec - kLoExp)) * 128 + (b & 0x7Fu);
  const uint32_t t = tab[idx];
  const uint32_t half = f32_to_bf16(__uint_as_float(b << 16) * 0.5f);
  const uint32_t big = (e == 0xFFu || (b & 0x8000u) == 0) ? b : 0x8000u;
  return in_band ? t : (e < (uint32_t)kLoExp ? half : big);
}

__device__ __forceinline__ uint32_t gelu_bf16x2(uint32_t w, const uint16_t* tab) {
  return gelu_one(w & 0xFFFFu, tab) | (gelu_one(w >> 16, tab) << 16);
}

// The bf16 GELU of the inputs outside the wide band (low 16 bits of b):
// |x| < 2^-24 (zeros included) gives bf16_RNE(x / 2), |x| >= 2^14 gives x
// for positive x and -0 for negative x; inf and NaN map to themselves.
__device__ __forceinline__ uint32_t gelu_rule(uint32_t b) {
  const uint32_t e = (b >> 7) & 0xFFu;
  const uint32_t half = f32_to_bf16(__uint_as_float(b << 16) * 0.5f);
  const uint32_t big = (e == 0xFFu || (b & 0x8000u) == 0) ? b : 0x8000u;
  return e < (uint32_t)gelu_table::kWLoExp ? half : big;
}

}  // namespace svdq
