// Activation side of the SVDQuant W4A4 linear on gfx950: smoothing, 4-bit
// quantization and the fused low-rank down-projection in one pass over X.
//
// The Nunchaku engine fuses the down-projection of the low-rank branch into
// the quantization kernel so that both branches share one read of the
// activations (apatero.com page, section "O que e Nunchaku e como acelera
// modelos Qwen").  Here a workgroup owns 16 rows of X; its eight waves take
// 64-column tiles round-robin, each prefetching its next tile.  In a tile,
// lane l holds row l%16 and the 16 columns 16*(l/16) .. +15, which is also
// the A-operand layout of two v_mfma_f32_16x16x32_bf16, so the smoothed
// bf16 values feed the MFMA straight from registers.  Per-group absmax is a
// xor-shuffle over the lanes that share a row.  The T partials of the eight
// waves are summed through LDS at the end.
//
// Exact quotients without a division per element.  Both quotients of the
// contract, fp32(x / lambda) and fp32(x_hat / s), divide a bf16 value
// (8 significant bits) by an fp32 value (24 bits).  Such a quotient is never
// an fp32 rounding midpoint (a 25-bit odd significand times a 24-bit one
// cannot have only 8 significant bits) and, when it is not, it lies at least
// about 2^-48 (relative) away from every midpoint, while fp64(a * fp64(1/b))
// is within 2^-52 of a/b.  So fp32(fp64(a * fp64(1/b))) is exactly the
// correctly rounded fp32(a / b) (checked on the host for every bf16 a against
// 20000 fp32 b, subnormals and all-ones significands included).  The fp64
// reciprocals of lambda are computed once per workgroup into LDS, the one of
// s once per lane and group.
//
// Outputs: the codes, scales and T in the documented row-major layouts
// (each optional) and/or the activation operand image the GEMM reads
// (image.h): the same codes re-encoded in MFMA lane order (INT4 as 6-bit
// E2M3 fields with the bf16-split scale operands, FP4 as stored with one
// scale byte per lane) and T split into bf16 high and low parts.  With an
// image the grid also covers the padding rows up to a multiple of 256, which
// come out as zeros.
#include "common.h"
#include "image.h"
#include "kernels.h"
#include "nvfp4_codec.h"

namespace svdq {

constexpr int QA_ROWS = 16;
constexpr int QA_KCHUNK = 4096;  // columns whose reciprocals of lambda sit in LDS at once

// Waves per 16-row workgroup: INT4 16 (four per SIMD, to keep more of X in
// flight) unless the T partials of a large rank would not fit in LDS; FP4 8
// (measured faster).
template <int MODE, int RB>
struct QaShape {
  static constexpr int kWaves = (MODE == 0 && RB <= 8) ? 16 : 8;
  static constexpr int kThreads = 64 * kWaves;
};

// LDS: the reciprocal table during the main loop, the T partials afterwards.
template <int MODE, int RB>
struct QaLds {
  static constexpr int kRcp = QA_KCHUNK * 8;
  static constexpr int kRed = QaShape<MODE, RB>::kWaves * (RB > 0 ? RB : 1) * 4 * 64 * 4;
  static constexpr int kBytes = kRcp > kRed ? kRcp : kRed;
};

// 16 INT4 codes (nibbles 0..15, two's complement) -> 16 E2M3 fields of
// 6 bits (sign-magnitude, value q/8) packed little-endian into 96 bits.
__device__ __forceinline__ void fp6_fields16(const uint32_t (&c)[16], uint32_t& d0, uint32_t& d1,
                                             uint32_t& d2) {
  uint64_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint64_t f = c[i] < 8u ? c[i] : 0x30u - c[i];
    const int b = 6 * i;
    if (b < 64) {
      lo |= f << b;
      if (b > 58) hi |= f >> (64 - b);
    } else {
      hi |= f << (b - 64);
    }
  }
  d0 = (uint32_t)lo;
  d1 = (uint32_t)(lo >> 32);
  d2 = (uint32_t)hi;
}

// Where a lane writes the activation image: null img = no image.  With
// S > 1 the workgroup at blockIdx.y = s covers K range s and writes its T
// partial sums (tpart != 0) instead of T, for split_t_kernel to add.
struct QaImage {
  uint8_t* img;
  int64_t RT;
  size_t scale, lr, tpart;
  int S;
  const float* g = nullptr;  // NVFP4: the per-tensor scale (device)
};

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

}  // namespace gelu_table

__device__ constexpr gelu_table::Table kGeluBand = gelu_table::make();

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

// MODE 0 = INT4, 1 = FP4, 2 = NVFP4 (row-major codes and scales only, no
// image).  RB = rank / 16 (0 = no down-projection).
// CODES = false skips the quantizer (stand-alone down-projection).
template <int MODE, int RB, bool CODES, bool GELU>
__global__ __launch_bounds__((QaShape<MODE, RB>::kThreads)) void quantize_act_kernel(
    int64_t M, int K, const uint16_t* __restrict__ X, const float* __restrict__ lambda,
    const uint16_t* __restrict__ lora_down, uint8_t* __restrict__ xcodes,
    void* __restrict__ xscales, float* __restrict__ T, QaImage qi) {
  constexpr int QA_WAVES = QaShape<MODE, RB>::kWaves;
  constexpr int QA_THREADS = QaShape<MODE, RB>::kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t smem[QaLds<MODE, RB>::kBytes];
  double* rlam = reinterpret_cast<double*>(smem);
  // the GELU band table (7.5 KB), copied once; the first chunk's barrier
  // orders the copy before any lookup
  __shared__ uint16_t gtab[GELU ? gelu_table::kEntries : 2];
  if constexpr (GELU) {
    for (int i = threadIdx.x; i < gelu_table::kEntries / 2; i += QA_THREADS)
      reinterpret_cast<uint32_t*>(gtab)[i] = reinterpret_cast<const uint32_t*>(kGeluBand.v)[i];
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * QA_ROWS + r16;
  const bool row_ok = row < M;
  const int64_t irt = row >> 5;     // image row tile and lane slot of this row
  const int irr = (int)(row & 31);
  const uint16_t* xrow = X + (row_ok ? row : 0) * (int64_t)K;
  // this workgroup's K range: groups [G s / S, G (s + 1) / S)
  const int S = qi.S > 1 ? qi.S : 1;
  const int kbeg = (int)((int64_t)(K >> 6) * blockIdx.y / S) * 64;
  const int kend = (int)((int64_t)(K >> 6) * (blockIdx.y + 1) / S) * 64;

  v4f tacc[RB > 0 ? RB : 1];
#pragma unroll
  for (int b = 0; b < (RB > 0 ? RB : 1); ++b) tacc[b] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kc = kbeg; kc < kend; kc += QA_KCHUNK) {
    const int kn = min(QA_KCHUNK, kend - kc);
    __syncthreads();  // the previous chunk is done with the table
    for (int c = threadIdx.x; c < kn; c += QA_THREADS) rlam[c] = 1.0 / (double)lambda[kc + c];
    __syncthreads();
    const int ntiles = kn >> 6;
    // Loads of a tile without a branch (rows past M and tiles past the chunk
    // read a valid place; the flag zeroes them when the tile is used), so
    // that the compiler's wait counts stay exact across the loop.
    auto load_x = [&](int t, v4u& xa, v4u& xb, bool& ok) {
      ok = row_ok && t < ntiles;
      const int tc = t < ntiles ? t : ntiles - 1;
      const uint16_t* p = xrow + kc + tc * 64 + j * 16;
      xa = *reinterpret_cast<const v4u*>(p);
      xb = *reinterpret_cast<const v4u*>(p + 8);
    };
    v4u na, nb;
    bool nok;
    load_x(wave, na, nb, nok);
    for (int t = wave; t < ntiles; t += QA_WAVES) {
      const v4u zero4 = v4u{0u, 0u, 0u, 0u};
      const v4u xa = nok ? na : zero4, xb = nok ? nb : zero4;
      uint32_t xw[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
      load_x(t + QA_WAVES, na, nb, nok);  // next tile of this wave
      if constexpr (GELU) {
#pragma unroll
        for (int i = 0; i < 8; ++i) xw[i] = gelu_bf16x2(xw[i], gtab);
      }
      const int kl = t * 64 + j * 16;  // column within the chunk
      const int k0 = kc + kl;          // column within the row

      // X_hat = bf16_RNE(fp32(X / lambda)), kept as bf16 bits and as fp32.
      uint32_t hb[16];
      float xh[16];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float q[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t xbits = (xw[i >> 1] >> (e * 16)) & 0xFFFFu;
          q[e] = (float)((double)bf16_to_f32(xbits) * rlam[kl + i + e]);
        }
        // RNE to bf16 (v_cvt_pk_bf16_f32: the same rounding as the
        // bit-level definition for every finite value)
        const v2f qv = {q[0], q[1]};
        const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(qv, v2bf));
        hb[i] = pk & 0xFFFFu;
        hb[i + 1] = pk >> 16;
        xh[i] = __uint_as_float(pk << 16);
        xh[i + 1] = __uint_as_float(pk & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(xh[i]), fabsf(xh[i + 1])));
      }

      if constexpr (CODES) {
        if constexpr (MODE == 0) {
          // INT4: group of 64 = the four lanes sharing this row.
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const float s = amax / 7.0f;
          uint32_t c[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) c[i] = 0u;
          if (s != 0.f) {
            const double rs = 1.0 / (double)s;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float q = __builtin_rintf((float)((double)xh[i] * rs));  // = rint(fp32(xh / s))
              q = fminf(fmaxf(q, -8.0f), 7.0f);
              c[i] = (uint32_t)(int)q & 0xFu;
            }
          }
          if (xcodes != nullptr && row_ok) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              w0 |= c[i] << (4 * i);
              w1 |= c[8 + i] << (4 * i);
            }
            *reinterpret_cast<v2u*>(xcodes + row * (int64_t)(K >> 1) + (k0 >> 1)) = v2u{w0, w1};
            if (j == 0) reinterpret_cast<float*>(xscales)[row * (int64_t)(K >> 6) + (k0 >> 6)] = s;
          }
          if (qi.img != nullptr) {
            // this lane's 16 fields are fields 0..15 (j even) or 16..31 (j odd)
            // of K half j/2 of group k0/64
            uint8_t* blk = qi.img + ((int64_t)(k0 >> 6) * qi.RT + irt) * I4_BLOCK;
            uint8_t* half = blk + (j >> 1) * 768;
            uint32_t d0, d1, d2;
            fp6_fields16(c, d0, d1, d2);
            if ((j & 1) == 0) {
              *reinterpret_cast<v2u*>(half + 16 * irr) = v2u{d0, d1};
              *reinterpret_cast<uint32_t*>(half + 16 * irr + 8) = d2;
            } else {
              *reinterpret_cast<uint32_t*>(half + 16 * irr + 12) = d0;
              *reinterpret_cast<v2u*>(half + 512 + 8 * irr) = v2u{d1, d2};
            }
            // scale operand, X pattern: slot irr {hi | lo << 16, hi}, slot 32 + irr {lo, 0}
            if (j < 2) {
              const uint32_t hb = f32_to_bf16(s);
              const uint32_t lb = f32_to_bf16(s - bf16_to_f32(hb));
              const v2u so = j == 0 ? v2u{hb | (lb << 16), hb} : v2u{lb, 0u};
              *reinterpret_cast<v2u*>(blk + 1536 + 8 * (32 * j + irr)) = so;
            }
          }
        } else if constexpr (MODE == 1) {
          // FP4: block of 32 = lane pairs (j = 0,1) and (j = 2,3).
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          const int e = e8m0_exponent(amax);
          const float sc = exp2i(-e);
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) w0 |= e2m1_code(xh[i] * sc) << (4 * i);
#pragma unroll
          for (int i = 0; i < 8; ++i) w1 |= e2m1_code(xh[8 + i] * sc) << (4 * i);
          if (xcodes != nullptr && row_ok) {
            *reinterpret_cast<v2u*>(xcodes + row * (int64_t)(K >> 1) + (k0 >> 1)) = v2u{w0, w1};
            if ((j & 1) == 0)
              reinterpret_cast<uint8_t*>(xscales)[row * (int64_t)(K >> 5) + (k0 >> 5)] =
                  (uint8_t)(e + 127);
          }
          if (qi.img != nullptr) {
            // lane slot 32 h + row of the (group, row tile) block, h = j/2
            const int64_t b = (int64_t)(k0 >> 6) * qi.RT + irt;
            const int slot = 32 * (j >> 1) + irr;
            *reinterpret_cast<v2u*>(qi.img + b * F4_CBLOCK + 16 * slot + 8 * (j & 1)) = v2u{w0, w1};
            if ((j & 1) == 0) qi.img[qi.scale + b * F4_SBLOCK + slot] = (uint8_t)(e + 127);
          }
        } else {
          // NVFP4: this lane's 16 elements are one block.  s =
          // E4M3_RNE_sat(fp32(amax / fp32(6 g))), d = fp32(s g), codes of
          // fp32(x_hat / d); the quotient comes from d's fp64 reciprocal,
          // exact for a bf16 numerator as x / lambda above.
          const float g = *qi.g;
          const uint32_t sb = e4m3_encode(amax / __fmul_rn(6.0f, g));
          const float sv = e4m3_value(sb);
          uint32_t w0 = 0, w1 = 0;
          if (sv > 0.f) {
            const double rd = 1.0 / (double)__fmul_rn(sv, g);
#pragma unroll
            for (int i = 0; i < 8; ++i) w0 |= e2m1_code((float)((double)xh[i] * rd)) << (4 * i);
#pragma unroll
            for (int i = 0; i < 8; ++i) w1 |= e2m1_code((float)((double)xh[8 + i] * rd)) << (4 * i);
          }
          if (xcodes != nullptr && row_ok) {
            *reinterpret_cast<v2u*>(xcodes + row * (int64_t)(K >> 1) + (k0 >> 1)) = v2u{w0, w1};
            reinterpret_cast<uint8_t*>(xscales)[row * (int64_t)(K >> 4) + (k0 >> 4)] = (uint8_t)sb;
          }
        }
      }

      if constexpr (RB > 0) {
        // T += X_hat[16 rows, 64 cols] . L1[64 cols, 16*RB]: element i of
        // this lane is column k0 + i; the B operand takes the same columns of
        // lora_down (= L1^T) rows.
        v8bf a0, a1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a0[i] = __builtin_bit_cast(__bf16, (uint16_t)hb[i]);
          a1[i] = __builtin_bit_cast(__bf16, (uint16_t)hb[8 + i]);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint16_t* ld = lora_down + (int64_t)(b * 16 + r16) * K + k0;
          const v8bf b0 = *reinterpret_cast<const v8bf*>(ld);
          const v8bf b1 = *reinterpret_cast<const v8bf*>(ld + 8);
          tacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, tacc[b], 0, 0, 0);
          tacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, tacc[b], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (RB > 0) {
    // Sum the eight waves' partial T tiles through LDS (in a fixed order).
    __syncthreads();  // the table is no longer read
    float(*red)[RB][4][64] = reinterpret_cast<float(*)[RB][4][64]>(smem);
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[wave][b][q][lane] = tacc[b][q];
    __syncthreads();
    // One thread per (row, 8 consecutive ranks): the 8 partial sums of a
    // row and rank chunk are 8 consecutive lanes of one MFMA output register
    // (lane l, element q -> row 4 (l/16) + q, column l%16).
    const int rank = RB * 16;
    for (int idx = threadIdx.x; idx < QA_ROWS * (rank / 8); idx += QA_THREADS) {
      const int mr = idx / (rank / 8);
      const int c8 = idx - mr * (rank / 8);
      const int b = c8 >> 1, q = mr & 3, l0 = 16 * (mr >> 2) + 8 * (c8 & 1);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = red[0][b][q][l0 + i];
#pragma unroll
      for (int w = 1; w < QA_WAVES; ++w)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += red[w][b][q][l0 + i];
      const int64_t m = (int64_t)blockIdx.x * QA_ROWS + mr;
      if (S > 1) {
        // partial sums of K range blockIdx.y, added by split_t_kernel
        float* tp = reinterpret_cast<float*>(qi.img + qi.tpart) +
                    ((int64_t)blockIdx.y * qi.RT * 32 + m) * rank + 8 * c8;
        *reinterpret_cast<v4f*>(tp) = v4f{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<v4f*>(tp + 4) = v4f{v[4], v[5], v[6], v[7]};
        continue;
      }
      if (T != nullptr && m < M) {
        float* tp = T + m * rank + 8 * c8;
        *reinterpret_cast<v4f*>(tp) = v4f{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<v4f*>(tp + 4) = v4f{v[4], v[5], v[6], v[7]};
      }
      if (qi.img != nullptr) {
        // slice b, lane slot 32 (c8 & 1) + row: hi at 16 slot, lo at 1024 + 16 slot
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
          hi[i] = h0 | (h1 << 16);
          lo[i] = f32_to_bf16(v[2 * i] - bf16_to_f32(h0)) |
                  (f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1)) << 16);
        }
        uint8_t* blk = qi.img + qi.lr + ((int64_t)b * qi.RT + (m >> 5)) * LR_XBLOCK;
        const int slot = 32 * (c8 & 1) + (int)(m & 31);
        *reinterpret_cast<v4u*>(blk + 16 * slot) = v4u{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<v4u*>(blk + 1024 + 16 * slot) = v4u{lo[0], lo[1], lo[2], lo[3]};
      }
    }
  }
}

// T of the image (and of the row-major output when T != null) from the S
// partial sums, added in the order of the K ranges; one thread per (row,
// 8 consecutive ranks).
__global__ __launch_bounds__(256) void split_t_kernel(int64_t M, int rank, float* __restrict__ T,
                                                      QaImage qi) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c8n = rank / 8;
  const int64_t rows = qi.RT * 32;
  if (idx >= rows * c8n) return;
  const int64_t m = idx / c8n;
  const int c8 = (int)(idx - m * c8n);
  const float* tp = reinterpret_cast<const float*>(qi.img + qi.tpart) + m * rank + 8 * c8;
  v4f a = *reinterpret_cast<const v4f*>(tp), bq = *reinterpret_cast<const v4f*>(tp + 4);
  for (int sp = 1; sp < qi.S; ++sp) {
    const float* q = tp + (int64_t)sp * rows * rank;
    const v4f x = *reinterpret_cast<const v4f*>(q), y = *reinterpret_cast<const v4f*>(q + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] += x[i];
      bq[i] += y[i];
    }
  }
  const float v[8] = {a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
  if (T != nullptr && m < M) {
    *reinterpret_cast<v4f*>(T + m * rank + 8 * c8) = a;
    *reinterpret_cast<v4f*>(T + m * rank + 8 * c8 + 4) = bq;
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    hi[i] = h0 | (h1 << 16);
    lo[i] = f32_to_bf16(v[2 * i] - bf16_to_f32(h0)) |
            (f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1)) << 16);
  }
  const int b = c8 >> 1;
  uint8_t* blk = qi.img + qi.lr + ((int64_t)b * qi.RT + (m >> 5)) * LR_XBLOCK;
  const int slot = 32 * (c8 & 1) + (int)(m & 31);
  *reinterpret_cast<v4u*>(blk + 16 * slot) = v4u{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<v4u*>(blk + 1024 + 16 * slot) = v4u{lo[0], lo[1], lo[2], lo[3]};
}

template <int MODE, bool CODES, bool GELU>
static hipError_t launch_qa_rank(int rb, dim3 grid, hipStream_t s, int64_t M, int K,
                                 const uint16_t* X, const float* lam, const uint16_t* ld,
                                 uint8_t* xc, void* xs, float* T, QaImage qi) {
#define SVDQ_QA_CASE(R)                                                                   \
  case R:                                                                                 \
    hipLaunchKernelGGL((quantize_act_kernel<MODE, R, CODES, GELU>), grid, dim3(QaShape<MODE, R>::kThreads), 0, \
                       s, M, K, X, lam, ld, xc, xs, T, qi);                               \
    break;
  switch (rb) {
    SVDQ_QA_CASE(0) SVDQ_QA_CASE(1) SVDQ_QA_CASE(2) SVDQ_QA_CASE(3) SVDQ_QA_CASE(4)
    SVDQ_QA_CASE(5) SVDQ_QA_CASE(6) SVDQ_QA_CASE(7) SVDQ_QA_CASE(8) SVDQ_QA_CASE(9)
    SVDQ_QA_CASE(10) SVDQ_QA_CASE(11) SVDQ_QA_CASE(12) SVDQ_QA_CASE(13) SVDQ_QA_CASE(14)
    SVDQ_QA_CASE(15) SVDQ_QA_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef SVDQ_QA_CASE
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize_act(int64_t M, int K, int rank, const uint16_t* X,
                                     const float* lambda, const float* g,
                                     const uint16_t* lora_down, uint8_t* xcodes, uint8_t* xscales,
                                     float* T, hipStream_t s) {
  QaImage qi{nullptr, 0, 0, 0, 0, 1, g};
  const dim3 grid((unsigned)((M + QA_ROWS - 1) / QA_ROWS));
  return launch_qa_rank<2, true, false>(lora_down ? rank / 16 : 0, grid, s, M, K, X, lambda,
                                        lora_down, xcodes, xscales, T, qi);
}

size_t act_image_bytes(int mode, int64_t M, int K, int rank) {
  return act_image(mode, M, K, rank).bytes;
}

hipError_t launch_quantize_act(int mode, int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down,
                               uint8_t* xcodes, void* xscales, float* T, void* ximage,
                               bool gelu, hipStream_t s) {
  QaImage qi{nullptr, 0, 0, 0, 0, 1};
  int64_t rows = M;
  if (ximage != nullptr) {
    const ActImage a = act_image(mode, M, K, rank);
    qi = QaImage{reinterpret_cast<uint8_t*>(ximage), a.RT, a.scale, a.lr, a.tpart, a.S};
    rows = a.RT * 32;  // cover the padding rows too
  }
  const int rb = lora_down ? rank / 16 : 0;
  const dim3 grid((unsigned)((rows + QA_ROWS - 1) / QA_ROWS), (unsigned)qi.S);
  hipError_t e;
  if (mode == 0)
    e = gelu ? launch_qa_rank<0, true, true>(rb, grid, s, M, K, X, lambda, lora_down, xcodes,
                                             xscales, T, qi)
             : launch_qa_rank<0, true, false>(rb, grid, s, M, K, X, lambda, lora_down, xcodes,
                                              xscales, T, qi);
  else
    e = gelu ? launch_qa_rank<1, true, true>(rb, grid, s, M, K, X, lambda, lora_down, xcodes,
                                             xscales, T, qi)
             : launch_qa_rank<1, true, false>(rb, grid, s, M, K, X, lambda, lora_down, xcodes,
                                              xscales, T, qi);
  if (e != hipSuccess || rb == 0 || qi.S <= 1) return e;
  const int64_t n = qi.RT * 32 * (rank / 8);
  hipLaunchKernelGGL(split_t_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, M, rank,
                     T, qi);
  return hipGetLastError();
}

hipError_t launch_lowrank_down(int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down, float* T,
                               bool gelu, hipStream_t s) {
  const dim3 grid((unsigned)((M + QA_ROWS - 1) / QA_ROWS));
  const QaImage qi{nullptr, 0, 0, 0, 0, 1};
  return gelu ? launch_qa_rank<0, false, true>(rank / 16, grid, s, M, K, X, lambda, lora_down,
                                               nullptr, nullptr, T, qi)
              : launch_qa_rank<0, false, false>(rank / 16, grid, s, M, K, X, lambda, lora_down,
                                                nullptr, nullptr, T, qi);
}

}  // namespace svdq
