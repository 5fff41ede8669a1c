// Activation side of the SVDQuant W4A4 linear on gfx950: smoothing, 4-bit
// quantization and the fused low-rank down-projection in one pass over X.
//
// The Nunchaku engine fuses the down-projection of the low-rank branch into
// the quantization kernel so that both branches share one read of the
// activations (apatero.com page, section "O que e Nunchaku e como acelera
// modelos Qwen").  Here a workgroup owns one or two 16-row blocks of X (see
// QaShape); its waves take 64-column tiles round-robin, each prefetching its
// next tile.  In a tile, lane l holds row l%16 of a block and the 16 columns
// 16*(l/16) .. +15, which is also the A-operand layout of two
// v_mfma_f32_16x16x32_bf16, so the smoothed bf16 values feed the MFMA
// straight from registers; lora_down reaches the B operand through a
// per-wave LDS staging buffer.  The per-group absmax is a maximum over the
// lanes that share a row, exchanged by the gfx950 lane swaps.  The waves' T
// partials are summed through LDS at the end.
//
// Exact quotients without a division per element.  Both quotients of the
// contract, fp32(x / lambda) and fp32(x_hat / s), divide a bf16 value
// (8 significant bits) by an fp32 value (24 bits).  Such a quotient is never
// an fp32 rounding midpoint (a 25-bit odd significand times a 24-bit one
// cannot have only 8 significant bits) and, when it is not, it lies at least
// about 2^-48 (relative) away from every midpoint, while fp64(a * fp64(1/b))
// is within 2^-52 of a/b.  So fp32(fp64(a * fp64(1/b))) is exactly the
// correctly rounded fp32(a / b), provided fp64(1/b) is the correctly rounded
// reciprocal (tests/test_exact_quotient.py checks this on the CPU for every
// finite bf16 a against thousands of divisors: subnormals, all-ones
// significands, INT4 scales, NVFP4 s g values).  Each wave computes the fp64
// reciprocals of its tile's 64 lambdas into its own LDS slot (one per lane),
// so the waves need no barrier before the T partials are summed.  The
// reciprocal of s is computed once per lane and group (for INT4 codes only
// to within a relative 2^-50, which is enough there; see the code).
//
// Outputs: the codes, scales and T in the documented row-major layouts
// (each optional) and/or the activation operand image the GEMM reads
// (image.h): the same codes re-encoded in MFMA lane order (INT4 as 6-bit
// E2M3 fields with the bf16-split scale operands, FP4 as stored with one
// scale byte per lane) and T split into bf16 high and low parts.  With an
// image the grid also covers the padding rows up to a multiple of 256, which
// come out as zeros.
#include "common.h"
#include "gelu_table.h"
#include "image.h"
#include "kernels.h"
#include "nvfp4_codec.h"

namespace svdq {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int QA_RCP = 72;  // fp64 slots of a wave's reciprocals of lambda (64 + padding)

// Rows and waves of a workgroup.  Ranks up to 32: one 16-row block, with
// 16 waves for INT4 (four per SIMD, to keep more of X in flight) and 8 for
// FP4 (measured faster).  Ranks 48..128 (not NVFP4): two 16-row blocks on
// 8 waves, so that each lora_down slice a wave stages serves both blocks'
// MFMAs: the whole K range of L1 streams through every workgroup, and at
// rank 128 that stream, not X, bounds the pass.  Larger ranks: one block on
// 8 waves (the T partials of two blocks would not fit in LDS).
template <int MODE, int RB>
struct QaShape {
  static constexpr int kBlocks = (MODE != 2 && RB > 2 && RB <= 8) ? 2 : 1;
  static constexpr int kWaves = kBlocks == 2 ? 8 : ((MODE == 0 && RB <= 8) ? 16 : 8);
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 16 * kBlocks;
};

// The fp64 reciprocals of a tile's 64 lambdas sit in LDS with 16 bytes of
// padding after every 16 entries: the four lanes of a row read entries 16
// apart, which then fall into different banks.
__device__ __forceinline__ int rl_idx(int c) { return c + ((c >> 4) << 1); }

// max(v, v of lane l ^ 16) and max(v, v of lane l ^ 32): v_permlane16_swap
// exchanges the odd 16-lane rows of one operand with the even rows of the
// other, v_permlane32_swap the upper half of one with the lower half of the
// other, so with v in both operands each lane ends up with its own value and
// its partner's, one in each result.
__device__ __forceinline__ uint32_t max_xor16(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return p[0] > p[1] ? p[0] : p[1];
}
__device__ __forceinline__ uint32_t max_xor32(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return p[0] > p[1] ? p[0] : p[1];
}

// LDS: during the main loop, per wave, the reciprocals of its tile's lambdas
// (two slots: this tile's and the next one's) and, with a down-projection, a 2 KB staging buffer (one 16-rank slice of a
// lora_down tile); the T partials afterwards.
template <int MODE, int RB>
struct QaLds {
  static constexpr int kRcp = QaShape<MODE, RB>::kWaves * 2 * QA_RCP * 8;
  static constexpr int kStage = RB > 0 ? QaShape<MODE, RB>::kWaves * 2048 : 0;
  static constexpr int kRed =
      QaShape<MODE, RB>::kWaves * QaShape<MODE, RB>::kBlocks * (RB > 0 ? RB : 1) * 4 * 64 * 4;
  static constexpr int kBytes = kRcp + kStage > kRed ? kRcp + kStage : kRed;
};

// 16 INT4 codes as 16 E2M3 fields of 6 bits (sign-magnitude, value q/8)
// packed little-endian into 96 bits (three dwords), the layout of half a
// K half of the image, from 16 clamped quotients cq (in [-8, 7]) by the gfx950
// conversion to FP6 (E2M3): it divides by 2^3 (the exponent of the scale
// operand 8), rounds to nearest even on the E2M3 grid, whose step is 1/8 on
// [0, 2), so field i is the E2M3 encoding of rint_even(cq[i]) / 8.  Its two
// sources are interleaved (field 2i from the first, 2i + 1 from the second);
// the upper halves of both are left undefined, only fields 0..15 (the low
// 96 bits) are kept.  A quotient that rounds to zero from below gives the
// negative-zero field 0x20, which the matrix instruction reads as 0.
__device__ __forceinline__ void fp6_fields16_hw(const float (&cq)[16], uint32_t& d0, uint32_t& d1,
                                                uint32_t& d2) {
  v16f ev, od;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ev[i] = cq[2 * i];
    od[i] = cq[2 * i + 1];
  }
  const v6i f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
  d0 = (uint32_t)f[0];
  d1 = (uint32_t)f[1];
  d2 = (uint32_t)f[2];
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
  constexpr int NB = QaShape<MODE, RB>::kBlocks;     // 16-row blocks of the workgroup
  constexpr int QA_WROWS = QaShape<MODE, RB>::kRows;
  // lora_down slices loaded at the top of a tile (the rest when used)
  constexpr int QA_EARLY = QA_WAVES == 16 ? (RB <= 2 ? RB : 0) : (RB < 4 ? RB : 4);
  __shared__ __attribute__((aligned(16))) uint8_t smem[QaLds<MODE, RB>::kBytes];
  // the wide GELU band table (19 KB), copied once before any lookup
  __shared__ uint16_t gtab[GELU ? gelu_table::kWEntries : 2];
  if constexpr (GELU) {
    for (int i = threadIdx.x; i < gelu_table::kWEntries / 2; i += QA_THREADS)
      reinterpret_cast<uint32_t*>(gtab)[i] = reinterpret_cast<const uint32_t*>(kGeluWide.v)[i];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  double* rlam = reinterpret_cast<double*>(smem) + wave * 2 * QA_RCP;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  // this lane's row in block 0 (block sb adds 16 sb)
  const int64_t row0 = (int64_t)blockIdx.x * QA_WROWS + r16;
  const bool block_full = (int64_t)blockIdx.x * QA_WROWS + QA_WROWS <= M;
  // this workgroup's K range: groups [G s / S, G (s + 1) / S)
  const int S = qi.S > 1 ? qi.S : 1;
  const int kbeg = (int)((int64_t)(K >> 6) * blockIdx.y / S) * 64;
  const int kend = (int)((int64_t)(K >> 6) * (blockIdx.y + 1) / S) * 64;

  v4f tacc[NB][RB > 0 ? RB : 1];
#pragma unroll
  for (int sb = 0; sb < NB; ++sb)
#pragma unroll
    for (int b = 0; b < (RB > 0 ? RB : 1); ++b) tacc[sb][b] = v4f{0.f, 0.f, 0.f, 0.f};

  // The waves run independently until the T partials are summed: each takes
  // its tiles of this workgroup's K range round-robin, prefetching the next
  // one's X and lambdas, and makes its tile's reciprocals of lambda itself
  // (one per lane) in its own LDS slot.
  const int ntiles = (kend - kbeg) >> 6;
  {
    // Loads of a tile without a branch (rows past M and tiles past the range
    // read a valid place; the flag zeroes them when the tile is used), so
    // that the compiler's wait counts stay exact across the loop.
    auto load_x = [&](int sb, int t, v4u& xa, v4u& xb, bool& ok) {
      const int64_t rw = row0 + 16 * sb;
      ok = rw < M && t < ntiles;
      const int tc = t < ntiles ? t : ntiles - 1;
      const uint16_t* p = X + (rw < M ? rw : 0) * (int64_t)K + kbeg + tc * 64 + j * 16;
      xa = *reinterpret_cast<const v4u*>(p);
      xb = *reinterpret_cast<const v4u*>(p + 8);
    };
    auto load_lam = [&](int t) { return lambda[kbeg + (t < ntiles ? t : ntiles - 1) * 64 + lane]; };
    // lambda first: waiting for it does not wait for the X loads behind it
    float nlam = load_lam(wave);
    v4u na[NB], nb[NB];
    bool nok[NB];
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) load_x(sb, wave, na[sb], nb[sb], nok[sb]);
    // the first tile's reciprocals of lambda (column t*64 + lane of the range)
    rlam[rl_idx(lane)] = 1.0 / (double)nlam;
    // The tiles of a wave: round-robin over the waves, except that with 16
    // waves (four per SIMD) each of waves 12..15 hands its last tile (when
    // it has two or more) to wave w - 12, which takes it after its own.  A
    // SIMD issues its oldest ready wave first, so otherwise the youngest
    // four waves finish about a tile and a half behind the oldest four and
    // the workgroup waits for them at the T reduction.  Static, so the T
    // sums keep one order from run to run.
    auto next_tile = [&](int t) -> int {
      if constexpr (QA_WAVES == 16) {
        if (wave >= 12) return t + 32 < ntiles ? t + 16 : ntiles;
        if (wave < 4) {
          const int d0 = wave + 12;  // the donor's first tile
          if ((t & 15) == d0) return ntiles;  // the donated tile comes last
          if (t + 16 < ntiles) return t + 16;
          if (d0 + 16 >= ntiles) return ntiles;  // the donor keeps its only tile
          return d0 + 16 * ((ntiles - 1 - d0) / 16);
        }
      }
      return t + QA_WAVES;
    };
    int slot = 0;
    for (int t = wave; t < ntiles; t = next_tile(t)) {
      const double* rcur = rlam + slot * QA_RCP;
      __builtin_amdgcn_wave_barrier();
      const int tn = next_tile(t);
      nlam = load_lam(tn);  // the next tile's, made into reciprocals at the end
      uint32_t xwb[NB][8];
#pragma unroll
      for (int sb = 0; sb < NB; ++sb) {
        v4u xa = na[sb], xb = nb[sb];
        if (!block_full) {  // rows past M read as zeros (uniform: most blocks skip it)
          const v4u zero4 = v4u{0u, 0u, 0u, 0u};
          xa = nok[sb] ? na[sb] : zero4;
          xb = nok[sb] ? nb[sb] : zero4;
        }
        xwb[sb][0] = xa[0]; xwb[sb][1] = xa[1]; xwb[sb][2] = xa[2]; xwb[sb][3] = xa[3];
        xwb[sb][4] = xb[0]; xwb[sb][5] = xb[1]; xwb[sb][6] = xb[2]; xwb[sb][7] = xb[3];
      }
      // This tile's lora_down columns, read as whole 128-byte row segments:
      // load h of slice b gives lane L row b*16 + 8h + L/8 and its 16-byte
      // chunk L%8, so each load covers 8 cache lines in full.  (In the MFMA
      // operand order a load would touch 16 lines, half of each, and such
      // loads measured several times slower.)
      // The first QA_EARLY slices are requested here, ahead of the tile's
      // work, the others (large ranks, for want of registers) when used.
      const uint16_t* l1t = lora_down + (int64_t)(lane >> 3) * K + kbeg + t * 64 + (lane & 7) * 8;
      auto load_l1 = [&](int b, int h) {
        return *reinterpret_cast<const v4u*>(l1t + (int64_t)(b * 16 + 8 * h) * K);
      };
      v4u lg[QA_EARLY > 0 ? QA_EARLY : 1][2];
#pragma unroll
      for (int b = 0; b < QA_EARLY; ++b) {
        lg[b][0] = load_l1(b, 0);
        lg[b][1] = load_l1(b, 1);
      }
#pragma unroll
      for (int sb = 0; sb < NB; ++sb) load_x(sb, tn, na[sb], nb[sb], nok[sb]);  // next tile
      const int kl = j * 16;                // column within the tile
      const int k0 = kbeg + t * 64 + kl;  // column within the row

      // X_hat as packed bf16 pairs, per block (the T MFMA's A operands)
      uint32_t hpk[NB][8];
#pragma unroll
      for (int sb = 0; sb < NB; ++sb) {
        uint32_t* xw = xwb[sb];
        const int64_t row = row0 + 16 * sb;
        const bool row_ok = row < M;
        const int64_t irt = row >> 5;  // image row tile and lane slot of this row
        const int irr = (int)(row & 31);
        if constexpr (GELU) {
          // GELU of the 16 inputs from the wide band table, two at a time with
          // packed 16-bit index arithmetic: the offset into the band, clamped
          // to the sentinel for inputs outside it, plus the sign's half.  The
          // rare out-of-band inputs are redone by the rules, on a branch that
          // the whole wave skips when none of its inputs needs it.
          using namespace gelu_table;
          const us2 lo_off = us2{(unsigned short)(kWLoExp * 128), (unsigned short)(kWLoExp * 128)};
          const us2 sent = us2{(unsigned short)(kWBand * 128), (unsigned short)(kWBand * 128)};
          const us2 half_sz = us2{(unsigned short)kWHalf, (unsigned short)kWHalf};
          uint32_t xin[8];
          us2 worst = us2{0, 0};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            xin[i] = xw[i];
            const us2 off = __builtin_elementwise_min(
                __builtin_bit_cast(us2, xw[i] & 0x7FFF7FFFu) - lo_off, sent);
            worst = __builtin_elementwise_max(worst, off);
            const us2 idx = off + __builtin_bit_cast(us2, (xw[i] >> 15) & 0x00010001u) * half_sz;
            xw[i] = (uint32_t)gtab[idx[0]] | ((uint32_t)gtab[idx[1]] << 16);
          }
          if (__any((worst[0] == sent[0]) | (worst[1] == sent[1]))) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const uint32_t b = (xin[i] >> (16 * h)) & 0xFFFFu;
                const uint32_t e = (b >> 7) & 0xFFu;
                if (e < (uint32_t)kWLoExp || e > (uint32_t)kWHiExp)
                  xw[i] = (xw[i] & (0xFFFF0000u >> (16 * h))) | (gelu_rule(b) << (16 * h));
              }
          }
        }
        // X_hat = bf16_RNE(fp32(X / lambda)), kept as bf16 bits and as fp32.
        float xh[16];
        // largest |x_hat| of the lane as bf16 bits: for finite values the
        // order of the magnitudes is that of their bit patterns with the sign
        // cleared, so a packed 16-bit integer maximum serves
        us2 am2 = us2{0, 0};
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float q[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t xbits = (xw[i >> 1] >> (e * 16)) & 0xFFFFu;
            q[e] = (float)((double)bf16_to_f32(xbits) * rcur[rl_idx(kl + i + e)]);
          }
          // RNE to bf16 (v_cvt_pk_bf16_f32: the same rounding as the
          // bit-level definition for every finite value)
          const v2f qv = {q[0], q[1]};
          const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(qv, v2bf));
          hpk[sb][i >> 1] = pk;
          xh[i] = __uint_as_float(pk << 16);
          xh[i + 1] = __uint_as_float(pk & 0xFFFF0000u);
          am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(us2, pk & 0x7FFF7FFFu));
        }
        uint32_t amb = am2[0] > am2[1] ? am2[0] : am2[1];

        if constexpr (CODES) {
          if constexpr (MODE == 0) {
            // INT4: group of 64 = the four lanes sharing this row.
            amb = max_xor32(max_xor16(amb));
            const float amax = __uint_as_float(amb << 16);
            // s = fp32(amax / 7), exactly: amax is a bf16 value, so the fp64
            // product with the correctly rounded fp64 1/7 rounds to it (the
            // exact-quotient note above)
            const float s = (float)((double)amax * (1.0 / 7.0));
            // cq = fp32(xh / s); the code is rint_even(clamp(cq, -8, 7)).  The
            // clamp never acts: |cq| <= amax / s, and s is within a relative
            // 2^-24 of amax / 7 when normal, and within 2^-150 / (2^-133 / 7)
            // < 2^-14 when subnormal (a nonzero bf16 amax is at least 2^-133),
            // so |cq| < 7.0004 and its rounding lies in [-7, 7] either way.
            // 1/s need not be correctly rounded here: a reciprocal within a
            // relative 2^-50 keeps fp32(xh * (1/s)) = fp32(xh / s) wherever the
            // quotient is a normal fp32 value (the margin is about 2^-48), and a
            // quotient in the subnormal range gives code 0 either way.  So the
            // hardware reciprocal with two Newton steps serves (each step
            // squares its relative error).  An all-zero group (s = 0) takes
            // 1/s = 0: codes 0.
            const double sd = (double)s;
            double rs = __builtin_amdgcn_rcp(sd);
            rs = __builtin_fma(rs, __builtin_fma(-sd, rs, 1.0), rs);
            rs = __builtin_fma(rs, __builtin_fma(-sd, rs, 1.0), rs);
            rs = s != 0.f ? rs : 0.0;
            float cq[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) cq[i] = (float)((double)xh[i] * rs);
            if (xcodes != nullptr && row_ok) {
              uint32_t w0 = 0, w1 = 0;
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                w0 |= ((uint32_t)(int)__builtin_rintf(cq[i]) & 0xFu) << (4 * i);
                w1 |= ((uint32_t)(int)__builtin_rintf(cq[8 + i]) & 0xFu) << (4 * i);
              }
              *reinterpret_cast<v2u*>(xcodes + row * (int64_t)(K >> 1) + (k0 >> 1)) = v2u{w0, w1};
              if (j == 0) reinterpret_cast<float*>(xscales)[row * (int64_t)(K >> 6) + (k0 >> 6)] = s;
            }
            if (qi.img != nullptr) {
              // this lane's 16 fields are fields 0..15 (j even) or 16..31 (j odd)
              // of K half j/2 of group k0/64: an 8-byte and a 4-byte store,
              // chosen without a branch
              uint8_t* blk = qi.img + ((int64_t)(k0 >> 6) * qi.RT + irt) * I4_BLOCK;
              uint8_t* half = blk + (j >> 1) * 768;
              uint32_t d0, d1, d2;
              fp6_fields16_hw(cq, d0, d1, d2);
              const bool ev = (j & 1) == 0;
              *reinterpret_cast<v2u*>(half + (ev ? 16 * irr : 512 + 8 * irr)) = ev ? v2u{d0, d1} : v2u{d1, d2};
              *reinterpret_cast<uint32_t*>(half + 16 * irr + (ev ? 8 : 12)) = ev ? d2 : d0;
              // scale operand, X pattern: slot irr {hi | lo << 16, hi}, slot
              // 32 + irr {lo, 0}; lanes j = 2, 3 store the same bytes as j = 0, 1
              const uint32_t hb = f32_to_bf16(s);
              const uint32_t lb = f32_to_bf16(s - bf16_to_f32(hb));
              const v2u so = ev ? v2u{hb | (lb << 16), hb} : v2u{lb, 0u};
              *reinterpret_cast<v2u*>(blk + 1536 + 8 * (32 * (j & 1) + irr)) = so;
            }
          } else if constexpr (MODE == 1) {
            // FP4: block of 32 = lane pairs (j = 0,1) and (j = 2,3).
            amb = max_xor16(amb);
            const float amax = __uint_as_float(amb << 16);
            const int e = e8m0_exponent(amax);
            uint32_t w0 = 0, w1 = 0;
            if (e >= -100) {
              // the gfx950 conversion: E2M1 nearest-even of x * 2^-e (the
              // exponent of the scale operand), saturating at 6, sign kept
              const float sc = exp2i(e);
              w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[0], xh[1], sc, 0);
              w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[2], xh[3], sc, 1);
              w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[4], xh[5], sc, 2);
              w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[6], xh[7], sc, 3);
              w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[8], xh[9], sc, 0);
              w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[10], xh[11], sc, 1);
              w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[12], xh[13], sc, 2);
              w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[14], xh[15], sc, 3);
            } else {
              // blocks whose maximum is below 2^-98: the scaled values can come
              // from fp32 subnormals, whose handling by the conversion is not
              // relied on
              const float sc = exp2i(-e);
#pragma unroll
              for (int i = 0; i < 8; ++i) w0 |= e2m1_code(xh[i] * sc) << (4 * i);
#pragma unroll
              for (int i = 0; i < 8; ++i) w1 |= e2m1_code(xh[8 + i] * sc) << (4 * i);
            }
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
              // both lanes of the pair store the block's scale byte (the same)
              qi.img[qi.scale + b * F4_SBLOCK + slot] = (uint8_t)(e + 127);
            }
          } else {
            // NVFP4: this lane's 16 elements are one block.  s =
            // E4M3_RNE_sat(fp32(amax / fp32(6 g))), d = fp32(s g), codes of
            // fp32(x_hat / d); the quotient comes from d's fp64 reciprocal,
            // exact for a bf16 numerator as x / lambda above.
            const float g = *qi.g;
            const float amax = __uint_as_float(amb << 16);
            const uint32_t sbits = e4m3_encode(amax / __fmul_rn(6.0f, g));
            const float sv = e4m3_value(sbits);
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
              reinterpret_cast<uint8_t*>(xscales)[row * (int64_t)(K >> 4) + (k0 >> 4)] = (uint8_t)sbits;
            }
          }
        }
      }

      // the next tile's reciprocals of lambda, into the other slot (its
      // lambda was requested at the top of this tile)
      slot ^= 1;
      rlam[slot * QA_RCP + rl_idx(lane)] = 1.0 / (double)nlam;

      if constexpr (RB > 0) {
        // T += X_hat[16 rows, 64 cols] . L1[64 cols, 16*RB]: element i of
        // this lane is column k0 + i; the B operand takes the same columns of
        // lora_down (= L1^T) rows.
        v8bf a0[NB], a1[NB];
#pragma unroll
        for (int sb = 0; sb < NB; ++sb) {
          a0[sb] = __builtin_bit_cast(v8bf, v4u{hpk[sb][0], hpk[sb][1], hpk[sb][2], hpk[sb][3]});
          a1[sb] = __builtin_bit_cast(v8bf, v4u{hpk[sb][4], hpk[sb][5], hpk[sb][6], hpk[sb][7]});
        }
        // Each slice goes through this wave's staging buffer, 16 rows of 128
        // bytes whose 16-byte chunk c of row n sits at position c ^ (n % 8),
        // so that both the row-segment writes and the operand reads (lane l:
        // row l%16, chunks 2(l/16) and 2(l/16) + 1, the columns of a0 and a1)
        // meet every bank once per eight lanes.  The wave's LDS operations run
        // in order, so a slice's writes follow the previous slice's reads
        // without a wait.
        uint8_t* stg = smem + QaLds<MODE, RB>::kRcp + wave * 2048;
        const int wr = lane >> 3, wc = lane & 7;
        const int rd0 = r16 * 128 + (((2 * j) ^ (r16 & 7)) << 4);
        const int rd1 = r16 * 128 + (((2 * j + 1) ^ (r16 & 7)) << 4);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const v4u g0 = b < QA_EARLY ? lg[b < QA_EARLY ? b : 0][0] : load_l1(b, 0);
          const v4u g1 = b < QA_EARLY ? lg[b < QA_EARLY ? b : 0][1] : load_l1(b, 1);
          *reinterpret_cast<v4u*>(stg + wr * 128 + ((wc ^ wr) << 4)) = g0;
          *reinterpret_cast<v4u*>(stg + (8 + wr) * 128 + ((wc ^ wr) << 4)) = g1;
          __builtin_amdgcn_wave_barrier();
          const v8bf b0 = *reinterpret_cast<const v8bf*>(stg + rd0);
          const v8bf b1 = *reinterpret_cast<const v8bf*>(stg + rd1);
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int sb = 0; sb < NB; ++sb) {
            tacc[sb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[sb], b0, tacc[sb][b], 0, 0, 0);
            tacc[sb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[sb], b1, tacc[sb][b], 0, 0, 0);
          }
        }
      }
    }
  }

  if constexpr (RB > 0) {
    // Sum the waves' partial T tiles through LDS, wave 0 first.
    __syncthreads();  // every wave is done with its LDS slots
    float(*red)[NB][RB][4][64] = reinterpret_cast<float(*)[NB][RB][4][64]>(smem);
#pragma unroll
    for (int sb = 0; sb < NB; ++sb)
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][sb][b][q][lane] = tacc[sb][b][q];
    __syncthreads();
    // Four consecutive entries of the wave-0 tile per thread take the sum
    // over the waves in place (each entry is read and written by its own
    // thread alone), all loads in flight at once.
    for (int f = 4 * threadIdx.x; f < NB * RB * 256; f += 4 * QA_THREADS) {
      v4f part[QA_WAVES];
#pragma unroll
      for (int w = 0; w < QA_WAVES; ++w)
        part[w] = *reinterpret_cast<const v4f*>(&red[w][0][0][0][0] + f);
      v4f acc = part[0];
#pragma unroll
      for (int w = 1; w < QA_WAVES; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += part[w][i];
      *reinterpret_cast<v4f*>(&red[0][0][0][0][0] + f) = acc;
    }
    __syncthreads();
    // One thread per (row, 8 consecutive ranks): the 8 sums of a row and
    // rank chunk are 8 consecutive lanes of one MFMA output register (lane
    // l, element q -> row 4 (l/16) + q, column l%16).
    const int rank = RB * 16;
    for (int idx = threadIdx.x; idx < QA_WROWS * (rank / 8); idx += QA_THREADS) {
      const int mr = idx / (rank / 8);  // row of the workgroup
      const int c8 = idx - mr * (rank / 8);
      const int sb = mr >> 4, m16 = mr & 15;
      const int b = c8 >> 1, q = m16 & 3, l0 = 16 * (m16 >> 2) + 8 * (c8 & 1);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = red[0][sb][b][q][l0 + i];
      const int64_t m = (int64_t)blockIdx.x * QA_WROWS + mr;
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

// rows: the rows the grid covers (M, or the image's padded rows); gy: the K
// ranges.
template <int MODE, bool CODES, bool GELU>
static hipError_t launch_qa_rank(int rb, int64_t rows, unsigned gy, hipStream_t s, int64_t M,
                                 int K, const uint16_t* X, const float* lam, const uint16_t* ld,
                                 uint8_t* xc, void* xs, float* T, QaImage qi) {
#define SVDQ_QA_CASE(R)                                                                      \
  case R:                                                                                    \
    hipLaunchKernelGGL((quantize_act_kernel<MODE, R, CODES, GELU>),                          \
                       dim3((unsigned)((rows + QaShape<MODE, R>::kRows - 1) /                \
                                       QaShape<MODE, R>::kRows), gy),                        \
                       dim3(QaShape<MODE, R>::kThreads), 0, s, M, K, X, lam, ld, xc, xs, T, qi); \
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
  return launch_qa_rank<2, true, false>(lora_down ? rank / 16 : 0, M, 1, s, M, K, X, lambda,
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
  const unsigned gy = (unsigned)qi.S;
  hipError_t e;
  if (mode == 0)
    e = gelu ? launch_qa_rank<0, true, true>(rb, rows, gy, s, M, K, X, lambda, lora_down, xcodes,
                                             xscales, T, qi)
             : launch_qa_rank<0, true, false>(rb, rows, gy, s, M, K, X, lambda, lora_down, xcodes,
                                              xscales, T, qi);
  else
    e = gelu ? launch_qa_rank<1, true, true>(rb, rows, gy, s, M, K, X, lambda, lora_down, xcodes,
                                             xscales, T, qi)
             : launch_qa_rank<1, true, false>(rb, rows, gy, s, M, K, X, lambda, lora_down, xcodes,
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
  const QaImage qi{nullptr, 0, 0, 0, 0, 1};
  return gelu ? launch_qa_rank<0, false, true>(rank / 16, M, 1, s, M, K, X, lambda, lora_down,
                                               nullptr, nullptr, T, qi)
              : launch_qa_rank<0, false, false>(rank / 16, M, 1, s, M, K, X, lambda, lora_down,
                                                nullptr, nullptr, T, qi);
}

}  // namespace svdq
