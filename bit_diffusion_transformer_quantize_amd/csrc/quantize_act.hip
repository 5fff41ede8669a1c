// Activation side of the SVDQuant W4A4 linear on gfx950: smoothing, 4-bit
// quantization and the fused low-rank down-projection in one pass over X.
//
// The Nunchaku engine fuses the down-projection of the low-rank branch into
// the quantization kernel so that both branches share one read of the
// activations (apatero.com page, section "O que e Nunchaku e como acelera
// modelos Qwen").  Here a workgroup owns 16 rows of X; its four waves take
// 64-column tiles round-robin.  In a tile, lane l holds row l%16 and the 16
// columns 16*(l/16) .. +15, which is also the A-operand layout of two
// v_mfma_f32_16x16x32_bf16, so the smoothed bf16 values feed the MFMA
// straight from registers.  Per-group absmax is a two-step xor-shuffle over
// the four lanes that share a row.  The T partials of the four waves are
// summed through LDS at the end.
#include "common.h"
#include "kernels.h"

namespace svdq {

constexpr int QA_ROWS = 16;
constexpr int QA_WAVES = 4;
constexpr int QA_THREADS = 64 * QA_WAVES;

// MODE 0 = INT4, 1 = FP4.  RB = rank / 16 (0 = no down-projection).
// CODES = false skips the quantizer (stand-alone down-projection).
template <int MODE, int RB, bool CODES>
__global__ __launch_bounds__(QA_THREADS) void quantize_act_kernel(
    int64_t M, int K, const uint16_t* __restrict__ X, const float* __restrict__ lambda,
    const uint16_t* __restrict__ lora_down, uint8_t* __restrict__ xcodes,
    void* __restrict__ xscales, float* __restrict__ T) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * QA_ROWS + r16;
  const bool row_ok = row < M;
  const int ntiles = K >> 6;
  const uint16_t* xrow = X + (row_ok ? row : 0) * (int64_t)K;

  v4f tacc[RB > 0 ? RB : 1];
#pragma unroll
  for (int b = 0; b < (RB > 0 ? RB : 1); ++b) tacc[b] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int t = wave; t < ntiles; t += QA_WAVES) {
    const int k0 = t * 64 + j * 16;
    v4u xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
    if (row_ok) {
      xa = *reinterpret_cast<const v4u*>(xrow + k0);
      xb = *reinterpret_cast<const v4u*>(xrow + k0 + 8);
    }
    const v4f l0 = *reinterpret_cast<const v4f*>(lambda + k0);
    const v4f l1 = *reinterpret_cast<const v4f*>(lambda + k0 + 4);
    const v4f l2 = *reinterpret_cast<const v4f*>(lambda + k0 + 8);
    const v4f l3 = *reinterpret_cast<const v4f*>(lambda + k0 + 12);
    const float lam[16] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3],
                           l2[0], l2[1], l2[2], l2[3], l3[0], l3[1], l3[2], l3[3]};
    const uint32_t xw[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};

    // X_hat = bf16_RNE(fp32(X / lambda)), kept as bf16 bits and as fp32.
    uint32_t hb[16];
    float xh[16];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t xbits = (xw[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      const float q = bf16_to_f32(xbits) / lam[i];
      hb[i] = f32_to_bf16(q);
      xh[i] = bf16_to_f32(hb[i]);
      amax = fmaxf(amax, fabsf(xh[i]));
    }

    if constexpr (CODES) {
      if constexpr (MODE == 0) {
        // INT4: group of 64 = the four lanes sharing this row.
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float s = amax / 7.0f;
        uint32_t w0 = 0, w1 = 0;
        if (s != 0.f) {
#pragma unroll
          for (int i = 0; i < 8; ++i) w0 |= ((uint32_t)int4_code(xh[i], s) & 0xFu) << (4 * i);
#pragma unroll
          for (int i = 0; i < 8; ++i) w1 |= ((uint32_t)int4_code(xh[8 + i], s) & 0xFu) << (4 * i);
        }
        if (row_ok) {
          *reinterpret_cast<v2u*>(xcodes + row * (int64_t)(K >> 1) + (k0 >> 1)) = v2u{w0, w1};
          if (j == 0) reinterpret_cast<float*>(xscales)[row * (int64_t)(K >> 6) + t] = s;
        }
      } else {
        // FP4: block of 32 = lane pairs (j = 0,1) and (j = 2,3).
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        const int e = e8m0_exponent(amax);
        const float sc = exp2i(-e);
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w0 |= e2m1_code(xh[i] * sc) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) w1 |= e2m1_code(xh[8 + i] * sc) << (4 * i);
        if (row_ok) {
          *reinterpret_cast<v2u*>(xcodes + row * (int64_t)(K >> 1) + (k0 >> 1)) = v2u{w0, w1};
          if ((j & 1) == 0)
            reinterpret_cast<uint8_t*>(xscales)[row * (int64_t)(K >> 5) + 2 * t + (j >> 1)] =
                (uint8_t)(e + 127);
        }
      }
    }

    if constexpr (RB > 0) {
      // T += X_hat[16 rows, 64 cols] . L1[64 cols, 16*RB]: element i of this
      // lane is column k0 + i; the B operand takes the same columns of
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

  if constexpr (RB > 0) {
    // Sum the four waves' partial T tiles through LDS.
    __shared__ float red[QA_WAVES][RB][4][64];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[wave][b][q][lane] = tacc[b][q];
    __syncthreads();
    const int rank = RB * 16;
    for (int idx = threadIdx.x; idx < RB * 4 * 64; idx += QA_THREADS) {
      const int b = idx / 256;
      const int q = (idx / 64) & 3;
      const int l = idx & 63;
      const float v = red[0][b][q][l] + red[1][b][q][l] + red[2][b][q][l] + red[3][b][q][l];
      // MFMA 16x16 output: lane l, element q -> row 4*(l/16)+q, column l%16.
      const int64_t m = (int64_t)blockIdx.x * QA_ROWS + 4 * (l >> 4) + q;
      if (m < M) T[m * rank + b * 16 + (l & 15)] = v;
    }
  }
}

template <int MODE, bool CODES>
static hipError_t launch_qa_rank(int rb, dim3 grid, hipStream_t s, int64_t M, int K,
                                 const uint16_t* X, const float* lam, const uint16_t* ld,
                                 uint8_t* xc, void* xs, float* T) {
#define SVDQ_QA_CASE(R)                                                                   \
  case R:                                                                                 \
    hipLaunchKernelGGL((quantize_act_kernel<MODE, R, CODES>), grid, dim3(QA_THREADS), 0, \
                       s, M, K, X, lam, ld, xc, xs, T);                                   \
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

hipError_t launch_quantize_act(int mode, int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down,
                               uint8_t* xcodes, void* xscales, float* T, hipStream_t s) {
  const dim3 grid((unsigned)((M + QA_ROWS - 1) / QA_ROWS));
  const int rb = lora_down ? rank / 16 : 0;
  if (mode == 0)
    return launch_qa_rank<0, true>(rb, grid, s, M, K, X, lambda, lora_down, xcodes, xscales, T);
  return launch_qa_rank<1, true>(rb, grid, s, M, K, X, lambda, lora_down, xcodes, xscales, T);
}

hipError_t launch_lowrank_down(int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down, float* T,
                               hipStream_t s) {
  const dim3 grid((unsigned)((M + QA_ROWS - 1) / QA_ROWS));
  return launch_qa_rank<0, false>(rank / 16, grid, s, M, K, X, lambda, lora_down, nullptr,
                                  nullptr, T);
}

}  // namespace svdq
