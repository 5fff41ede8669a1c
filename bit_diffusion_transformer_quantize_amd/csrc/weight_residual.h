// The residual of the smoothed weight and its low-rank part, for the weight
// packers (pack_weight.hip, nvfp4.hip).  Layout of the caller: a lane owns 16
// consecutive columns k0.. of weight row n.
#pragma once

#include "common.h"

namespace svdq {

// r[i] = fp32(fp32(W[n][k0+i] * lambda[k0+i]) - acc_i), acc_i = sum over q in
// order of fp32(L1[k0+i][q] * L2[q][n]) added in fp32 (each product is exact),
// with no fused multiply-add anywhere.
__device__ __forceinline__ void weight_residual16(int n, int k0, int K, int rank,
                                                  const uint16_t* __restrict__ W,
                                                  const float* __restrict__ lambda,
                                                  const uint16_t* __restrict__ lora_down,
                                                  const uint16_t* __restrict__ lora_up,
                                                  float (&r)[16]) {
  const v4u wa = *reinterpret_cast<const v4u*>(W + (int64_t)n * K + k0);
  const v4u wb = *reinterpret_cast<const v4u*>(W + (int64_t)n * K + k0 + 8);
  const uint32_t ww[8] = {wa[0], wa[1], wa[2], wa[3], wb[0], wb[1], wb[2], wb[3]};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float w = bf16_to_f32((ww[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu);
    r[i] = __fmul_rn(w, lambda[k0 + i]);  // W_hat
  }
  if (rank > 0) {
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int q = 0; q < rank; ++q) {
      const float u = bf16_to_f32(lora_up[(int64_t)n * rank + q]);  // L2[q][n]
      const uint16_t* ld = lora_down + (int64_t)q * K + k0;           // L1[k][q]
      const v4u da = *reinterpret_cast<const v4u*>(ld);
      const v4u db = *reinterpret_cast<const v4u*>(ld + 8);
      const uint32_t dd[8] = {da[0], da[1], da[2], da[3], db[0], db[1], db[2], db[3]};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float d = bf16_to_f32((dd[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu);
        acc[i] = __fadd_rn(acc[i], __fmul_rn(d, u));  // product exact in fp32
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = __fsub_rn(r[i], acc[i]);
  }
}

}  // namespace svdq
