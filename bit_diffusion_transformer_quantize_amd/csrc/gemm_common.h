// Pieces shared by the W4A4 GEMM kernels: the 32x32 MFMA accumulator
// layout, the low-rank up-projection epilogue and the output store.
#pragma once

#include "common.h"

namespace svdq {

// 32x32 MFMA accumulator layout (same for the i8, bf16 and f8f6f4 forms):
// lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// acc[tr][tc] += T[rows] L2[cols] for a TR x TC block of 32x32 tiles whose
// top-left output is (mbase, nbase); rows >= M and columns >= N contribute
// nothing (their outputs are never stored).  T (fp32) is split into a bf16
// high and low part, so the two bf16 MFMAs per 16-wide slice of the rank
// keep the branch accurate to about 2^-16 of |T|.
template <int TR, int TC>
__device__ __forceinline__ void lowrank_up_tiles(v16f (&acc)[TR][TC], int rank, int64_t M,
                                                 int N, int64_t mbase, int nbase, int lane,
                                                 const float* __restrict__ T,
                                                 const uint16_t* __restrict__ lora_up) {
  for (int rb = 0; rb < rank; rb += 16) {
    v8bf thi[TR], tlo[TR], bv[TC];
#pragma unroll
    for (int tr = 0; tr < TR; ++tr) {
      const int64_t m = mbase + tr * 32 + (lane & 31);
      v4f t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
      if (m < M) {
        const float* tp = T + m * rank + rb + (lane >> 5) * 8;
        t0 = *reinterpret_cast<const v4f*>(tp);
        t1 = *reinterpret_cast<const v4f*>(tp + 4);
      }
      const float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t h = f32_to_bf16(tv[i]);
        const uint32_t l = f32_to_bf16(tv[i] - bf16_to_f32(h));
        thi[tr][i] = __builtin_bit_cast(__bf16, (uint16_t)h);
        tlo[tr][i] = __builtin_bit_cast(__bf16, (uint16_t)l);
      }
    }
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      const int n = nbase + tc * 32 + (lane & 31);
      if (n < N) {
        bv[tc] = *reinterpret_cast<const v8bf*>(lora_up + (int64_t)n * rank + rb + (lane >> 5) * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bv[tc][i] = __builtin_bit_cast(__bf16, (uint16_t)0);
      }
    }
#pragma unroll
    for (int tr = 0; tr < TR; ++tr)
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(thi[tr], bv[tc], acc[tr][tc], 0, 0, 0);
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tlo[tr], bv[tc], acc[tr][tc], 0, 0, 0);
      }
  }
}

// Y[rows, cols] (=|+=) acc + bias, bf16 (RNE) or fp32; rows >= M and
// columns >= N are skipped.
template <int TR, int TC>
__device__ __forceinline__ void store_tiles(const v16f (&acc)[TR][TC], int64_t M, int N,
                                            int64_t mbase, int nbase, int lane,
                                            const uint16_t* __restrict__ bias, bool out_f32,
                                            void* __restrict__ Y, bool accumulate) {
#pragma unroll
  for (int tc = 0; tc < TC; ++tc) {
    const int n = nbase + tc * 32 + (lane & 31);
    if (n >= N) continue;
    const float b = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int tr = 0; tr < TR; ++tr)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = mbase + tr * 32 + acc_row(i, lane);
        if (m < M) {
          const int64_t o = m * N + n;
          float v = acc[tr][tc][i] + b;
          if (out_f32) {
            float* y = reinterpret_cast<float*>(Y) + o;
            *y = accumulate ? *y + v : v;
          } else {
            uint16_t* y = reinterpret_cast<uint16_t*>(Y) + o;
            if (accumulate) v += bf16_to_f32(*y);
            *y = (uint16_t)f32_to_bf16(v);
          }
        }
      }
  }
}

}  // namespace svdq
