// W4A4 GEMM of the SVDQuant linear on gfx950, with the low-rank
// up-projection and the bias in its epilogue.
//
// The Nunchaku engine fuses the up-projection of the 16-bit low-rank branch
// into the 4-bit compute kernel (apatero.com page, section "O que e Nunchaku
// e como acelera modelos Qwen"); weights and activations are both 4-bit
// (axbrief.com page, section "The Mechanics of 4-Bit Efficiency and
// SVDQuant").
//
// Tiling: a 256-thread workgroup computes a 128x128 tile of Y; each of its
// four waves a 64x64 quarter made of 2x2 32x32 MFMA tiles.  Packed 4-bit
// tiles of 128 K-elements (64 bytes per row) are staged through LDS with
// double buffering (one barrier per stage), rows padded to 80 bytes so the
// 16-byte fragment reads of 32 consecutive rows hit distinct banks.
//
// INT4 mode: a fragment is 32 codes of one row; the nibbles are widened to
// int8 holding 16*q (even and odd elements in separate dwords) and fed to
// v_mfma_i32_32x32x32_i8, two per 64-element group, so every group sum is an
// exact int32 (scaled by 256).  It is then converted to fp32 and
// accumulated with the product of the two fp32 group scales.
//
// FP4 mode: a fragment is 32 E2M1 codes of one row, the operand of
// v_mfma_scale_f32_32x32x64_f8f6f4 as is; the E8M0 block scales go to the
// instruction's scale operands, so the hardware applies them and the
// accumulation over K stays inside the MFMA.
//
// Epilogue: Y += T L2 with v_mfma_f32_32x32x16_bf16, T split into a bf16
// high and low part (two MFMAs) so the 16-bit branch keeps fp32 accuracy,
// then + bias and the bf16 (or fp32) store.
#include "common.h"
#include "kernels.h"

namespace svdq {

constexpr int GM_BM = 128;
constexpr int GM_BN = 128;
constexpr int GM_BK = 128;  // K elements per LDS stage (64 bytes of codes per row)
constexpr int GM_THREADS = 256;
constexpr int LDS_ROW = 80;  // bytes per staged row: 64 + 16 padding

// 32x32 MFMA accumulator layout: lane l, element i -> row 8*(i/4) + 4*(l/32)
// + i%4, column l%32.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// acc += T[rows] L2[cols] for one 32x32 tile pair, T split hi/lo in bf16.
__device__ __forceinline__ void lowrank_up_tile(v16f (&acc)[2][2], int rank, int64_t M,
                                                int64_t mbase, int nbase, int lane,
                                                const float* __restrict__ T,
                                                const uint16_t* __restrict__ lora_up) {
  for (int rb = 0; rb < rank; rb += 16) {
    v8bf thi[2], tlo[2], bv[2];
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
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
    for (int tc = 0; tc < 2; ++tc) {
      const int n = nbase + tc * 32 + (lane & 31);
      bv[tc] = *reinterpret_cast<const v8bf*>(lora_up + (int64_t)n * rank + rb + (lane >> 5) * 8);
    }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(thi[tr], bv[tc], acc[tr][tc], 0, 0, 0);
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tlo[tr], bv[tc], acc[tr][tc], 0, 0, 0);
      }
  }
}

__device__ __forceinline__ void store_tiles(const v16f (&acc)[2][2], int64_t M, int N,
                                            int64_t mbase, int nbase, int lane,
                                            const uint16_t* __restrict__ bias, bool out_f32,
                                            void* __restrict__ Y, bool accumulate) {
#pragma unroll
  for (int tc = 0; tc < 2; ++tc) {
    const int n = nbase + tc * 32 + (lane & 31);
    const float b = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
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

template <int MODE>
__global__ __launch_bounds__(GM_THREADS) void w4a4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ xcodes,
    const void* __restrict__ xscales, const float* __restrict__ T,
    const uint8_t* __restrict__ wcodes, const void* __restrict__ wscales,
    const uint16_t* __restrict__ lora_up, const uint16_t* __restrict__ bias,
    void* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][GM_BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][GM_BN * LDS_ROW];
  // Scales of one stage.  INT4: [group 0/1][row] as fp32.  FP4: [0][row]
  // holds the stage's four E8M0 bytes of that row.
  __shared__ __attribute__((aligned(16))) uint32_t SX[2][2][GM_BM];
  __shared__ __attribute__((aligned(16))) uint32_t SW[2][2][GM_BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = N / GM_BN;
  const int tile_n = blockIdx.x % ntn;
  const int64_t tile_m = blockIdx.x / ntn;
  const int64_t m0 = tile_m * GM_BM;
  const int n0 = tile_n * GM_BN;
  const int64_t KB = K >> 1;
  const int nstages = K / GM_BK;
  const int ld_row = tid >> 2, ld_chunk = tid & 3;
  const int h = lane >> 5;

  v4u ga[2], gb[2];
  uint32_t gs0 = 0, gs1 = 0;

  auto global_load = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ld_row + 64 * i;
      const int64_t m = m0 + r;
      ga[i] = v4u{0u, 0u, 0u, 0u};
      if (m < M) ga[i] = *reinterpret_cast<const v4u*>(xcodes + m * KB + s * 64 + ld_chunk * 16);
      gb[i] = *reinterpret_cast<const v4u*>(wcodes + (int64_t)(n0 + r) * KB + s * 64 + ld_chunk * 16);
    }
    if (MODE == 0) {
      const int G = K >> 6;
      if (tid < GM_BM) {
        const int64_t m = m0 + tid;
        gs0 = gs1 = 0;
        if (m < M) {
          const v2u v = *reinterpret_cast<const v2u*>(reinterpret_cast<const float*>(xscales) + m * G + 2 * s);
          gs0 = v[0];
          gs1 = v[1];
        }
      } else {
        const int n = n0 + tid - GM_BM;
        const v2u v = *reinterpret_cast<const v2u*>(reinterpret_cast<const float*>(wscales) + (int64_t)n * G + 2 * s);
        gs0 = v[0];
        gs1 = v[1];
      }
    } else {
      const int B = K >> 5;
      if (tid < GM_BM) {
        const int64_t m = m0 + tid;
        gs0 = 0;
        if (m < M) gs0 = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(xscales) + m * B + 4 * s);
      } else {
        const int n = n0 + tid - GM_BM;
        gs0 = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(wscales) + (int64_t)n * B + 4 * s);
      }
    }
  };
  auto lds_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ld_row + 64 * i;
      *reinterpret_cast<v4u*>(&As[buf][r * LDS_ROW + ld_chunk * 16]) = ga[i];
      *reinterpret_cast<v4u*>(&Bs[buf][r * LDS_ROW + ld_chunk * 16]) = gb[i];
    }
    if (tid < GM_BM) {
      SX[buf][0][tid] = gs0;
      SX[buf][1][tid] = gs1;
    } else {
      SW[buf][0][tid - GM_BM] = gs0;
      SW[buf][1][tid - GM_BM] = gs1;
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  global_load(0);
  lds_store(0);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) global_load(s + 1);

    if constexpr (MODE == 0) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        v4i ae[2], ao[2], be[2], bo[2];
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          const int r = wm * 64 + tr * 32 + (lane & 31);
          const v4u w = *reinterpret_cast<const v4u*>(&As[buf][r * LDS_ROW + g * 32 + h * 16]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t e, o;
            int4x8_to_int8x16(w[q], e, o);
            ae[tr][q] = (int)e;
            ao[tr][q] = (int)o;
          }
        }
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
          const int r = wn * 64 + tc * 32 + (lane & 31);
          const v4u w = *reinterpret_cast<const v4u*>(&Bs[buf][r * LDS_ROW + g * 32 + h * 16]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t e, o;
            int4x8_to_int8x16(w[q], e, o);
            be[tc][q] = (int)e;
            bo[tc][q] = (int)o;
          }
        }
        float sw[2];
#pragma unroll
        for (int tc = 0; tc < 2; ++tc)
          sw[tc] = __uint_as_float(SW[buf][g][wn * 64 + tc * 32 + (lane & 31)]);
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          float sx[16];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const v4u v = *reinterpret_cast<const v4u*>(&SX[buf][g][wm * 64 + tr * 32 + 8 * a + 4 * h]);
#pragma unroll
            for (int q = 0; q < 4; ++q) sx[4 * a + q] = __uint_as_float(v[q]);
          }
#pragma unroll
          for (int tc = 0; tc < 2; ++tc) {
            v16i p = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            p = __builtin_amdgcn_mfma_i32_32x32x32_i8(ae[tr], be[tc], p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[tr], bo[tc], p, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i)
              acc[tr][tc][i] = fmaf((float)p[i], sx[i] * sw[tc], acc[tr][tc][i]);
          }
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i af[2], bf[2];
        int sa[2], sb[2];
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          const int r = wm * 64 + tr * 32 + (lane & 31);
          const v4u w = *reinterpret_cast<const v4u*>(&As[buf][r * LDS_ROW + ks * 32 + h * 16]);
          af[tr] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          sa[tr] = (int)(SX[buf][0][r] >> (8 * (2 * ks + h)));
        }
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
          const int r = wn * 64 + tc * 32 + (lane & 31);
          const v4u w = *reinterpret_cast<const v4u*>(&Bs[buf][r * LDS_ROW + ks * 32 + h * 16]);
          bf[tc] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          sb[tc] = (int)(SW[buf][0][r] >> (8 * (2 * ks + h)));
        }
#pragma unroll
        for (int tr = 0; tr < 2; ++tr)
#pragma unroll
          for (int tc = 0; tc < 2; ++tc)
            acc[tr][tc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[tr], bf[tc], acc[tr][tc], 4, 4, 0, sa[tr], 0, sb[tc]);
      }
    }

    if (s + 1 < nstages) lds_store(buf ^ 1);
    __syncthreads();
  }

  if constexpr (MODE == 0) {
    // remove the 16*16 factor of the widened nibbles (exact)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] *= (1.0f / 256.0f);
  }

  const int64_t mbase = m0 + wm * 64;
  const int nbase = n0 + wn * 64;
  if (T != nullptr) lowrank_up_tile(acc, rank, M, mbase, nbase, lane, T, lora_up);
  store_tiles(acc, M, N, mbase, nbase, lane, bias, out_f32 != 0, Y, false);
}

// Stand-alone up-projection for the unfused schedule: Y += T L2.
__global__ __launch_bounds__(GM_THREADS) void lowrank_up_kernel(int64_t M, int N, int rank,
                                                                int out_f32,
                                                                const float* __restrict__ T,
                                                                const uint16_t* __restrict__ lora_up,
                                                                void* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ntn = N / GM_BN;
  const int64_t mbase = (int64_t)(blockIdx.x / ntn) * GM_BM + (wave >> 1) * 64;
  const int nbase = (blockIdx.x % ntn) * GM_BN + (wave & 1) * 64;
  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  lowrank_up_tile(acc, rank, M, mbase, nbase, lane, T, lora_up);
  store_tiles(acc, M, N, mbase, nbase, lane, nullptr, out_f32 != 0, Y, true);
}

hipError_t launch_linear_forward(int mode, int rank, bool out_f32, int64_t M, int N, int K,
                                 const uint8_t* xcodes, const void* xscales, const float* T,
                                 const uint8_t* wcodes, const void* wscales,
                                 const uint16_t* lora_up, const uint16_t* bias, void* Y,
                                 hipStream_t s) {
  const int64_t tiles = ((M + GM_BM - 1) / GM_BM) * (N / GM_BN);
  const dim3 grid((unsigned)tiles);
  if (mode == 0)
    hipLaunchKernelGGL(w4a4_gemm_kernel<0>, grid, dim3(GM_THREADS), 0, s, M, N, K, rank,
                       (int)out_f32, xcodes, xscales, T, wcodes, wscales, lora_up, bias, Y);
  else
    hipLaunchKernelGGL(w4a4_gemm_kernel<1>, grid, dim3(GM_THREADS), 0, s, M, N, K, rank,
                       (int)out_f32, xcodes, xscales, T, wcodes, wscales, lora_up, bias, Y);
  return hipGetLastError();
}

hipError_t launch_lowrank_up(int rank, bool out_f32, int64_t M, int N, const float* T,
                             const uint16_t* lora_up, void* Y, hipStream_t s) {
  const int64_t tiles = ((M + GM_BM - 1) / GM_BM) * (N / GM_BN);
  hipLaunchKernelGGL(lowrank_up_kernel, dim3((unsigned)tiles), dim3(GM_THREADS), 0, s, M, N,
                     rank, (int)out_f32, T, lora_up, Y);
  return hipGetLastError();
}

}  // namespace svdq
