// Offline side of the SVDQuant W4A4 linear on gfx950: smoothing-factor
// calibration and weight packing.
//
// The weight side follows the decomposition of the Nunchaku Lite page
// (axbrief.com, section "The Mechanics of 4-Bit Efficiency and SVDQuant"):
// the smoothed weight W_hat = W diag(lambda) minus its 16-bit low-rank part
// L1 L2 is the residual R that is stored in 4 bits.  Every step is written
// with explicit round-to-nearest operations (no contraction into FMA; the
// library is also built with -ffp-contract=off) so that the codes and scales
// are bit-identical to the definition.
#include "common.h"
#include "kernels.h"

namespace svdq {

// ---------------------------------------------------------------- lambda
// One workgroup per 64 columns: its four waves stride over the rows of X and
// of W, lane l owning column c0 + l (128 contiguous bytes per row and wave).
constexpr int CAL_THREADS = 256;

__global__ __launch_bounds__(CAL_THREADS) void calibrate_lambda_kernel(
    int64_t M, int K, int N, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    float* __restrict__ lambda) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float ax = 0.f, aw = 0.f;
  for (int64_t m = wave; m < M; m += 4) ax = fmaxf(ax, fabsf(bf16_to_f32(X[m * K + c])));
  for (int64_t n = wave; n < N; n += 4) aw = fmaxf(aw, fabsf(bf16_to_f32(W[n * K + c])));
  __shared__ float sx[4][64], sw[4][64];
  sx[wave][lane] = ax;
  sw[wave][lane] = aw;
  __syncthreads();
  if (wave == 0) {
    ax = fmaxf(fmaxf(sx[0][lane], sx[1][lane]), fmaxf(sx[2][lane], sx[3][lane]));
    aw = fmaxf(fmaxf(sw[0][lane], sw[1][lane]), fmaxf(sw[2][lane], sw[3][lane]));
    float lam = 1.0f;
    if (ax > 0.f && aw > 0.f) lam = (float)__builtin_sqrt((double)ax / (double)aw);
    lambda[c] = lam;
  }
}

hipError_t launch_calibrate_lambda(int64_t M, int K, int N, const uint16_t* X,
                                   const uint16_t* W, float* lambda, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_lambda_kernel, dim3(K / 64), dim3(CAL_THREADS), 0, s, M, K, N,
                     X, W, lambda);
  return hipGetLastError();
}

// ---------------------------------------------------------------- packing
// Same lane layout as the activation kernel: 16 rows per workgroup, lane l
// owns row l%16 and the 16 columns 16*(l/16).. of each 64-column tile, so an
// INT4 group (64) is the four lanes of a row and an FP4 block (32) a lane
// pair.
constexpr int PW_ROWS = 16;
constexpr int PW_THREADS = 256;

template <int MODE>
__global__ __launch_bounds__(PW_THREADS) void pack_weight_kernel(
    int N, int K, int rank, const uint16_t* __restrict__ W, const float* __restrict__ lambda,
    const uint16_t* __restrict__ lora_down, const uint16_t* __restrict__ lora_up,
    uint8_t* __restrict__ wcodes, void* __restrict__ wscales) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int n = blockIdx.x * PW_ROWS + r16;  // N % 128 == 0: always in range
  const int ntiles = K >> 6;
  for (int t = wave; t < ntiles; t += 4) {
    const int k0 = t * 64 + j * 16;
    float r[16];
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
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(r[i]));
    uint32_t w0 = 0, w1 = 0;
    if constexpr (MODE == 0) {
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float s = amax / 7.0f;
      if (s != 0.f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w0 |= ((uint32_t)int4_code(r[i], s) & 0xFu) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) w1 |= ((uint32_t)int4_code(r[8 + i], s) & 0xFu) << (4 * i);
      }
      if (j == 0) reinterpret_cast<float*>(wscales)[(int64_t)n * (K >> 6) + t] = s;
    } else {
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      const int e = e8m0_exponent(amax);
      const float sc = exp2i(-e);
#pragma unroll
      for (int i = 0; i < 8; ++i) w0 |= e2m1_code(r[i] * sc) << (4 * i);
#pragma unroll
      for (int i = 0; i < 8; ++i) w1 |= e2m1_code(r[8 + i] * sc) << (4 * i);
      if ((j & 1) == 0)
        reinterpret_cast<uint8_t*>(wscales)[(int64_t)n * (K >> 5) + 2 * t + (j >> 1)] =
            (uint8_t)(e + 127);
    }
    *reinterpret_cast<v2u*>(wcodes + (int64_t)n * (K >> 1) + (k0 >> 1)) = v2u{w0, w1};
  }
}

hipError_t launch_pack_weight(int mode, int rank, int N, int K, const uint16_t* W,
                              const float* lambda, const uint16_t* lora_down,
                              const uint16_t* lora_up, uint8_t* wcodes, void* wscales,
                              hipStream_t s) {
  const dim3 grid(N / PW_ROWS);
  if (mode == 0)
    hipLaunchKernelGGL(pack_weight_kernel<0>, grid, dim3(PW_THREADS), 0, s, N, K, rank, W,
                       lambda, lora_down, lora_up, wcodes, wscales);
  else
    hipLaunchKernelGGL(pack_weight_kernel<1>, grid, dim3(PW_THREADS), 0, s, N, K, rank, W,
                       lambda, lora_down, lora_up, wcodes, wscales);
  return hipGetLastError();
}

}  // namespace svdq
