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
#include "weight_residual.h"

namespace svdq {

// ---------------------------------------------------------------- lambda
// Per-column absolute maxima, one workgroup per 64 columns (so the maxima of
// a column never leave the workgroup and no scratch memory is needed).  Its
// 16 waves stride over the rows: lane l reads 16 bytes (8 columns) of row
// 8 wave + l/8 (+ 128 i), so a wave-wide load covers 8 rows x 64 columns.
// The 8 lanes of a column chunk combine by shuffles, the waves through LDS.
// A maximum is exact in any order.
constexpr int CAL_WAVES = 16;
constexpr int CAL_THREADS = 64 * CAL_WAVES;

// Maxima of |A[r][c0 .. c0+63]| over all rows; the result for column c0 + i
// is returned by thread i (i < 64) of the workgroup, 0 for the others.
__device__ float colmax64(int64_t R, int K, const uint16_t* __restrict__ A, int c0,
                          float (*red)[64]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cl = (lane & 7) * 8;
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.f;
  const uint16_t* base = A + c0 + cl;
#pragma unroll 4
  for (int64_t r = wave * 8 + (lane >> 3); r < R; r += 8 * CAL_WAVES) {
    const v4u v = *reinterpret_cast<const v4u*>(base + r * K);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] = fmaxf(m[2 * e], fabsf(bf16_to_f32(v[e] & 0xFFFFu)));
      m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(bf16_to_f32(v[e] >> 16)));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m[e] = fmaxf(m[e], __shfl_xor(m[e], 8, 64));
    m[e] = fmaxf(m[e], __shfl_xor(m[e], 16, 64));
    m[e] = fmaxf(m[e], __shfl_xor(m[e], 32, 64));
  }
  __syncthreads();  // red may still be read by a previous call
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][cl + e] = m[e];
  }
  __syncthreads();
  float out = 0.f;
  if (threadIdx.x < 64) {
    for (int w = 0; w < CAL_WAVES; ++w) out = fmaxf(out, red[w][threadIdx.x]);
  }
  return out;
}

__device__ __forceinline__ float lambda_of(float ax, float aw) {
  return (ax > 0.f && aw > 0.f) ? (float)__builtin_sqrt((double)ax / (double)aw) : 1.0f;
}

__global__ __launch_bounds__(CAL_THREADS) void calibrate_lambda_kernel(
    int64_t M, int K, int N, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    float* __restrict__ lambda) {
  __shared__ float red[CAL_WAVES][64];
  const int c0 = blockIdx.x * 64;
  const float ax = colmax64(M, K, X, c0, red);
  const float aw = colmax64(N, K, W, c0, red);
  if (threadIdx.x < 64) lambda[c0 + threadIdx.x] = lambda_of(ax, aw);
}

__global__ __launch_bounds__(CAL_THREADS) void column_absmax_kernel(
    int64_t R, int K, const uint16_t* __restrict__ A, float* __restrict__ amax, int accumulate) {
  __shared__ float red[CAL_WAVES][64];
  const int c0 = blockIdx.x * 64;
  const float a = colmax64(R, K, A, c0, red);
  if (threadIdx.x < 64) {
    const int c = c0 + threadIdx.x;
    amax[c] = accumulate ? fmaxf(amax[c], a) : a;
  }
}

__global__ __launch_bounds__(256) void lambda_from_absmax_kernel(int K, const float* __restrict__ xmax,
                                                                 const float* __restrict__ wmax,
                                                                 float* __restrict__ lambda) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < K) lambda[c] = lambda_of(xmax[c], wmax[c]);
}

hipError_t launch_calibrate_lambda(int64_t M, int K, int N, const uint16_t* X,
                                   const uint16_t* W, float* lambda, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_lambda_kernel, dim3(K / 64), dim3(CAL_THREADS), 0, s, M, K, N,
                     X, W, lambda);
  return hipGetLastError();
}

hipError_t launch_column_absmax(int64_t R, int K, const uint16_t* A, float* amax, bool accumulate,
                                hipStream_t s) {
  hipLaunchKernelGGL(column_absmax_kernel, dim3(K / 64), dim3(CAL_THREADS), 0, s, R, K, A, amax,
                     accumulate ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_lambda_from_absmax(int K, const float* xmax, const float* wmax, float* lambda,
                                     hipStream_t s) {
  hipLaunchKernelGGL(lambda_from_absmax_kernel, dim3((K + 255) / 256), dim3(256), 0, s, K, xmax,
                     wmax, lambda);
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
    weight_residual16(n, k0, K, rank, W, lambda, lora_down, lora_up, r);
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
