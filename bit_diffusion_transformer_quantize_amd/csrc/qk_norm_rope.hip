// Attention input after the QKV projection on gfx950: per-head RMSNorm of Q
// and K, then the rotary embedding of adjacent feature pairs.
//
// The fused engine of the Nunchaku Lite page (axbrief.com, section "The
// Trade-off Between Fused Kernels and Generality") takes the QKV projection
// through the Q/K normalisation and the rotary embedding.  For one token the
// projection output row (ld features) starts with Q and K, H heads of 128
// features each ([Q | K | V ...]); for every
// head of Q and of K (each with its own scale vector):
//   x_hat[d] = x[d] * (1 / sqrt(sum_d x[d]^2 / 128 + eps)) * scale[d],
//   out[2i] = cos_i x_hat[2i] - sin_i x_hat[2i+1],
//   out[2i+1] = sin_i x_hat[2i] + cos_i x_hat[2i+1],
// in fp32, rounded to bf16; V is left as it is.
//
// An HBM-bound pass: 8 lanes per (token, head), each lane 16 features (two
// 16-byte loads and stores), the sum of squares reduced by shuffles within
// the 8 lanes; the lane's eight pairs take their cos/sin with two 16-byte
// loads each.
#include "common.h"
#include "kernels.h"

namespace svdq {
namespace {

constexpr int QKR_THREADS = 256;
constexpr int QKR_LANES = 8;                          // lanes per (token, head), 16 features each
constexpr int QKR_ROWS = QKR_THREADS / QKR_LANES;     // (token, head) rows per workgroup

__global__ __launch_bounds__(QKR_THREADS) void qk_norm_rope_kernel(
    int64_t rows, int heads, int64_t ld, uint16_t* __restrict__ Y, const uint16_t* __restrict__ q_scale,
    const uint16_t* __restrict__ k_scale, const float* __restrict__ cosv,
    const float* __restrict__ sinv, float eps) {
  const int64_t hr = (int64_t)blockIdx.x * QKR_ROWS + (threadIdx.x / QKR_LANES);
  if (hr >= rows) return;
  const int sub = threadIdx.x % QKR_LANES;
  const int64_t m = hr / (2 * heads);
  const int hh = (int)(hr - m * 2 * heads);            // 0..H-1: Q heads, H..2H-1: K heads
  uint16_t* y = Y + m * ld + (int64_t)hh * 128 + 16 * sub;
  const uint16_t* sc = (hh < heads ? q_scale : k_scale) + 16 * sub;

  v4u raw[2], sraw[2];
  v4f c[2], s[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) raw[h] = reinterpret_cast<const v4u*>(y)[h];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    sraw[h] = reinterpret_cast<const v4u*>(sc)[h];
    c[h] = reinterpret_cast<const v4f*>(cosv + m * 64 + 8 * sub)[h];
    s[h] = reinterpret_cast<const v4f*>(sinv + m * 64 + 8 * sub)[h];
  }
  float x[16];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * h + 2 * e] = bf16_to_f32(raw[h][e] & 0xFFFFu);
      x[8 * h + 2 * e + 1] = bf16_to_f32(raw[h][e] >> 16);
    }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) ss += x[e] * x[e];
  ss += __shfl_xor(ss, 1, QKR_LANES);
  ss += __shfl_xor(ss, 2, QKR_LANES);
  ss += __shfl_xor(ss, 4, QKR_LANES);
  const float r = 1.0f / __builtin_sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v4u out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = x[8 * h + 2 * e] * r * bf16_to_f32(sraw[h][e] & 0xFFFFu);
      const float b = x[8 * h + 2 * e + 1] * r * bf16_to_f32(sraw[h][e] >> 16);
      out[e] = pack_bf16x2(c[h][e] * a - s[h][e] * b, s[h][e] * a + c[h][e] * b);
    }
    reinterpret_cast<v4u*>(y)[h] = out;
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(int64_t M, int heads, int64_t ld, uint16_t* Y, const uint16_t* q_scale,
                               const uint16_t* k_scale, const float* cosv, const float* sinv,
                               float eps, hipStream_t s) {
  const int64_t rows = M * 2 * heads;
  const int64_t blocks = (rows + QKR_ROWS - 1) / QKR_ROWS;
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)blocks), dim3(QKR_THREADS), 0, s, rows,
                     heads, ld, Y, q_scale, k_scale, cosv, sinv, eps);
  return hipGetLastError();
}

}  // namespace svdq
