// Builders of the prepared weight (image.h): the packed weight codes and
// scales re-laid in MFMA lane order, the low-rank factor L2 and the bias.
// This is offline work, done once per layer (like the one-time packing of
// the 4-bit weights into the kernel layout that the apatero.com page
// describes, section "O que e Nunchaku e como acelera modelos Qwen").
#include "common.h"
#include "image.h"
#include "kernels.h"

namespace svdq {

// 32 two's-complement int4 codes (16 bytes, element 2j in the low nibble of
// byte j) -> 32 E2M3 sign-magnitude fields of 6 bits (value q/8) packed
// little-endian into six dwords.  For a nibble x the field is x when x < 8
// and 0x20 | (16 - x) = 0x30 - x otherwise.
__device__ __forceinline__ void int4x32_to_fp6x32(const v4u& w, uint32_t (&o)[6]) {
  uint64_t bits[3] = {0, 0, 0};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t x = (w[j >> 3] >> (4 * (j & 7))) & 15u;
    const uint64_t f = x < 8u ? x : 0x30u - x;
    const int b = 6 * j;
    bits[b >> 6] |= f << (b & 63);
    if ((b & 63) > 58) bits[(b >> 6) + 1] |= f >> (64 - (b & 63));
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    o[2 * i] = (uint32_t)bits[i];
    o[2 * i + 1] = (uint32_t)(bits[i] >> 32);
  }
}

// INT4 code blocks of the weight: one wave per (group, 32-row tile).  Rows
// R .. RP-1 are zero.  Scale operand, W pattern: lanes 0..31
// {hi | hi << 16, lo}, lanes 32..63 {lo, 0}, so that with the activation
// pattern {hi | lo << 16, hi} / {lo, 0} the K slots 0..3 of the outer-product
// MFMA hold hi*hi, lo*hi, hi*lo, 0 and slot 4 lo*lo.
__global__ __launch_bounds__(256) void int4_code_image_kernel(int64_t R, int64_t RT, int K,
                                                              const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ scales,
                                                              uint8_t* __restrict__ image) {
  const int G = K >> 6;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= (int64_t)G * RT) return;
  const int g = (int)(blk / RT);
  const int64_t r = (blk - (int64_t)g * RT) * 32 + (threadIdx.x & 31);
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  uint8_t* out = image + blk * I4_BLOCK;
  v4u w = {0u, 0u, 0u, 0u};
  float sv = 0.f;
  if (r < R) {
    w = *reinterpret_cast<const v4u*>(codes + r * (K >> 1) + g * 32 + h * 16);
    sv = scales[r * G + g];
  }
  uint32_t o[6];
  int4x32_to_fp6x32(w, o);
  *reinterpret_cast<v4u*>(out + h * 768 + l32 * 16) = v4u{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<v2u*>(out + h * 768 + 512 + l32 * 8) = v2u{o[4], o[5]};
  const uint32_t hb = f32_to_bf16(sv);
  const uint32_t lb = f32_to_bf16(sv - bf16_to_f32(hb));
  const v2u so = h == 0 ? v2u{hb | (hb << 16), lb} : v2u{lb, 0u};
  *reinterpret_cast<v2u*>(out + 1536 + lane * 8) = so;
}

// FP4 code and scale blocks of the weight: one wave per (group, 32-row
// tile); lane l copies the 16 code bytes of row l%32, K half l/32, and its
// E8M0 byte.  Rows R .. RP-1 are zero.
__global__ __launch_bounds__(256) void fp4_code_image_kernel(int64_t R, int64_t RT, int K,
                                                             const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             uint8_t* __restrict__ image,
                                                             size_t scale_off) {
  const int G = K >> 6;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= (int64_t)G * RT) return;
  const int g = (int)(blk / RT);
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t r = (blk - (int64_t)g * RT) * 32 + (lane & 31);
  v4u w = {0u, 0u, 0u, 0u};
  uint8_t sc = 0;
  if (r < R) {
    w = *reinterpret_cast<const v4u*>(codes + r * (K >> 1) + g * 32 + h * 16);
    sc = scales[r * (K >> 5) + 2 * g + h];
  }
  *reinterpret_cast<v4u*>(image + blk * F4_CBLOCK + lane * 16) = w;
  image[scale_off + blk * F4_SBLOCK + lane] = sc;
}

// Low-rank and bias blocks of the weight image.  Threads [0, nlr) write one
// 16-byte lane entry of an L2 block each (slice q, column tile ct, lane l:
// column 32 ct + l%32, ranks 16 q + 8 (l/32) .. +7); the next threads write
// the bias blocks and the zero tail, 16 bytes each.
__global__ __launch_bounds__(256) void lr_bias_image_kernel(int N, int rank, int64_t CT,
                                                            const uint16_t* __restrict__ lora_up,
                                                            const uint16_t* __restrict__ bias,
                                                            uint8_t* __restrict__ lr_out,
                                                            uint8_t* __restrict__ bias_out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nlr = (int64_t)(rank / 16) * CT * 64;
  const int64_t nbias = (CT * BIAS_BLOCK + BIAS_TAIL) / 16;
  if (t < nlr) {
    const int64_t blk = t >> 6;  // (q, ct)
    const int l = (int)(t & 63);
    const int q = (int)(blk / CT);
    const int64_t ct = blk - (int64_t)q * CT;
    const int64_t n = ct * 32 + (l & 31);
    v4u v = {0u, 0u, 0u, 0u};
    if (n < N) v = *reinterpret_cast<const v4u*>(lora_up + n * rank + 16 * q + 8 * (l >> 5));
    *reinterpret_cast<v4u*>(lr_out + blk * LR_WBLOCK + 16 * l) = v;
  } else if (t < nlr + nbias) {
    const int64_t e = (t - nlr) * 8;  // first of 8 bf16
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (bias != nullptr) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t n = e + i;
        const uint32_t b = n < N ? bias[n] : 0u;
        w[i >> 1] |= b << (16 * (i & 1));
      }
    }
    *reinterpret_cast<v4u*>(bias_out + 2 * e) = v4u{w[0], w[1], w[2], w[3]};
  }
}

size_t weight_image_bytes(int mode, int N, int K, int rank) {
  return weight_image(mode, N, K, rank).bytes;
}

hipError_t launch_prepare_weight(int mode, int N, int K, int rank, const uint8_t* wcodes,
                                 const void* wscales, const uint16_t* lora_up,
                                 const uint16_t* bias, void* wimage, hipStream_t s) {
  const WeightImage wi = weight_image(mode, N, K, rank);
  uint8_t* img = reinterpret_cast<uint8_t*>(wimage);
  const int64_t blocks = ((int64_t)(K / 64) * wi.CT + 3) / 4;
  if (mode == 0)
    hipLaunchKernelGGL(int4_code_image_kernel, dim3((unsigned)blocks), dim3(256), 0, s, N, wi.CT,
                       K, wcodes, static_cast<const float*>(wscales), img + wi.code);
  else
    hipLaunchKernelGGL(fp4_code_image_kernel, dim3((unsigned)blocks), dim3(256), 0, s, N, wi.CT,
                       K, wcodes, static_cast<const uint8_t*>(wscales), img + wi.code, wi.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nthreads = (int64_t)(rank / 16) * wi.CT * 64 + (wi.CT * BIAS_BLOCK + BIAS_TAIL) / 16;
  hipLaunchKernelGGL(lr_bias_image_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0,
                     s, N, rank, wi.CT, lora_up, bias, img + wi.lr, img + wi.bias);
  return hipGetLastError();
}

}  // namespace svdq
