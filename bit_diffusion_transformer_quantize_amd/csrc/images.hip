// Builders of the prepared weight (image.h): the packed weight codes and
// scales re-laid in MFMA lane order, the low-rank factor L2 and the bias.
// This is offline work, done once per layer (like the one-time packing of
// the 4-bit weights into the kernel layout that the apatero.com page
// describes, section "O que e Nunchaku e como acelera modelos Qwen").
#include "common.h"
#include "image.h"
#include "kernels.h"

namespace svdq {

// The code blocks are written one wave per (group, 32-row tile).  A
// workgroup of four waves takes one row tile and four consecutive groups:
// it first stages the 32 rows' 128-byte runs of packed codes (and their
// scales) in LDS, each load covering whole row segments (8 lanes per row:
// 8 cache lines in full, where loading in the lanes' final order touches 32
// lines, a quarter of each), then each wave reads its group's block back in
// lane order.  The 16-byte chunk c of staged row n sits at position
// c ^ (n % 8), so both sides meet every bank once per eight lanes.

// INT4 code block: lane l converts the 32 codes w of row l%32, K half l/32,
// to E2M3 sign-magnitude fields of 6 bits (value q/8, exact for every code)
// packed little-endian into six dwords, by the gfx950 conversion to FP6
// (scale operand 8: it divides by 2^3; its two sources give the even and
// the odd fields).  Scale operand, W pattern: lanes 0..31
// {hi | hi << 16, lo}, lanes 32..63 {lo, 0}, so that with the activation
// pattern {hi | lo << 16, hi} / {lo, 0} the K slots 0..3 of the
// outer-product MFMA hold hi*hi, lo*hi, hi*lo, 0 and slot 4 lo*lo.
// ACT: the activation pattern of the scale operand instead of the weight
// one (lanes 0..31 {hi | lo << 16, hi}, lanes 32..63 {lo, 0}).
template <bool ACT>
__device__ __forceinline__ void int4_code_block(uint8_t* __restrict__ out, int lane, const v4u& w,
                                                float sv) {
  const int h = lane >> 5, l32 = lane & 31;
  v16f ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // element 2i is the low nibble of byte i, 2i + 1 the high one
    const uint32_t byte = w[i >> 2] >> (8 * (i & 3));
    ev[i] = (float)((int32_t)(byte << 28) >> 28);
    od[i] = (float)((int32_t)(byte << 24) >> 28);
  }
  const v6i f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
  *reinterpret_cast<v4u*>(out + h * 768 + l32 * 16) =
      v4u{(uint32_t)f[0], (uint32_t)f[1], (uint32_t)f[2], (uint32_t)f[3]};
  *reinterpret_cast<v2u*>(out + h * 768 + 512 + l32 * 8) = v2u{(uint32_t)f[4], (uint32_t)f[5]};
  const uint32_t hb = f32_to_bf16(sv);
  const uint32_t lb = f32_to_bf16(sv - bf16_to_f32(hb));
  const v2u so = h == 0 ? (ACT ? v2u{hb | (lb << 16), hb} : v2u{hb | (hb << 16), lb}) : v2u{lb, 0u};
  *reinterpret_cast<v2u*>(out + 1536 + lane * 8) = so;
}

// The code blocks of row tile rt, groups 4 quad .. 4 quad + 3 (MODE 0 INT4,
// 1 FP4: the 16 code bytes as they are and the E8M0 byte of row l%32, K half
// l/32).  Rows R .. RP-1 and groups past G come out as zeros.
template <int MODE, bool ACT>
__device__ __forceinline__ void code_blocks(int64_t R, int64_t RT, int K, int64_t rt, int quad,
                                            const uint8_t* __restrict__ codes,
                                            const void* __restrict__ scales,
                                            uint8_t* __restrict__ image, size_t scale_off) {
  __shared__ v4u cst[32][8];
  __shared__ uint32_t sst[32][9];  // INT4: fp32 scale bits [row][group]; FP4: bytes [row][2 group + half]
  const int G = K >> 6;
  const int t = threadIdx.x;
  {
    const int row = t >> 3, c = t & 7;
    const int64_t r = rt * 32 + row;
    v4u v = {0u, 0u, 0u, 0u};
    if (r < R && quad * 4 + (c >> 1) < G)
      v = *reinterpret_cast<const v4u*>(codes + r * (K >> 1) + quad * 128 + c * 16);
    cst[row][c ^ (row & 7)] = v;
    if constexpr (MODE == 0) {
      if (t < 128) {
        const int row2 = t >> 2, j = t & 3;
        const int64_t r2 = rt * 32 + row2;
        const int g = quad * 4 + j;
        sst[row2][j] = (r2 < R && g < G)
                           ? __float_as_uint(static_cast<const float*>(scales)[r2 * G + g])
                           : 0u;
      }
    } else {
      // lane t: row t/8, byte t%8 of the row's run of scale bytes
      const int64_t r2 = rt * 32 + row;
      const int b = quad * 8 + c;
      sst[row][c] = (r2 < R && b < 2 * G)
                        ? (uint32_t) static_cast<const uint8_t*>(scales)[r2 * (K >> 5) + b]
                        : 0u;
    }
  }
  __syncthreads();
  const int w = t >> 6, lane = t & 63;
  const int g = quad * 4 + w;
  if (g >= G) return;
  const int h = lane >> 5, l32 = lane & 31;
  const v4u cw = cst[l32][(2 * w + h) ^ (l32 & 7)];
  const int64_t blk = (int64_t)g * RT + rt;
  if constexpr (MODE == 0) {
    int4_code_block<ACT>(image + blk * I4_BLOCK, lane, cw, __uint_as_float(sst[l32][w]));
  } else {
    *reinterpret_cast<v4u*>(image + blk * F4_CBLOCK + lane * 16) = cw;
    image[scale_off + blk * F4_SBLOCK + lane] = (uint8_t)sst[l32][2 * w + h];
  }
}

// Low-rank and bias blocks of the weight image.  Thread t < nlr writes one
// 16-byte lane entry of an L2 block (slice q, column tile ct, lane l: column
// 32 ct + l%32, ranks 16 q + 8 (l/32) .. +7); the next threads write the
// bias blocks and the zero tail, 16 bytes each.
__device__ __forceinline__ void lr_bias_entry(int N, int rank, int64_t CT, int64_t t,
                                              const uint16_t* __restrict__ lora_up,
                                              const uint16_t* __restrict__ bias,
                                              uint8_t* __restrict__ lr_out,
                                              uint8_t* __restrict__ bias_out) {
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

// The whole prepared weight in one launch: workgroups [0, ncode) write the
// code blocks (one per row tile and four groups), the rest the low-rank and
// bias blocks.
template <int MODE>
__global__ __launch_bounds__(256) void weight_image_kernel(int N, int K, int rank, int64_t RT,
                                                           int64_t ncode,
                                                           const uint8_t* __restrict__ codes,
                                                           const void* __restrict__ scales,
                                                           const uint16_t* __restrict__ lora_up,
                                                           const uint16_t* __restrict__ bias,
                                                           uint8_t* __restrict__ img,
                                                           WeightImage wi) {
  if ((int64_t)blockIdx.x < ncode) {
    const int nq = ((K >> 6) + 3) >> 2;  // group quads per row tile
    const int64_t rt = (int64_t)blockIdx.x / nq;
    code_blocks<MODE, false>(N, RT, K, rt, (int)((int64_t)blockIdx.x - rt * nq), codes, scales,
                             img + wi.code, wi.scale);
    return;
  }
  const int64_t t = ((int64_t)blockIdx.x - ncode) * 256 + threadIdx.x;
  lr_bias_entry(N, rank, RT, t, lora_up, bias, img + wi.lr, img + wi.bias);
}

hipError_t launch_prepare_weight(int mode, int N, int K, int rank, const uint8_t* wcodes,
                                 const void* wscales, const uint16_t* lora_up,
                                 const uint16_t* bias, void* wimage, hipStream_t s) {
  const WeightImage wi = weight_image(mode, N, K, rank);
  uint8_t* img = reinterpret_cast<uint8_t*>(wimage);
  const int64_t ncode = (int64_t)((K / 64 + 3) / 4) * wi.CT;
  const int64_t nthreads = (int64_t)(rank / 16) * wi.CT * 64 + (wi.CT * BIAS_BLOCK + BIAS_TAIL) / 16;
  const dim3 grid((unsigned)(ncode + (nthreads + 255) / 256));
  if (mode == 0)
    hipLaunchKernelGGL(weight_image_kernel<0>, grid, dim3(256), 0, s, N, K, rank, wi.CT, ncode,
                       wcodes, wscales, lora_up, bias, img, wi);
  else
    hipLaunchKernelGGL(weight_image_kernel<1>, grid, dim3(256), 0, s, N, K, rank, wi.CT, ncode,
                       wcodes, wscales, lora_up, bias, img, wi);
  return hipGetLastError();
}

// The activation image from the row-major codes, scales and T (rather than
// from X, as the activation pass writes it): workgroups [0, ncode) write the
// code blocks as for the weight image, with the activation pattern of the
// INT4 scale operand; the rest the low-rank blocks, one 16-byte lane entry
// of T hi and of T lo per thread (slice q, row tile rt, lane l: row
// 32 rt + l%32, ranks 16 q + 8 (l/32) .. +7; rows past M are zero).  The
// partial-sum region of the image is not used by the GEMM and is left as
// it is.
template <int MODE>
__global__ __launch_bounds__(256) void act_image_kernel(int64_t M, int K, int rank, int64_t ncode,
                                                        const uint8_t* __restrict__ codes,
                                                        const void* __restrict__ scales,
                                                        const float* __restrict__ T,
                                                        uint8_t* __restrict__ img, ActImage ai) {
  if ((int64_t)blockIdx.x < ncode) {
    const int nq = ((K >> 6) + 3) >> 2;  // group quads per row tile
    const int64_t rt = (int64_t)blockIdx.x / nq;
    code_blocks<MODE, true>(M, ai.RT, K, rt, (int)((int64_t)blockIdx.x - rt * nq), codes, scales,
                            img + ai.code, ai.scale);
    return;
  }
  const int64_t t = ((int64_t)blockIdx.x - ncode) * 256 + threadIdx.x;
  const int64_t nlr = (int64_t)(rank / 16) * ai.RT * 64;
  if (t >= nlr) return;
  const int64_t blk = t >> 6;  // (q, rt)
  const int l = (int)(t & 63);
  const int q = (int)(blk / ai.RT);
  const int64_t rt = blk - (int64_t)q * ai.RT;
  const int64_t m = rt * 32 + (l & 31);
  v4f a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  if (m < M) {
    const float* tr = T + m * rank + 16 * q + 8 * (l >> 5);
    a = *reinterpret_cast<const v4f*>(tr);
    b = *reinterpret_cast<const v4f*>(tr + 4);
  }
  // hi = bf16_RNE(T), lo = bf16_RNE(T - hi), as the activation pass writes them
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    hi[i] = h0 | (h1 << 16);
    lo[i] = f32_to_bf16(v[2 * i] - bf16_to_f32(h0)) |
            (f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1)) << 16);
  }
  uint8_t* out = img + ai.lr + blk * LR_XBLOCK;
  *reinterpret_cast<v4u*>(out + 16 * l) = v4u{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<v4u*>(out + 1024 + 16 * l) = v4u{lo[0], lo[1], lo[2], lo[3]};
}

hipError_t launch_act_image_from_codes(int mode, int64_t M, int K, int rank, const uint8_t* xcodes,
                                       const void* xscales, const float* T, void* ximage,
                                       hipStream_t s) {
  const ActImage ai = act_image(mode, M, K, rank);
  uint8_t* img = reinterpret_cast<uint8_t*>(ximage);
  const int64_t ncode = (int64_t)((K / 64 + 3) / 4) * ai.RT;
  const int64_t nthreads = (int64_t)(rank / 16) * ai.RT * 64;
  const dim3 grid((unsigned)(ncode + (nthreads + 255) / 256));
  if (mode == 0)
    hipLaunchKernelGGL(act_image_kernel<0>, grid, dim3(256), 0, s, M, K, rank, ncode, xcodes,
                       xscales, T, img, ai);
  else
    hipLaunchKernelGGL(act_image_kernel<1>, grid, dim3(256), 0, s, M, K, rank, ncode, xcodes,
                       xscales, T, img, ai);
  return hipGetLastError();
}

size_t weight_image_bytes(int mode, int N, int K, int rank) {
  return weight_image(mode, N, K, rank).bytes;
}

}  // namespace svdq
