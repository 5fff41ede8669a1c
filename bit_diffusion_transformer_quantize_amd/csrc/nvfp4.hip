// The NVFP4 variant of the W4A4 layer on gfx950.
//
// NVFP4 (the 4-bit float format the pages name for the FP4 path: Nunchaku
// Lite page on axbrief.com, sections "The Mechanics of 4-Bit Efficiency and
// SVDQuant" and "Hardware Specialization and the Compression Workflow"; the
// layout is NVIDIA's published one) stores E2M1 codes in blocks of 16 along K
// with an FP8 E4M3 scale per block and one fp32 scale g per tensor:
//   t = fp32(6 g); per block a = max |v|, s = E4M3_RNE_sat(fp32(a / t)),
//   d = fp32(s g), code = E2M1_RNE_sat(fp32(v / d)) (all 0 when s = 0);
//   value = code * s * g.
// gfx950's scaled matrix instructions take only power-of-two (E8M0) block
// scales for 32 elements, so an E4M3 scale per 16 cannot ride in them.  A
// code times its block scale has at most 6 significant bits, which bf16
// holds exactly, so the GEMM dequantizes both operands to bf16 in LDS and
// runs the bf16 matrix instruction: every product is exact in fp32 and the
// sums are fp32, as for the other modes.  g_x g_w is applied once per output.
#include <algorithm>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"
#include "nvfp4_codec.h"
#include "weight_residual.h"

namespace svdq {
namespace {

constexpr int NV_BLOCK = 16;

// One block of 16 values: codes (two dwords, element 2j in the low nibble of
// byte j) and the scale byte, for per-tensor scale g and t = fp32(6 g).
__device__ __forceinline__ void nvfp4_block(const float (&v)[16], float g, float t, uint32_t& w0,
                                            uint32_t& w1, uint32_t& sbyte) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
  sbyte = e4m3_encode(a / t);
  const float sv = e4m3_value(sbyte);
  w0 = w1 = 0u;
  if (sv > 0.f) {
    const float d = __fmul_rn(sv, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) w0 |= e2m1_code(v[i] / d) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) w1 |= e2m1_code(v[8 + i] / d) << (4 * i);
  }
}

// g = fp32(max_k amax[k] / 2688), 1 when the maximum is 0 (one workgroup).
__global__ __launch_bounds__(256) void nvfp4_scale_from_absmax_kernel(int n,
                                                                      const float* __restrict__ amax,
                                                                      float* __restrict__ g) {
  __shared__ float red[4];
  float a = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) a = fmaxf(a, amax[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    *g = m > 0.f ? m / 2688.0f : 1.0f;
  }
}

// ------------------------------------------------------------------ weights
// The residual R of the smoothed weight, 16 rows x 64 columns per wave step
// (lane: row l % 16, columns 16 (l / 16)..), as the other modes' packer.
constexpr int NVW_ROWS = 16;

__global__ __launch_bounds__(64) void nvfp4_zero_kernel(uint32_t* __restrict__ p) {
  if (threadIdx.x == 0) *p = 0u;
}

// max |R| over the tensor into *amax_bits (the bits of a non-negative float
// order like the values, so an integer maximum is the float maximum).
__global__ __launch_bounds__(256) void nvfp4_weight_amax_kernel(
    int N, int K, int rank, const uint16_t* __restrict__ W, const float* __restrict__ lambda,
    const uint16_t* __restrict__ lora_down, const uint16_t* __restrict__ lora_up,
    uint32_t* __restrict__ amax_bits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * NVW_ROWS + (lane & 15);
  float a = 0.f;
  for (int t = wave; t < (K >> 6); t += 4) {
    float r[16];
    weight_residual16(n, t * 64 + (lane >> 4) * 16, K, rank, W, lambda, lora_down, lora_up, r);
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(r[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  if (lane == 0) atomicMax(amax_bits, __float_as_uint(a));
}

// In place: the maximum's bits -> g = fp32(amax / 2688), 1 when it is 0.
__global__ __launch_bounds__(64) void nvfp4_weight_scale_kernel(float* __restrict__ g) {
  if (threadIdx.x == 0) {
    const float a = __uint_as_float(*reinterpret_cast<const uint32_t*>(g));
    *g = a > 0.f ? a / 2688.0f : 1.0f;
  }
}

__global__ __launch_bounds__(256) void nvfp4_weight_quant_kernel(
    int N, int K, int rank, const uint16_t* __restrict__ W, const float* __restrict__ lambda,
    const uint16_t* __restrict__ lora_down, const uint16_t* __restrict__ lora_up,
    const float* __restrict__ gptr, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * NVW_ROWS + (lane & 15);
  const float g = *gptr;
  const float t6 = __fmul_rn(6.0f, g);
  for (int t = wave; t < (K >> 6); t += 4) {
    const int k0 = t * 64 + (lane >> 4) * 16;
    float r[16];
    weight_residual16(n, k0, K, rank, W, lambda, lora_down, lora_up, r);
    uint32_t w0, w1, sb;
    nvfp4_block(r, g, t6, w0, w1, sb);
    *reinterpret_cast<v2u*>(codes + (int64_t)n * (K / 2) + k0 / 2) = v2u{w0, w1};
    scales[(int64_t)n * (K / NV_BLOCK) + k0 / NV_BLOCK] = (uint8_t)sb;
  }
}

// ------------------------------------------------------------------ GEMM
// A 256 x 256 output tile per workgroup (8 waves of 64 x 128, 2 x 4 MFMA
// tiles each), K in steps of 64 (four blocks): every thread loads 16 bytes
// of codes (two blocks of 16) and their two scale bytes of one X row and
// one W row and dequantizes them to bf16 in LDS, then each wave issues 32
// v_mfma_f32_32x32x16_bf16 with the weight as the A operand (the transposed
// accumulator layout of gemm_common.h).  LDS holds two steps: while the
// waves' matrix instructions read step ks, each thread dequantizes step
// ks + 1 (its codes loaded during step ks - 1) into the other buffer, so
// the vector and matrix work overlap and one barrier per step separates
// them.  Steps of 64 rather than 32 halve the strided row loads and the
// barriers per K (14% less time at the fused-projection shape; steps of 128
// were slower again), and the second buffer took another 5%.  The
// dequantization is VALU work per element, so the tile is as large as the
// registers allow: 128 elements dequantized per matrix instruction.
// Epilogue: * g_x g_w, + T L2 on the same instruction (T as a bf16 hi/lo
// split), + bias.
constexpr int NV_BM = 256, NV_BN = 256, NV_KS = 64, NV_THREADS = 512;
// LDS holds each operand tile of a step in the matrix instruction's
// fragment order:
// 16-byte unit ((r / 32) * 4 + kb) * 64 + r % 32 + 32 * h holds row r's
// eight values of half h of block kb of the step, so a wave reads a
// fragment as 64 consecutive units and a thread writes each of its blocks
// as two units of a lane-consecutive run (no bank conflicts either way).
constexpr int NV_TILE_UNITS = NV_BM / 32 * 4 * 64;

struct NvRaw {
  v4u xc, wc;
  uint32_t xs, ws;
};

// bf16 values of a block of 16 codes (two dwords) with scale s, by byte
// permutes.  The 8 magnitudes E2M1(i) * s are exact in fp32 with at most 6
// significant bits, so their fp32 bytes 0 and 1 are zero and bytes 2 and 3
// are the bf16 value; tables H (bytes 3) and L (bytes 2) of 8 entries each
// take two dwords.  v_perm_b32 looks up four code magnitudes at a time in
// each (its selector bytes 0-3 address the second source, 4-7 the first),
// and the code's sign goes to bit 7 of the high byte.  The 8 values of a
// code dword come out in the order 0 2 4 6 1 3 5 7 (low nibbles, then high
// nibbles): both operands use this order, and a dot product does not depend
// on the order of its terms.
__device__ __forceinline__ void nv_dequant16(v2u c, float s, v4u& o0, v4u& o1) {
  const uint32_t f1 = __float_as_uint(s * 0.5f), f2 = __float_as_uint(s);
  const uint32_t f3 = __float_as_uint(s * 1.5f), f4 = __float_as_uint(s * 2.0f);
  const uint32_t f5 = __float_as_uint(s * 3.0f), f6 = __float_as_uint(s * 4.0f);
  const uint32_t f7 = __float_as_uint(s * 6.0f);
  const uint32_t p12 = __builtin_amdgcn_perm(f2, f1, 0x07060302u);  // hi16(f1) | hi16(f2) << 16
  const uint32_t p45 = __builtin_amdgcn_perm(f5, f4, 0x07060302u);
  const uint32_t p67 = __builtin_amdgcn_perm(f7, f6, 0x07060302u);
  // entry 0 takes byte 0 of f3, which is zero
  const uint32_t L0 = __builtin_amdgcn_perm(f3, p12, 0x06020004u);
  const uint32_t H0 = __builtin_amdgcn_perm(f3, p12, 0x07030104u);
  const uint32_t L1 = __builtin_amdgcn_perm(p67, p45, 0x06040200u);
  const uint32_t H1 = __builtin_amdgcn_perm(p67, p45, 0x07050301u);
  v4u* o[2] = {&o0, &o1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = c[h];
    const uint32_t ml = w & 0x07070707u, mh = (w >> 4) & 0x07070707u;
    const uint32_t hl = __builtin_amdgcn_perm(H1, H0, ml) | ((w << 4) & 0x80808080u);
    const uint32_t hh = __builtin_amdgcn_perm(H1, H0, mh) | (w & 0x80808080u);
    const uint32_t ll = __builtin_amdgcn_perm(L1, L0, ml);
    const uint32_t lh = __builtin_amdgcn_perm(L1, L0, mh);
    (*o[h])[0] = __builtin_amdgcn_perm(hl, ll, 0x05010400u);
    (*o[h])[1] = __builtin_amdgcn_perm(hl, ll, 0x07030602u);
    (*o[h])[2] = __builtin_amdgcn_perm(hh, lh, 0x05010400u);
    (*o[h])[3] = __builtin_amdgcn_perm(hh, lh, 0x07030602u);
  }
}

__global__ __launch_bounds__(NV_THREADS) void nvfp4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ xcodes,
    const uint8_t* __restrict__ xscales, const float* __restrict__ gx,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales,
    const float* __restrict__ gw, const float* __restrict__ T,
    const uint16_t* __restrict__ lora_up, const uint16_t* __restrict__ bias,
    void* __restrict__ Y) {
  __shared__ v4u xs_l[2][NV_TILE_UNITS];
  __shared__ v4u ws_l[2][NV_TILE_UNITS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * NV_BM;
  const int n0 = blockIdx.y * NV_BN;
  const int nbk = K / NV_BLOCK;
  // this thread's blocks of each operand: row 32 * wave + lane % 32, blocks
  // 2 (lane / 32) and 2 (lane / 32) + 1 of the step; rows past M or N are read from the last row (their
  // outputs are not stored)
  const int lr = 32 * wave + (lane & 31), kb = lane >> 5;
  const int64_t xrow = std::min<int64_t>(m0 + lr, M - 1);
  const int64_t wrow = std::min(n0 + lr, N - 1);
  const uint8_t* xcp = xcodes + xrow * (K / 2) + kb * 16;
  const uint8_t* xsp = xscales + xrow * nbk + kb * 2;
  const uint8_t* wcp = wcodes + wrow * (K / 2) + kb * 16;
  const uint8_t* wsp = wscales + wrow * nbk + kb * 2;
  auto load = [&](int ks, NvRaw& r) {
    r.xc = *reinterpret_cast<const v4u*>(xcp + ks * (NV_KS / 2));
    r.wc = *reinterpret_cast<const v4u*>(wcp + ks * (NV_KS / 2));
    r.xs = *reinterpret_cast<const uint16_t*>(xsp + ks * 4);
    r.ws = *reinterpret_cast<const uint16_t*>(wsp + ks * 4);
  };
  const int dst = (wave * 4 + 2 * kb) * 64 + (lane & 31);
  v16f acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nks = K / NV_KS;
  // dequantize a step's raw codes into buffer b; gfx950's fp8 conversion
  // decodes an OCP E4M3 byte exactly (subnormals included): the same value
  // as e4m3_value in one instruction
  auto stage = [&](const NvRaw& r, int b) {
    v4u a0, a1, a2, a3, b0, b1, b2, b3;
    nv_dequant16(v2u{r.xc[0], r.xc[1]}, __builtin_amdgcn_cvt_f32_fp8((int)r.xs, 0), a0, a1);
    nv_dequant16(v2u{r.xc[2], r.xc[3]}, __builtin_amdgcn_cvt_f32_fp8((int)r.xs, 1), a2, a3);
    nv_dequant16(v2u{r.wc[0], r.wc[1]}, __builtin_amdgcn_cvt_f32_fp8((int)r.ws, 0), b0, b1);
    nv_dequant16(v2u{r.wc[2], r.wc[3]}, __builtin_amdgcn_cvt_f32_fp8((int)r.ws, 1), b2, b3);
    xs_l[b][dst] = a0;
    xs_l[b][dst + 32] = a1;
    xs_l[b][dst + 64] = a2;
    xs_l[b][dst + 96] = a3;
    ws_l[b][dst] = b0;
    ws_l[b][dst + 32] = b1;
    ws_l[b][dst + 64] = b2;
    ws_l[b][dst + 96] = b3;
  };
  NvRaw nxt;
  {
    NvRaw r0;
    load(0, r0);
    load(std::min(1, nks - 1), nxt);
    stage(r0, 0);
  }
  const int l32 = lane & 31;
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int b = ks & 1;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      v8bf af[4], bfr[2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[t] = __builtin_bit_cast(v8bf, ws_l[b][((wn * 4 + t) * 4 + k2) * 64 + lane]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        bfr[t] = __builtin_bit_cast(v8bf, xs_l[b][((wm * 2 + t) * 4 + k2) * 64 + lane]);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < 4; ++tc)
          acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tc], bfr[tr], acc[tr][tc], 0, 0, 0);
    }
    if (ks + 1 < nks) {
      stage(nxt, b ^ 1);
      load(std::min(ks + 2, nks - 1), nxt);
    }
    __syncthreads();
  }

  const int kh = (lane >> 5) * 8;
  const int64_t mbase = m0 + wm * 64;
  const int nbase = n0 + wn * 128;
  if (nbase >= N) return;  // a partial last column tile: this wave's columns are all past N
  const float gg = __fmul_rn(*gx, *gw);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = __fmul_rn(acc[a][b][i], gg);
  // T L2: T rows (B operand, bf16 hi + lo), lora_up rows (A operand)
  for (int q0 = 0; q0 < rank; q0 += 16) {
    v8bf lu[4], thi[2], tlo[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      lu[t] = *reinterpret_cast<const v8bf*>(lora_up + (int64_t)(nbase + 32 * t + l32) * rank + q0 + kh);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t tm = std::min<int64_t>(mbase + 32 * t + l32, M - 1);
      const v4f t0 = *reinterpret_cast<const v4f*>(T + tm * rank + q0 + kh);
      const v4f t1 = *reinterpret_cast<const v4f*>(T + tm * rank + q0 + kh + 4);
      const float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = f32_to_bf16(tv[e]);
        thi[t][e] = __builtin_bit_cast(__bf16, (uint16_t)h);
        tlo[t][e] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16(tv[e] - bf16_to_f32(h)));
      }
    }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int tc = 0; tc < 4; ++tc) {
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lu[tc], thi[tr], acc[tr][tc], 0, 0, 0);
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lu[tc], tlo[tr], acc[tr][tc], 0, 0, 0);
      }
  }
  if (bias != nullptr) {
#pragma unroll
    for (int tc = 0; tc < 4; ++tc)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float bv = bf16_to_f32(bias[nbase + 32 * tc + acc_row(i, lane)]);
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) acc[tr][tc][i] = __fadd_rn(acc[tr][tc][i], bv);
      }
  }
  store_tiles_t<2, 4>(acc, M, N, mbase, nbase, lane, out_f32 != 0, Y);
}

}  // namespace

hipError_t launch_nvfp4_scale_from_absmax(int n, const float* amax, float* g, hipStream_t s) {
  hipLaunchKernelGGL(nvfp4_scale_from_absmax_kernel, dim3(1), dim3(256), 0, s, n, amax, g);
  return hipGetLastError();
}

hipError_t launch_nvfp4_pack_weight(int N, int K, int rank, const uint16_t* W, const float* lambda,
                                    const uint16_t* lora_down, const uint16_t* lora_up,
                                    uint8_t* codes, uint8_t* scales, float* g, hipStream_t s) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(g);
  hipLaunchKernelGGL(nvfp4_zero_kernel, dim3(1), dim3(64), 0, s, bits);
  hipLaunchKernelGGL(nvfp4_weight_amax_kernel, dim3(N / NVW_ROWS), dim3(256), 0, s, N, K, rank, W,
                     lambda, lora_down, lora_up, bits);
  hipLaunchKernelGGL(nvfp4_weight_scale_kernel, dim3(1), dim3(64), 0, s, g);
  hipLaunchKernelGGL(nvfp4_weight_quant_kernel, dim3(N / NVW_ROWS), dim3(256), 0, s, N, K, rank, W,
                     lambda, lora_down, lora_up, g, codes, scales);
  return hipGetLastError();
}

hipError_t launch_nvfp4_linear(bool out_f32, int64_t M, int N, int K, int rank,
                               const uint8_t* xcodes, const uint8_t* xscales, const float* gx,
                               const uint8_t* wcodes, const uint8_t* wscales, const float* gw,
                               const float* T, const uint16_t* lora_up, const uint16_t* bias,
                               void* Y, hipStream_t s) {
  const dim3 grid((unsigned)((M + NV_BM - 1) / NV_BM), (N + NV_BN - 1) / NV_BN);
  hipLaunchKernelGGL(nvfp4_gemm_kernel, grid, dim3(NV_THREADS), 0, s, M, N, K, rank, (int)out_f32, xcodes,
                     xscales, gx, wcodes, wscales, gw, T, lora_up, bias, Y);
  return hipGetLastError();
}

}  // namespace svdq
