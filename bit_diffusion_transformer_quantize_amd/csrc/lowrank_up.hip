// Stand-alone up-projection Y += T L2 for the unfused schedule (kept to
// measure what the fusion saves: the apatero.com page, section "O que e
// Nunchaku e como acelera modelos Qwen", quotes the overhead of running the
// low-rank branch as separate kernels).
//
// HBM-bound: Y is read and written once.  128 x 128 output tiles, four waves
// of 2 x 2 MFMA tiles with L2 as the A operand and T as the B operand, so a
// lane's accumulator holds one output row and quads of consecutive columns;
// after one exchange between the lane halves every lane reads, adds and
// writes 16 contiguous bytes of Y (bf16) or 16 bytes per quad (fp32).  T
// enters as bf16 high and low parts (two MFMAs per 16 ranks), as in the
// fused kernels.
#include "gemm_common.h"
#include "kernels.h"

namespace svdq {

constexpr int LU_BM = 128;
constexpr int LU_BN = 128;
constexpr int LU_THREADS = 256;

__global__ __launch_bounds__(LU_THREADS) void lowrank_up_kernel(int64_t M, int N, int rank,
                                                                int out_f32,
                                                                const float* __restrict__ T,
                                                                const uint16_t* __restrict__ lora_up,
                                                                void* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int ntn = N / LU_BN;
  const int64_t mbase = (int64_t)(blockIdx.x / ntn) * LU_BM + (wave >> 1) * 64;
  const int nbase = (blockIdx.x % ntn) * LU_BN + (wave & 1) * 64;
  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  // B operand (T): lane l row l%32, ranks rb + 8 (l/32) .. +7; rows past M
  // read row 0 and are zeroed
  const float* tp[2];
  bool tok[2];
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
    const int64_t m = mbase + tr * 32 + l32;
    tok[tr] = m < M;
    tp[tr] = T + (tok[tr] ? m : 0) * rank + 8 * h;
  }
  // A operand (L2 = lora_up^T): lane l column l%32, the same ranks
  const uint16_t* lp[2];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc) lp[tc] = lora_up + (int64_t)(nbase + tc * 32 + l32) * rank + 8 * h;
  for (int rb = 0; rb < rank; rb += 16) {
    v8bf thi[2], tlo[2], lb[2];
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v4f a = *reinterpret_cast<const v4f*>(tp[tr] + rb);
      const v4f b = *reinterpret_cast<const v4f*>(tp[tr] + rb + 4);
      split_bf16x8(tok[tr] ? a : z, tok[tr] ? b : z, thi[tr], tlo[tr]);
    }
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) lb[tc] = *reinterpret_cast<const v8bf*>(lp[tc] + rb);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], thi[tr], acc[tr][tc], 0, 0, 0);
        acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], tlo[tr], acc[tr][tc], 0, 0, 0);
      }
  }
  // Y += acc: lane l holds row l%32 and columns 8 q + 4 (l/32) .. +3 of each
  // 32-column tile (quad q = element 4q .. 4q+3)
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
    const int64_t m = mbase + tr * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      const int n0 = nbase + tc * 32;
      if (out_f32) {
        float* yr = reinterpret_cast<float*>(Y) + m * N + n0 + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v4f y = *reinterpret_cast<const v4f*>(yr + 8 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += acc[tr][tc][4 * q + e];
          *reinterpret_cast<v4f*>(yr + 8 * q) = y;
        }
      } else {
        // 16-byte chunk qp holds columns 16 qp + 8 (l/32) .. +7: own quad 2qp
        // and the other half's quad 2qp (lanes < 32), the other half's quad
        // 2qp+1 and own quad 2qp+1 (lanes >= 32)
        uint16_t* yr = reinterpret_cast<uint16_t*>(Y) + m * N + n0;
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto sw = __builtin_amdgcn_permlane32_swap(
                __float_as_uint(acc[tr][tc][4 * (2 * qp) + e]),
                __float_as_uint(acc[tr][tc][4 * (2 * qp + 1) + e]), false, false);
            v[e] = __uint_as_float(sw[0]);
            v[4 + e] = __uint_as_float(sw[1]);
          }
          uint16_t* yp = yr + 16 * qp + 8 * h;
          const v4u old = *reinterpret_cast<const v4u*>(yp);
          uint32_t o[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float lo = bf16_to_f32(old[d] & 0xFFFFu) + v[2 * d];
            const float hi = bf16_to_f32(old[d] >> 16) + v[2 * d + 1];
            o[d] = pack_bf16x2(lo, hi);
          }
          *reinterpret_cast<v4u*>(yp) = v4u{o[0], o[1], o[2], o[3]};
        }
      }
    }
  }
}

hipError_t launch_lowrank_up(int rank, bool out_f32, int64_t M, int N, const float* T,
                             const uint16_t* lora_up, void* Y, hipStream_t s) {
  const int64_t tiles = ((M + LU_BM - 1) / LU_BM) * (N / LU_BN);
  hipLaunchKernelGGL(lowrank_up_kernel, dim3((unsigned)tiles), dim3(LU_THREADS), 0, s, M, N,
                     rank, (int)out_f32, T, lora_up, Y);
  return hipGetLastError();
}

}  // namespace svdq
