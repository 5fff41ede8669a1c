// Stand-alone up-projection Y += T L2 for the unfused schedule (kept to
// measure what the fusion saves: the apatero.com page, section "O que e
// Nunchaku e como acelera modelos Qwen", quotes the overhead of running the
// low-rank branch as separate kernels).
#include "gemm_common.h"
#include "kernels.h"

namespace svdq {

constexpr int LU_BM = 128;
constexpr int LU_BN = 128;
constexpr int LU_THREADS = 256;

// 128 x 128 output tiles, four waves of 2 x 2 MFMA tiles.
__global__ __launch_bounds__(LU_THREADS) void lowrank_up_kernel(int64_t M, int N, int rank,
                                                                int out_f32,
                                                                const float* __restrict__ T,
                                                                const uint16_t* __restrict__ lora_up,
                                                                void* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  lowrank_up_tiles<2, 2>(acc, rank, M, N, mbase, nbase, lane, T, lora_up);
  store_tiles<2, 2, true>(acc, M, N, mbase, nbase, lane, nullptr, out_f32 != 0, Y);
}

hipError_t launch_lowrank_up(int rank, bool out_f32, int64_t M, int N, const float* T,
                             const uint16_t* lora_up, void* Y, hipStream_t s) {
  const int64_t tiles = ((M + LU_BM - 1) / LU_BM) * (N / LU_BN);
  hipLaunchKernelGGL(lowrank_up_kernel, dim3((unsigned)tiles), dim3(LU_THREADS), 0, s, M, N,
                     rank, (int)out_f32, T, lora_up, Y);
  return hipGetLastError();
}

}  // namespace svdq
