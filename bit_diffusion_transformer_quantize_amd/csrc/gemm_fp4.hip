// FP4-mode (MXFP4: E2M1 codes, E8M0 block scales) W4A4 GEMM of the SVDQuant
// linear on gfx950, with the low-rank up-projection and the bias in its
// epilogue.
//
// The Nunchaku engine fuses the up-projection of the 16-bit low-rank branch
// into the 4-bit compute kernel (apatero.com page, section "O que e Nunchaku
// e como acelera modelos Qwen"); the 4-bit floating-point precision is the
// one the pages pair with newer hardware (axbrief.com page, section
// "Hardware Specialization and the Compression Workflow").
//
// A fragment of 32 E2M1 codes of one row is the operand of
// v_mfma_scale_f32_32x32x64_f8f6f4 as stored; the E8M0 block scales go to the
// instruction's scale operands, so the hardware applies them and the whole K
// accumulation stays in the MFMA.  A 256-thread workgroup computes a 128x128
// tile of Y (four waves of 2x2 MFMA tiles); packed tiles of 128 K-elements
// are staged through LDS with double buffering, rows padded to 80 bytes.
#include "gemm_common.h"
#include "kernels.h"

namespace svdq {

constexpr int GM_BM = 128;
constexpr int GM_BN = 128;
constexpr int GM_BK = 128;  // K elements per LDS stage (64 bytes of codes per row)
constexpr int GM_THREADS = 256;
constexpr int LDS_ROW = 80;  // bytes per staged row: 64 + 16 padding

__global__ __launch_bounds__(GM_THREADS) void fp4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ xcodes,
    const uint8_t* __restrict__ xscales, const float* __restrict__ T,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales,
    const uint16_t* __restrict__ lora_up, const uint16_t* __restrict__ bias,
    void* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][GM_BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][GM_BN * LDS_ROW];
  // The four E8M0 bytes of one stage (4 blocks of 32) for each row.
  __shared__ __attribute__((aligned(16))) uint32_t SX[2][GM_BM];
  __shared__ __attribute__((aligned(16))) uint32_t SW[2][GM_BN];

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
  const int SB = K >> 5;
  const int nstages = K / GM_BK;
  const int ld_row = tid >> 2, ld_chunk = tid & 3;
  const int h = lane >> 5;

  v4u ga[2], gb[2];
  uint32_t gs = 0;

  auto global_load = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ld_row + 64 * i;
      const int64_t m = m0 + r;
      ga[i] = v4u{0u, 0u, 0u, 0u};
      if (m < M) ga[i] = *reinterpret_cast<const v4u*>(xcodes + m * KB + s * 64 + ld_chunk * 16);
      gb[i] = *reinterpret_cast<const v4u*>(wcodes + (int64_t)(n0 + r) * KB + s * 64 + ld_chunk * 16);
    }
    if (tid < GM_BM) {
      const int64_t m = m0 + tid;
      gs = 0;
      if (m < M) gs = *reinterpret_cast<const uint32_t*>(xscales + m * SB + 4 * s);
    } else {
      gs = *reinterpret_cast<const uint32_t*>(wscales + (int64_t)(n0 + tid - GM_BM) * SB + 4 * s);
    }
  };
  auto lds_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ld_row + 64 * i;
      *reinterpret_cast<v4u*>(&As[buf][r * LDS_ROW + ld_chunk * 16]) = ga[i];
      *reinterpret_cast<v4u*>(&Bs[buf][r * LDS_ROW + ld_chunk * 16]) = gb[i];
    }
    if (tid < GM_BM)
      SX[buf][tid] = gs;
    else
      SW[buf][tid - GM_BM] = gs;
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
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[2], bf[2];
      int sa[2], sb[2];
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const int r = wm * 64 + tr * 32 + (lane & 31);
        const v4u w = *reinterpret_cast<const v4u*>(&As[buf][r * LDS_ROW + ks * 32 + h * 16]);
        af[tr] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
        // lane l supplies the scale of (row l%32, block l/32) of this K-step
        sa[tr] = (int)(SX[buf][r] >> (8 * (2 * ks + h)));
      }
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const int r = wn * 64 + tc * 32 + (lane & 31);
        const v4u w = *reinterpret_cast<const v4u*>(&Bs[buf][r * LDS_ROW + ks * 32 + h * 16]);
        bf[tc] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
        sb[tc] = (int)(SW[buf][r] >> (8 * (2 * ks + h)));
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < 2; ++tc)
          acc[tr][tc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[tr], bf[tc], acc[tr][tc], 4, 4, 0, sa[tr], 0, sb[tc]);
    }
    if (s + 1 < nstages) lds_store(buf ^ 1);
    __syncthreads();
  }

  const int64_t mbase = m0 + wm * 64;
  const int nbase = n0 + wn * 64;
  if (T != nullptr) lowrank_up_tiles<2, 2>(acc, rank, M, N, mbase, nbase, lane, T, lora_up);
  store_tiles<2, 2, false>(acc, M, N, mbase, nbase, lane, bias, out_f32 != 0, Y);
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
  lowrank_up_tiles<2, 2>(acc, rank, M, N, mbase, nbase, lane, T, lora_up);
  store_tiles<2, 2, true>(acc, M, N, mbase, nbase, lane, nullptr, out_f32 != 0, Y);
}

// The FP4 weight image is the packed codes [N][K/2] followed, at the next
// 256-byte boundary, by the E8M0 scales [N][K/32].
static size_t fp4_scale_offset(int N, int K) {
  return ((size_t)N * (K / 2) + 255) & ~size_t(255);
}

size_t fp4_weight_image_bytes(int N, int K) {
  return fp4_scale_offset(N, K) + (size_t)N * (K / 32);
}

hipError_t launch_fp4_prepare_weight(int N, int K, const uint8_t* wcodes, const uint8_t* wscales,
                                     void* wimage, hipStream_t s) {
  uint8_t* img = reinterpret_cast<uint8_t*>(wimage);
  hipError_t e = hipMemcpyAsync(img, wcodes, (size_t)N * (K / 2), hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  return hipMemcpyAsync(img + fp4_scale_offset(N, K), wscales, (size_t)N * (K / 32),
                        hipMemcpyDeviceToDevice, s);
}

hipError_t launch_fp4_forward(int rank, bool out_f32, int64_t M, int N, int K,
                              const uint8_t* xcodes, const uint8_t* xscales, const float* T,
                              const void* wimage, const uint16_t* lora_up, const uint16_t* bias,
                              void* Y, hipStream_t s) {
  const uint8_t* wcodes = reinterpret_cast<const uint8_t*>(wimage);
  const uint8_t* wscales = wcodes + fp4_scale_offset(N, K);
  const int64_t tiles = ((M + GM_BM - 1) / GM_BM) * (N / GM_BN);
  hipLaunchKernelGGL(fp4_gemm_kernel, dim3((unsigned)tiles), dim3(GM_THREADS), 0, s, M, N, K,
                     rank, (int)out_f32, xcodes, xscales, T, wcodes, wscales, lora_up, bias, Y);
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
