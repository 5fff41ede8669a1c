// FP4-mode (MXFP4: E2M1 codes, E8M0 block scales) W4A4 GEMM of the SVDQuant
// linear on gfx950, with the low-rank up-projection and the bias in the
// prologue of each output tile.
//
// The Nunchaku engine fuses the up-projection of the 16-bit low-rank branch
// into the 4-bit compute kernel (apatero.com page, section "O que e Nunchaku
// e como acelera modelos Qwen"); the 4-bit floating-point precision is the
// one the pages pair with newer hardware (axbrief.com page, section
// "Hardware Specialization and the Compression Workflow").
//
// A fragment of 32 E2M1 codes of one row is the operand of
// v_mfma_scale_f32_32x32x64_f8f6f4 as stored; lane l supplies the E8M0
// scale of (row l%32, 32-block l/32), so the hardware applies the scales and
// the whole K accumulation stays in the MFMA: no per-group vector work.
//
// Operand images (same idea as the INT4 ones).  Rows are padded to a
// multiple of 256; per (64-group g, 32-row tile) there is
//   a 1024-byte code block: lane l's 16 bytes at 16 l are the codes of row
//     l%32, K elements 64 g + 32 (l/32) .. +31 (a plain copy of the packed
//     row), and
//   a 64-byte scale block: byte l is the E8M0 scale of that row and block.
// The code blocks of all groups come first ([G][rows/32][1024]), then the
// scale blocks ([G][rows/32][64]).  A workgroup's stage is then four
// contiguous runs (8 KB of X codes, 8 KB of W codes, 512 B of each side's
// scales) copied by the global->LDS DMA.
//
// Pipeline: a 512-thread workgroup computes 256 x 256 outputs; each of its 8
// waves owns 64 x 128 (2 x 4 tiles).  One stage = two 64-groups; LDS holds a
// ring of 4 stage slots, the DMA runs two stages ahead, and the fragments of
// the next group are read while the MFMAs of the current one run, so there
// is one barrier per two groups.
#include <type_traits>

#include "gemm_common.h"
#include "kernels.h"

namespace svdq {

constexpr int F4_BM = 256;
constexpr int F4_BN = 256;
constexpr int F4_THREADS = 512;
constexpr int F4_GROUP_M = 2;
constexpr int F4_NSLOT = 4;
constexpr int F4_CODE_BLOCK = 1024;  // bytes per (group, 32 rows)
constexpr int F4_SCALE_BLOCK = 64;
constexpr int F4_SL_BCODES = 8 * F4_CODE_BLOCK;             // W codes after 8 KB of X codes
constexpr int F4_SL_XSCALES = 16 * F4_CODE_BLOCK;           // then 512 B of X scales
constexpr int F4_SL_WSCALES = F4_SL_XSCALES + 8 * F4_SCALE_BLOCK;
constexpr int F4_GRP = F4_SL_WSCALES + 8 * F4_SCALE_BLOCK;  // 17408 bytes per group
constexpr int F4_SLOT = 2 * F4_GRP;                          // a stage holds two groups
constexpr int FP4_FMT = 4;                                   // f8f6f4 format code of E2M1

typedef __attribute__((address_space(3))) void lds_void_f4;

__host__ __device__ static inline int64_t f4_pad(int64_t R) { return (R + 255) / 256 * 256; }
// Bytes of an FP4 operand image of RP (padded) rows.
__host__ __device__ static inline size_t f4_image_bytes(int64_t RP, int K) {
  return (size_t)(K / 64) * (size_t)(RP / 32) * (F4_CODE_BLOCK + F4_SCALE_BLOCK);
}
__host__ __device__ static inline size_t f4_scale_offset(int64_t RP, int K) {
  return (size_t)(K / 64) * (size_t)(RP / 32) * F4_CODE_BLOCK;
}

size_t fp4_workspace_bytes(int64_t M, int K) {
  return (f4_image_bytes(f4_pad(M), K) + 255) & ~size_t(255);
}
size_t fp4_weight_image_bytes(int N, int K) { return f4_image_bytes(f4_pad(N), K); }

// Global -> LDS DMA of 16 (dwordx4) or 4 (dword) bytes per lane with a
// scalar base; see the INT4 kernel for why this is an asm block.
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma16_f4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_f4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// One wave per (group, 32-row tile): the code block (a 16-byte copy per
// lane) and the scale block.  Rows R .. RP-1 are zero.
__global__ __launch_bounds__(256) void fp4_image_kernel(int64_t R, int64_t RP, int K,
                                                        const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        uint8_t* __restrict__ image) {
  const int G = K >> 6;
  const int64_t RT = RP >> 5;
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
  *reinterpret_cast<v4u*>(image + blk * F4_CODE_BLOCK + lane * 16) = w;
  image[f4_scale_offset(RP, K) + blk * F4_SCALE_BLOCK + lane] = sc;
}

static hipError_t launch_fp4_image(int64_t R, int64_t RP, int K, const uint8_t* codes,
                                   const uint8_t* scales, uint8_t* image, hipStream_t s) {
  const int64_t blocks = ((int64_t)(K / 64) * (RP / 32) + 3) / 4;
  hipLaunchKernelGGL(fp4_image_kernel, dim3((unsigned)blocks), dim3(256), 0, s, R, RP, K, codes,
                     scales, image);
  return hipGetLastError();
}

hipError_t launch_fp4_prepare_weight(int N, int K, const uint8_t* wcodes, const uint8_t* wscales,
                                     void* wimage, hipStream_t s) {
  return launch_fp4_image(N, f4_pad(N), K, wcodes, wscales, reinterpret_cast<uint8_t*>(wimage), s);
}

__global__ __launch_bounds__(F4_THREADS) void fp4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ ximg,
    int x_tiles, const uint8_t* __restrict__ wimg, int w_tiles, const float* __restrict__ T,
    const uint16_t* __restrict__ lora_up, const uint16_t* __restrict__ bias,
    void* __restrict__ Y) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[F4_NSLOT * F4_SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile order: XCD-contiguous ranges, grouped by F4_GROUP_M tile rows
  const int num_m = x_tiles / (F4_BM / 32);
  const int num_n = w_tiles / (F4_BN / 32);
  const int nb = gridDim.x;
  int L = blockIdx.x;
  if ((nb & 7) == 0) L = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int band = L / (F4_GROUP_M * num_n);
  const int first_m = band * F4_GROUP_M;
  const int gm = min(num_m - first_m, F4_GROUP_M);
  const int in_band = L - band * F4_GROUP_M * num_n;
  const int tile_m = first_m + in_band % gm;
  const int tile_n = in_band / gm;
  const int64_t m0 = (int64_t)tile_m * F4_BM;
  const int n0 = tile_n * F4_BN;
  const int G = K >> 6;

  // ---- DMA plan per group: code chunks w (X) and w+8 (W) of 1 KB, and one
  // 256-byte scale chunk: (w & 3) = X scales rows 0-127, 128-255, W scales
  // rows 0-127, 128-255 (waves 4..7 repeat the chunk of wave w-4: the same
  // bytes to the same place), so every wave has three DMAs per group.
  const uint8_t* xrun = ximg + (int64_t)tile_m * 8 * F4_CODE_BLOCK;
  const uint8_t* wrun = wimg + (int64_t)tile_n * 8 * F4_CODE_BLOCK;
  const uint8_t* xsrun = ximg + f4_scale_offset((int64_t)x_tiles * 32, K) +
                         (int64_t)tile_m * 8 * F4_SCALE_BLOCK;
  const uint8_t* wsrun = wimg + f4_scale_offset((int64_t)w_tiles * 32, K) +
                         (int64_t)tile_n * 8 * F4_SCALE_BLOCK;
  const int64_t xstride = (int64_t)x_tiles * F4_CODE_BLOCK, wstride = (int64_t)w_tiles * F4_CODE_BLOCK;
  const int64_t xsstride = (int64_t)x_tiles * F4_SCALE_BLOCK, wsstride = (int64_t)w_tiles * F4_SCALE_BLOCK;
  const uint32_t voff_c = (uint32_t)(wave * 1024 + lane * 16);
  const int sch = wave & 3;
  const uint32_t voff_s = (uint32_t)((sch & 1) * 256 + lane * 4);
  const bool s_w = sch >= 2;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_f4*)lds;
  // DMA of one group into its half of its stage slot
  auto dma_group = [&](int g) {
    const uint32_t slot =
        lds_base + (uint32_t)(((g >> 1) & (F4_NSLOT - 1)) * F4_SLOT + (g & 1) * F4_GRP);
    dma16_f4(xrun + g * xstride, voff_c, slot + wave * 1024);
    dma16_f4(wrun + g * wstride, voff_c, slot + F4_SL_BCODES + wave * 1024);
    const uint8_t* sb = s_w ? wsrun + g * wsstride : xsrun + g * xsstride;
    dma4_f4(sb, voff_s, slot + F4_SL_XSCALES + sch * 256);
  };
  auto dma = [&](int st) {  // one stage = groups 2 st, 2 st + 1
    dma_group(2 * st);
    dma_group(2 * st + 1);
  };
  auto wait_dma = [&](auto og_tag) {
    constexpr int OG = decltype(og_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70 | (6 * OG));  // vmcnt(6 OG): 6 DMAs per stage
  };

  // ---- fragments: lane-linear reads within a slot
  const int fa = (wm * 2) * F4_CODE_BLOCK + lane * 16;
  const int fsa = F4_SL_XSCALES + (wm * 2) * F4_SCALE_BLOCK + lane;
  const int fb = F4_SL_BCODES + (wn * 4) * F4_CODE_BLOCK + lane * 16;
  const int fsb = F4_SL_WSCALES + (wn * 4) * F4_SCALE_BLOCK + lane;
  struct Frags {
    v8i a[2], b[4];
    int sa[2], sb[4];
  };
  auto load_frags = [&](Frags& f, int g) {
    const uint8_t* sp = lds + ((g >> 1) & (F4_NSLOT - 1)) * F4_SLOT + (g & 1) * F4_GRP;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const v4u x = *reinterpret_cast<const v4u*>(sp + fa + tr * F4_CODE_BLOCK);
      f.a[tr] = v8i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
      f.sa[tr] = sp[fsa + tr * F4_SCALE_BLOCK];
    }
#pragma unroll
    for (int tc = 0; tc < 4; ++tc) {
      const v4u x = *reinterpret_cast<const v4u*>(sp + fb + tc * F4_CODE_BLOCK);
      f.b[tc] = v8i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
      f.sb[tc] = sp[fsb + tc * F4_SCALE_BLOCK];
    }
  };

  v16f acc[2][4];
  const int64_t mbase = m0 + wm * 64;
  const int nbase = n0 + wn * 128;

  // ---- prologue: stages 0..2 in flight; the accumulators start from the
  // bias and the low-rank term T L2 (their loads are issued after the DMAs,
  // so waiting for them also waits for the DMAs: vmcnt counts in order).
  const int S = G >> 1;  // stages (G is even)
  dma(0);
  if (S > 1) dma(1);
  if (S > 2) dma(2);
  init_bias_tiles<2, 4>(acc, N, nbase, lane, bias);
  if (T != nullptr) lowrank_up_tiles<2, 4, false>(acc, rank, M, N, mbase, nbase, lane, T, lora_up);
  wait_dma(std::integral_constant<int, 0>{});
  asm volatile("s_barrier" ::: "memory");
  Frags f0, f1;
  load_frags(f0, 0);

  // One group g (of stage st = g / 2): prepare the next group's fragments,
  // then the 8 MFMAs.  KIND -1: the next group is in the same slot (even g);
  // for odd g the next group starts stage st+1, whose DMA must have landed
  // (own wait + barrier): KIND 0 also issues the DMA of stage st+3; 1: stage
  // st+2 is the last (nothing to issue); 2: st+1 is the last (nothing in
  // flight); 3: the last group of all.
  auto group = [&](int g, Frags& cur, Frags& nxt, auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    if constexpr (KIND >= 0 && KIND <= 2) {
      if constexpr (KIND <= 1) wait_dma(std::integral_constant<int, 1>{});
      if constexpr (KIND == 2) wait_dma(std::integral_constant<int, 0>{});
      asm volatile("s_barrier" ::: "memory");
      if constexpr (KIND == 0) dma((g >> 1) + 3);
    }
    if constexpr (KIND != 3) load_frags(nxt, g + 1);
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before the MFMAs
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int tc = 0; tc < 4; ++tc)
        acc[tr][tc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            cur.a[tr], cur.b[tc], acc[tr][tc], FP4_FMT, FP4_FMT, 0, cur.sa[tr], 0, cur.sb[tc]);
    __builtin_amdgcn_sched_barrier(0);
  };
  using KE = std::integral_constant<int, -1>;
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;

  // f0 holds the first group of every stage.  The tail is kinds 1 (if at
  // least 3 stages), 2 (if at least 2) and 3.
  int st = 0;
  for (; st + 3 < S; ++st) {
    group(2 * st, f0, f1, KE{});
    group(2 * st + 1, f1, f0, K0{});
  }
  if (S - st == 3) {
    group(2 * st, f0, f1, KE{});
    group(2 * st + 1, f1, f0, K1{});
    ++st;
  }
  if (S - st == 2) {
    group(2 * st, f0, f1, KE{});
    group(2 * st + 1, f1, f0, K2{});
    ++st;
  }
  group(2 * st, f0, f1, KE{});
  group(2 * st + 1, f1, f0, K3{});

  store_tiles<2, 4, false>(acc, M, N, mbase, nbase, lane, nullptr, out_f32 != 0, Y);
}

// Stand-alone up-projection for the unfused schedule: 128 x 128 output
// tiles, four waves of 2 x 2 MFMA tiles.
constexpr int LU_BM = 128;
constexpr int LU_BN = 128;
constexpr int LU_THREADS = 256;

// Stand-alone up-projection for the unfused schedule: Y += T L2.
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

hipError_t launch_fp4_forward(int rank, bool out_f32, int64_t M, int N, int K,
                              const uint8_t* xcodes, const uint8_t* xscales, const float* T,
                              const void* wimage, const uint16_t* lora_up, const uint16_t* bias,
                              void* Y, void* workspace, hipStream_t s) {
  const int64_t Mp = f4_pad(M), Np = f4_pad(N);
  uint8_t* ximg = reinterpret_cast<uint8_t*>(workspace);
  hipError_t e = launch_fp4_image(M, Mp, K, xcodes, xscales, ximg, s);
  if (e != hipSuccess) return e;
  const int64_t tiles = (Mp / F4_BM) * (Np / F4_BN);
  hipLaunchKernelGGL(fp4_gemm_kernel, dim3((unsigned)tiles), dim3(F4_THREADS), 0, s, M, N, K,
                     rank, (int)out_f32, ximg, (int)(Mp / 32),
                     reinterpret_cast<const uint8_t*>(wimage), (int)(Np / 32), T, lora_up, bias,
                     Y);
  return hipGetLastError();
}

hipError_t launch_lowrank_up(int rank, bool out_f32, int64_t M, int N, const float* T,
                             const uint16_t* lora_up, void* Y, hipStream_t s) {
  const int64_t tiles = ((M + LU_BM - 1) / LU_BM) * (N / LU_BN);
  hipLaunchKernelGGL(lowrank_up_kernel, dim3((unsigned)tiles), dim3(LU_THREADS), 0, s, M, N,
                     rank, (int)out_f32, T, lora_up, Y);
  return hipGetLastError();
}

}  // namespace svdq
