// INT4-mode W4A4 GEMM of the SVDQuant linear on gfx950.
//
//   Y0[m][n] = sum_g sx[m][g] sw[n][g] P_g[m][n],   P_g = sum_{k in g} qx qw
//
// Per 32x32 output tile and 64-element group g:
//   * P_g is one v_mfma_scale_f32_32x32x64_f8f6f4 on FP6 (E2M3) operands.  In
//     E2M3 the five magnitude bits of the codes 0..15 are the value times 8
//     (the subnormal and first normal binade are one linear range), so an
//     int4 code q is stored as the 6-bit sign-magnitude field of q, whose
//     value is q/8; with both block scales 2^3 the fp32 result is the exact
//     integer group sum.  FP6 runs at twice the FP8 rate on gfx950.
//   * S_g = sx[m][g] sw[n][g] is one v_mfma_f32_32x32x8_bf16 used as an outer
//     product of the bf16-split scales: K slots 0..3 (lanes 0..31) carry
//     hi*hi, lo*hi, hi*lo and slot 4 (lanes 32..63) lo*lo, so S_g is the
//     exact product of the split scales, within 2^-16 of sx*sw.
//   * acc += P_g * S_g is the one VALU FMA per output and group, inherent to
//     two-sided per-group fp32 scales.
//
// Operand images.  Both operands reach the kernel as a group-major "image"
// of 2048-byte blocks, one per (group g, 32-row tile), laid out exactly as
// the MFMA lanes read them:
//   [0, 768)     K half 0 (elements 0..31 of the group): 32 rows x 24 bytes,
//                the first 16 bytes of each row at 16*row, the last 8 at
//                512 + 8*row (so b128 and b64 reads are lane-linear);
//   [768, 1536)  K half 1, same layout;
//   [1536, 2048) the 8-byte bf16 scale operand of each of the 64 lanes.
// A row's 32 fields of 6 bits are packed little-endian (field j at bit 6j).
// The activation image is built per call by the prep kernel (workspace);
// the weight image is built once by svdq_prepare_weight.  A workgroup's
// stage is then two contiguous runs of the images (16 KB of X, 12 KB of W)
// that the global->LDS DMA copies verbatim.
//
// Pipeline: a 512-thread workgroup computes 256 x 192 outputs; each of its 8
// waves (two per SIMD) owns 64 x 96 (2 x 3 tiles).  One stage = one group;
// LDS holds a ring of 4 stage slots.  Within a group the MFMAs of tile t+1
// are issued before the FMAs of tile t, and every fragment register is
// reloaded for the next group right after its last MFMA has been issued, so
// no wave waits for LDS at a group boundary.  Once per group every wave
// waits for its own DMA of the next group, joins the barrier, and issues the
// DMA of the group three ahead.
// Workgroups are renumbered so that each XCD (own L2) walks a band of
// I4_GROUP_M row tiles of X across all weight columns.
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"
#include "kernels.h"

namespace svdq {

constexpr int I4_BM = 256;
constexpr int I4_BN = 192;
constexpr int I4_THREADS = 512;
constexpr int I4_SCALE_BYTE = 127 + 3;  // E2M3 field q has value q/8
constexpr int I4_GROUP_M = 2;           // tile rows walked together per XCD
constexpr int I4_NSLOT = 4;  // stage slots: DMA runs two groups ahead
constexpr int IMG_BLOCK = 2048;                                // bytes per (group, 32 rows)
constexpr int SLOT_A = (I4_BM / 32) * IMG_BLOCK;               // 16 KB of X
constexpr int SLOT_BYTES = SLOT_A + (I4_BN / 32) * IMG_BLOCK;  // + 12 KB of W
constexpr int FP6_FMT = 2;                                     // f8f6f4 format code of E2M3

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Rows of the activation image are padded to the workgroup's 256 rows and
// columns of the weight image to its 192 columns (zero codes and scales).
static inline int64_t pad_rows(int64_t M) { return (M + I4_BM - 1) / I4_BM * I4_BM; }
static inline int64_t pad_cols(int64_t N) { return (N + I4_BN - 1) / I4_BN * I4_BN; }
static inline size_t image_bytes(int64_t rows_padded, int K) {
  return (size_t)(K / 64) * (size_t)(rows_padded / 32) * IMG_BLOCK;
}

size_t int4_workspace_bytes(int64_t M, int K) { return align256(image_bytes(pad_rows(M), K)); }

size_t int4_weight_image_bytes(int N, int K) { return image_bytes(pad_cols(N), K); }

// Global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4 with a
// scalar base): lane i reads sbase + voff and writes LDS bytes
// [lds_addr + 16 i, +16).  Written as a small asm block (it has no register
// outputs) so that the compiler neither drains it at barriers nor serialises
// consecutive DMAs; the kernel waits for it with explicit s_waitcnt vmcnt.
// The base is wave-uniform by construction; readfirstlane makes that explicit
// so that it is kept in scalar registers.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  // (readfirstlane returns a signed int: zero-extend each half explicitly)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// ---------------------------------------------------------------- images
// 32 two's-complement int4 codes (16 bytes, element 2j in the low nibble of
// byte j) -> 32 E2M3 sign-magnitude fields of 6 bits (value q/8) packed into
// six dwords.  For a nibble x the field is x when x < 8 and 0x20 | (16 - x)
// = 0x30 - x otherwise.
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

// One wave per (group, 32-row tile) block of an operand image.  Rows R .. RP-1
// are zero.  XSIDE selects the scale-operand pattern:
//   X: lanes 0..31 {hi | lo << 16, hi}, lanes 32..63 {lo, 0}
//   W: lanes 0..31 {hi | hi << 16, lo}, lanes 32..63 {lo, 0}
// so that K slots 0..3 of the outer-product MFMA hold hi*hi, lo*hi, hi*lo, 0
// and slot 4 lo*lo.
template <bool XSIDE>
__global__ __launch_bounds__(256) void int4_image_kernel(int64_t R, int64_t RP, int K,
                                                         const uint8_t* __restrict__ codes,
                                                         const float* __restrict__ scales,
                                                         uint8_t* __restrict__ image) {
  const int G = K >> 6;
  const int64_t RT = RP >> 5;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= (int64_t)G * RT) return;
  const int g = (int)(blk / RT);
  const int64_t r = (blk - (int64_t)g * RT) * 32 + (threadIdx.x & 31);
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  uint8_t* out = image + blk * IMG_BLOCK;
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
  v2u so;
  if (h == 0)
    so = XSIDE ? v2u{hb | (lb << 16), hb} : v2u{hb | (hb << 16), lb};
  else
    so = v2u{lb, 0u};
  *reinterpret_cast<v2u*>(out + 1536 + lane * 8) = so;
}

static hipError_t launch_image(bool xside, int64_t R, int64_t RP, int K, const uint8_t* codes,
                               const float* scales, uint8_t* image, hipStream_t s) {
  const int64_t blocks = ((int64_t)(K / 64) * (RP / 32) + 3) / 4;
  if (xside)
    hipLaunchKernelGGL(int4_image_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, R, RP,
                       K, codes, scales, image);
  else
    hipLaunchKernelGGL(int4_image_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, R,
                       RP, K, codes, scales, image);
  return hipGetLastError();
}

hipError_t launch_int4_prepare_weight(int N, int K, const uint8_t* wcodes, const float* wscales,
                                      void* wimage, hipStream_t s) {
  return launch_image(false, N, pad_cols(N), K, wcodes, wscales,
                      reinterpret_cast<uint8_t*>(wimage), s);
}

// ---------------------------------------------------------------- GEMM
__global__ __launch_bounds__(I4_THREADS) void int4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ ximg,
    int x_tiles, const uint8_t* __restrict__ wimg, int w_tiles, const float* __restrict__ T,
    const uint16_t* __restrict__ lora_up, const uint16_t* __restrict__ bias,
    void* __restrict__ Y) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[I4_NSLOT * SLOT_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // tile order: XCD-contiguous ranges, grouped by I4_GROUP_M tile rows
  const int num_m = x_tiles / (I4_BM / 32);
  const int num_n = w_tiles / (I4_BN / 32);
  const int nb = gridDim.x;
  int L = blockIdx.x;
  if ((nb & 7) == 0) L = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int band = L / (I4_GROUP_M * num_n);
  const int first_m = band * I4_GROUP_M;
  const int gm = min(num_m - first_m, I4_GROUP_M);
  const int in_band = L - band * I4_GROUP_M * num_n;
  const int tile_m = first_m + in_band % gm;
  const int tile_n = in_band / gm;
  const int64_t m0 = (int64_t)tile_m * I4_BM;
  const int n0 = tile_n * I4_BN;
  const int G = K >> 6;

  // ---- DMA plan: a stage is 28 chunks of 1 KB (16 of X, then 12 of W) that
  // land at slot + 1 KB * chunk.  Wave w moves chunks w, w+8 (X) and w+16
  // (W); waves 0..3 also w+24 (W), while waves 4..7 repeat their chunk w+16
  // (the same bytes to the same place).  Every wave thus has four DMAs per
  // group and waits with the same counts, with no branch in the loop.
  const uint8_t* xrun = ximg + (int64_t)tile_m * (I4_BM / 32) * IMG_BLOCK;
  const uint8_t* wrun = wimg + (int64_t)tile_n * (I4_BN / 32) * IMG_BLOCK;
  const int64_t xstride = (int64_t)x_tiles * IMG_BLOCK;  // bytes per group
  const int64_t wstride = (int64_t)w_tiles * IMG_BLOCK;
  const uint32_t voff0 = (uint32_t)(wave * 1024 + lane * 16);
  const uint32_t voff1 = voff0 + 8 * 1024;
  const int wave4 = wave < 4 ? wave + 24 : wave + 16;  // LDS chunk of the 4th DMA
  const uint32_t voff3 = (uint32_t)((wave4 - 16) * 1024 + lane * 16);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  auto slot_of = [](int g) { return (g & (I4_NSLOT - 1)) * SLOT_BYTES; };
  auto dma = [&](int g) {
    const uint32_t slot = lds_base + (uint32_t)slot_of(g);
    const uint8_t* xs = xrun + g * xstride;
    const uint8_t* ws = wrun + g * wstride;
    dma16(xs, voff0, slot + wave * 1024);
    dma16(xs, voff1, slot + (wave + 8) * 1024);
    dma16(ws, voff0, slot + (wave + 16) * 1024);
    dma16(ws, voff3, slot + wave4 * 1024);
  };
  // wait until at most OG groups of this wave's DMA are still in flight
  auto wait_dma = [&](auto og_tag) {
    constexpr int OG = decltype(og_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70 | (4 * OG));  // vmcnt(4 OG)
  };
  using OG0 = std::integral_constant<int, 0>;
  using OG1 = std::integral_constant<int, 1>;

  // ---- fragment offsets within a slot (see the image layout above)
  const int fa = (wm * 2) * IMG_BLOCK + h * 768 + l32 * 16;
  const int fa8 = (wm * 2) * IMG_BLOCK + h * 768 + 512 + l32 * 8;
  const int fsa = (wm * 2) * IMG_BLOCK + 1536 + lane * 8;
  const int fb = SLOT_A + (wn * 3) * IMG_BLOCK + h * 768 + l32 * 16;
  const int fb8 = SLOT_A + (wn * 3) * IMG_BLOCK + h * 768 + 512 + l32 * 8;
  const int fsb = SLOT_A + (wn * 3) * IMG_BLOCK + 1536 + lane * 8;

  v8i af[2], bf[3];
  v4s sa[2], sb[3];
  auto load_a = [&](const uint8_t* sp, int tr) {
    const v4u x = *reinterpret_cast<const v4u*>(sp + fa + tr * IMG_BLOCK);
    const v2u y = *reinterpret_cast<const v2u*>(sp + fa8 + tr * IMG_BLOCK);
    af[tr] = v8i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], 0, 0};
    sa[tr] = *reinterpret_cast<const v4s*>(sp + fsa + tr * IMG_BLOCK);
  };
  auto load_b = [&](const uint8_t* sp, int tc) {
    const v4u x = *reinterpret_cast<const v4u*>(sp + fb + tc * IMG_BLOCK);
    const v2u y = *reinterpret_cast<const v2u*>(sp + fb8 + tc * IMG_BLOCK);
    bf[tc] = v8i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], 0, 0};
    sb[tc] = *reinterpret_cast<const v4s*>(sp + fsb + tc * IMG_BLOCK);
  };

  v16f zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero[i] = 0.f;
  v16f acc[2][3];
  v16f p[2], sc[2];

  // tile t of a wave = (t / 3, t % 3); its P and S live in p/sc[t & 1]
  auto mfma_p = [&](int t) {
    const int tr = t / 3, tc = t % 3, b = t & 1;
    p[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[tr], bf[tc], zero, FP6_FMT, FP6_FMT,
                                                           0, I4_SCALE_BYTE, 0, I4_SCALE_BYTE);
  };
  auto mfma_s = [&](int t) {
    const int tr = t / 3, tc = t % 3, b = t & 1;
    sc[b] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sa[tr], sb[tc], zero, 0, 0, 0);
  };
  auto mfma_tile = [&](int t) {
    mfma_p(t);
    mfma_s(t);
  };
  // FMAs i0 .. i0+7 of tile t: acc += P * S
  auto fma_half = [&](int t, int i0) {
    const int tr = t / 3, tc = t % 3, b = t & 1;
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) acc[tr][tc][i] = fmaf(p[b][i], sc[b][i], acc[tr][tc][i]);
  };
  // One step: the MFMAs of tile `next` (if any) interleaved with the FMAs of
  // tile `cur`, in the fixed order P MFMA, 8 FMAs, S MFMA, loads (of the
  // fragments both MFMAs just read for the last time), 8 FMAs, so that each
  // MFMA runs under a block of FMAs.
  auto step = [&](int next, int cur, auto&& loads) {
    if (next >= 0) mfma_p(next);
    __builtin_amdgcn_sched_barrier(0);
    fma_half(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (next >= 0) mfma_s(next);
    loads();
    __builtin_amdgcn_sched_barrier(0);
    fma_half(cur, 8);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One group.  The DMA of group g+3 is issued in group g; at the barrier
  // of group g the DMA of g+1 must have landed.  KIND 0: steady state
  // (group g+2 may still be in flight; issue g+3); 1: g+2 is the last group
  // (nothing to issue); 2: g+1 is the last (nothing in flight); 3: the last
  // group (no next group to prepare).  Every kind is straight-line code and
  // the sched_barriers fix the order of its steps.  Each fragment is
  // reloaded for the next group in the step that issues its last MFMA.
  auto group = [&](int g, auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr bool NEXT = KIND != 3;
    const uint8_t* nsp = lds + slot_of(g + 1);
    step(1, 0, [] {});
    // A tile row 0 is free after tile 2's MFMAs; the next slot must be ready
    step(2, 1, [&] {
      if constexpr (NEXT) {
        if constexpr (KIND <= 1) wait_dma(OG1{});
        if constexpr (KIND == 2) wait_dma(OG0{});
        asm volatile("s_barrier" ::: "memory");
        if constexpr (KIND == 0) dma(g + 3);
        load_a(nsp, 0);
      }
    });
    step(3, 2, [&] {  // B column 0 free
      if constexpr (NEXT) load_b(nsp, 0);
    });
    step(4, 3, [&] {  // B column 1 free
      if constexpr (NEXT) load_b(nsp, 1);
    });
    step(5, 4, [&] {  // A row 1 and B column 2 free
      if constexpr (NEXT) {
        load_a(nsp, 1);
        load_b(nsp, 2);
      }
    });
    step(NEXT ? 0 : -1, 5, [] {});  // first tile of the next group
  };

  // ---- prologue: the first groups in flight.  Meanwhile the accumulators start
  // from the bias and the low-rank term T L2 (its loads overlap the DMA
  // latency), so nothing but the store is left after the main loop.  G is
  // even (K % 128 == 0), so G >= 2.
  const int64_t mbase = m0 + wm * 64;
  const int nbase = n0 + wn * 96;
  // The loads of T and L2 are issued after the DMAs, so waiting for them
  // also waits for these DMAs (vmcnt counts in order).
  dma(0);
  dma(1);
  if (G > 2) dma(2);
  init_bias_tiles<2, 3>(acc, N, nbase, lane, bias);
  if (T != nullptr) lowrank_up_tiles<2, 3>(acc, rank, M, N, mbase, nbase, lane, T, lora_up);
  wait_dma(OG0{});
  asm volatile("s_barrier" ::: "memory");
  load_a(lds, 0);
  load_a(lds, 1);
  load_b(lds, 0);
  load_b(lds, 1);
  load_b(lds, 2);
  mfma_tile(0);

  // G is even: either G >= 4 (the tail is kinds 1..3) or G == 2 (2, 3)
  int g = 0;
  for (; g + 3 < G; ++g) group(g, std::integral_constant<int, 0>{});
  if (G >= 4) group(g++, std::integral_constant<int, 1>{});
  group(g++, std::integral_constant<int, 2>{});
  group(g, std::integral_constant<int, 3>{});

  store_tiles<2, 3, false>(acc, M, N, mbase, nbase, lane, nullptr, out_f32 != 0, Y);
}

hipError_t launch_int4_forward(int rank, bool out_f32, int64_t M, int N, int K,
                               const uint8_t* xcodes, const float* xscales, const float* T,
                               const void* wimage, const uint16_t* lora_up,
                               const uint16_t* bias, void* Y, void* workspace, hipStream_t s) {
  const int64_t Mp = pad_rows(M);
  const int64_t Np = pad_cols(N);
  uint8_t* ximg = reinterpret_cast<uint8_t*>(workspace);
  hipError_t e = launch_image(true, M, Mp, K, xcodes, xscales, ximg, s);
  if (e != hipSuccess) return e;
  const int64_t tiles = (Mp / I4_BM) * (Np / I4_BN);
  hipLaunchKernelGGL(int4_gemm_kernel, dim3((unsigned)tiles), dim3(I4_THREADS), 0, s, M, N, K,
                     rank, (int)out_f32, ximg, (int)(Mp / 32),
                     reinterpret_cast<const uint8_t*>(wimage), (int)(Np / 32), T, lora_up, bias,
                     Y);
  return hipGetLastError();
}

}  // namespace svdq
