// INT4-mode W4A4 GEMM of the SVDQuant linear on gfx950.
//
//   Y0[m][n] = sum_g sx[m][g] sw[n][g] P_g[m][n],   P_g = sum_{k in g} qx qw
//
// Per 32x32 output tile and 64-element group g:
//   * P_g is one v_mfma_scale_f32_32x32x64_f8f6f4 on FP8 operands: each int4
//     code q is stored as the e4m3 byte whose value is q * 2^-9 (the e4m3
//     subnormal range is linear, so the byte is the sign-magnitude form of q)
//     and both block scales are 2^9, so the fp32 result is the exact integer
//     group sum;
//   * S_g = sx[m][g] sw[n][g] is one v_mfma_f32_32x32x8_bf16 used as an outer
//     product of the bf16-split scales: K slots 0..3 (lanes 0..31) carry
//     hi*hi, lo*hi, hi*lo and slot 4 (lanes 32..63) lo*lo, so S_g is the
//     exact product of the split scales, within 2^-16 of sx*sw;
//   * acc += P_g * S_g is the one VALU FMA per output and group.
// The per-group rescale is inherent to two-sided per-group fp32 scales; with
// P_g and S_g on the matrix cores it is a single FMA, which co-issues with
// the MFMAs of the next tile.
//
// The prep kernel converts the activation codes to e4m3 bytes once per call
// and lays both scale matrices out as group-major MFMA operands (workspace);
// the packed weight codes are converted to e4m3 inside the GEMM, LDS to LDS,
// once per 256 rows of X.
//
// Pipeline: a 512-thread workgroup computes 256 x 128 outputs; each of its 8
// waves owns 64 x 64 (2 x 2 MFMA tiles).  One stage = one 64-element group.
// LDS holds a ring of 4 stage slots.  At stage t every wave
//   1. issues the global->LDS DMA (global_load_lds_dwordx4, no registers) of
//      stage t+4's A tile, scale operands and packed B tile into slot t%4,
//   2. reads stage t+1's MFMA fragments from LDS into registers,
//   3. computes stage t from the fragments read during stage t-1,
//   4. converts stage t+2's packed B tile to e4m3 (LDS to LDS),
//   5. waits for its own DMA of stage t+3, then joins the barrier.
// So the DMA has three stages to land and the fragment reads one stage.
// LDS rows are unpadded 64-byte rows whose four 16-byte chunks are XOR-
// swizzled by the row index, so the contiguous DMA writes and the fragment
// reads (32 lanes on 32 consecutive rows) are bank-conflict free.
// Workgroups are renumbered so that each XCD (own L2) walks a band of
// 256-row tiles of X across all weight columns, two tile rows at a time.
#include <algorithm>

#include "gemm_common.h"
#include "kernels.h"

namespace svdq {

constexpr int I4_BM = 256;
constexpr int I4_BN = 128;
constexpr int I4_THREADS = 512;
constexpr int I4_SCALE_BYTE = 127 + 9;
constexpr int I4_GROUP_M = 2;  // tile rows walked together (L2 reuse of weight tiles)
constexpr int I4_NSLOT = 4;

// one LDS stage slot
constexpr int SL_A = 0;                          // 256 rows x 64 B e4m3 (swizzled)
constexpr int SL_B = SL_A + I4_BM * 64;          // 128 rows x 64 B e4m3 (swizzled)
constexpr int SL_BP = SL_B + I4_BN * 64;         // 128 rows x 32 B packed codes
constexpr int SL_S = SL_BP + I4_BN * 32;         // 2 halves x 384 rows x 8 B scale operands
constexpr int SL_SH = (I4_BM + I4_BN) * 8;       // bytes of one half
constexpr int SL_BYTES = SL_S + 2 * SL_SH;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Rows of the X scale operands are padded to a multiple of 256 (zero rows)
// so that the 16-byte DMA of two 8-byte rows never leaves the array.
__host__ __device__ static inline int64_t pad_rows(int64_t M) { return (M + 255) & ~int64_t(255); }

// Workspace: e4m3 activation codes [M][K], then the scale operands as four
// group-major arrays of 8-byte entries: X half 0, X half 1 ([G][Mp]) and
// W half 0, W half 1 ([G][N]).
size_t int4_workspace_bytes(int64_t M, int N, int K) {
  const int64_t G = K / 64;
  return align256((size_t)M * K) + 2 * align256((size_t)G * pad_rows(M) * 8) +
         2 * align256((size_t)G * N * 8);
}

// Global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane i
// writes LDS bytes [lds_addr + 16 i, +16).  Written as a small asm block (it
// has no register outputs) so that the compiler neither drains it at
// barriers nor serialises consecutive DMAs; the kernel waits for it with
// explicit s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

// Workgroup barrier ordering LDS accesses only (waits for this wave's LDS
// instructions, not for its outstanding DMA).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte chunk swizzle of a 64-byte LDS row: measured conflict-free for
// 32 lanes reading 32 consecutive rows (and the same for rows r and r+32).
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// ---------------------------------------------------------------- prep
// blockIdx.y == 0: activation codes -> e4m3 bytes, one thread per 32 codes.
// blockIdx.y == 1 / 2: 64 x 64 tiles of the X / W scale matrices transposed
// through LDS into group-major 8-byte MFMA operands (two halves):
//   X: half 0 = {hi | lo << 16, hi}, half 1 = {lo, 0}
//   W: half 0 = {hi | hi << 16, lo}, half 1 = {lo, 0}
// Lanes 0..31 of the outer-product MFMA read half 0 (K slots 0..3), lanes
// 32..63 half 1 (slots 4..7).  X rows M .. Mp-1 are written as zeros.
__global__ __launch_bounds__(256) void int4_prep_kernel(
    int64_t M, int N, int K, const uint8_t* __restrict__ xcodes, const float* __restrict__ xscales,
    const float* __restrict__ wscales, uint8_t* __restrict__ xf8, v2u* __restrict__ sx0,
    v2u* __restrict__ sx1, v2u* __restrict__ sw0, v2u* __restrict__ sw1) {
  __shared__ float buf[64][65];
  const int G = K >> 6;
  if (blockIdx.y == 0) {
    const uint32_t chunks = (uint32_t)(K >> 5);
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
    if ((int64_t)idx >= M * chunks) return;
    const uint32_t m = idx / chunks;
    const uint32_t c = idx - m * chunks;
    const v4u w = *reinterpret_cast<const v4u*>(xcodes + (int64_t)m * (K >> 1) + c * 16);
    v4u lo, hi;
    int4x32_to_fp8x32(w, lo, hi);
    uint8_t* dst = xf8 + (int64_t)m * K + c * 32;
    *reinterpret_cast<v4u*>(dst) = lo;
    *reinterpret_cast<v4u*>(dst + 16) = hi;
    return;
  }
  const bool xside = blockIdx.y == 1;
  const int64_t R = xside ? M : N;                 // rows with data
  const int64_t RP = xside ? pad_rows(M) : N;      // rows in the arrays
  const float* __restrict__ src = xside ? xscales : wscales;
  v2u* __restrict__ d0 = xside ? sx0 : sw0;
  v2u* __restrict__ d1 = xside ? sx1 : sw1;
  const uint32_t gt = (uint32_t)((G + 63) >> 6);
  const uint32_t tile = blockIdx.x;
  const int64_t r0 = (int64_t)(tile / gt) * 64;
  const int g0 = (int)(tile % gt) * 64;
  if (r0 >= RP) return;  // uniform per block: no thread reaches the barrier
  for (int i = 0; i < 16; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int rr = idx >> 6, gg = idx & 63;
    float v = 0.f;
    if (r0 + rr < R && g0 + gg < G) v = src[(r0 + rr) * G + g0 + gg];
    buf[rr][gg] = v;
  }
  __syncthreads();
  for (int i = 0; i < 16; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int gg = idx >> 6, rr = idx & 63;
    const int g = g0 + gg;
    if (r0 + rr < RP && g < G) {
      const float sv = buf[rr][gg];
      const uint32_t hb = f32_to_bf16(sv);
      const uint32_t lb = f32_to_bf16(sv - bf16_to_f32(hb));
      const int64_t o = (int64_t)g * RP + r0 + rr;
      d0[o] = xside ? v2u{hb | (lb << 16), hb} : v2u{hb | (hb << 16), lb};
      d1[o] = v2u{lb, 0u};
    }
  }
}

// ---------------------------------------------------------------- GEMM
struct I4Frags {
  v8i af[2], bf[2];
  v4s sa[2], sb[2];
};

__global__ __launch_bounds__(I4_THREADS) void int4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ xf8,
    const v2u* __restrict__ sx0, const v2u* __restrict__ sx1, const uint8_t* __restrict__ wcodes,
    const v2u* __restrict__ sw0, const v2u* __restrict__ sw1, const float* __restrict__ T,
    const uint16_t* __restrict__ lora_up, const uint16_t* __restrict__ bias,
    void* __restrict__ Y) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[I4_NSLOT * SL_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // tile order: XCD-contiguous ranges, grouped by I4_GROUP_M tile rows
  const int num_m = (int)((M + I4_BM - 1) / I4_BM);
  const int num_n = N / I4_BN;
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
  const int64_t KB = K >> 1;

  // ---- DMA plan (per wave and stage): A wave-loads w and w+8 (16 rows of
  // 64 B each), then waves 0..5 one 64-row slice of the scale operands and
  // waves 6..7 two 32-row slices of the packed B tile.  Rows past M are
  // clamped to M-1 (their outputs are never stored).
  int64_t a_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave + 8 * i;
    const int r = 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ swz(r);
    a_off[i] = min(m0 + r, M - 1) * K + 16 * c;
  }
  // scale operands: waves 0..5 each move 128 rows (two per lane) of one
  // half array: X h0 rows 0-127, 128-255, X h1 rows 0-127, 128-255, W h0, W h1
  const bool s_wave = wave < 6;
  const v2u* s_base;
  int64_t s_stride;  // in 8-byte entries per group
  int s_lds;
  {
    const int w6 = s_wave ? wave : 0;
    const int half = (w6 < 4) ? (w6 >> 1) : (w6 - 4);
    const int r = (w6 < 4 ? 128 * (w6 & 1) : I4_BM) + 2 * lane;  // first of two rows
    if (w6 < 4) {
      s_base = (half ? sx1 : sx0) + m0 + r - 0;   // rows < pad_rows(M): always in the array
      s_stride = pad_rows(M);
    } else {
      s_base = (half ? sw1 : sw0) + n0 + (r - I4_BM);
      s_stride = N;
    }
    s_lds = SL_S + SL_SH * half + 8 * (r - 2 * lane);
  }
  int64_t bp_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = 2 * (wave & 1) + i;  // waves 6,7 -> slices 0,1 / 2,3
    const int r = 32 * j + (lane >> 1);
    bp_off[i] = (int64_t)(n0 + r) * KB + 16 * (lane & 1);
  }

  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  auto dma = [&](int t) {
    const uint32_t slot = lds_base + (uint32_t)((t & (I4_NSLOT - 1)) * SL_BYTES);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(xf8 + a_off[i] + t * 64, slot + SL_A + 1024 * (wave + 8 * i));
    if (s_wave) {
      dma16(s_base + (int64_t)t * s_stride, slot + s_lds);  // lane i -> rows r, r+1
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(wcodes + bp_off[i] + t * 32, slot + SL_BP + 1024 * (2 * (wave & 1) + i));
    }
  };
  // wait until this wave's DMA of every stage but the newest has landed:
  // vmcnt <= ops of one stage (3 for waves 0..5, 4 for waves 6..7)
  auto wait_dma_all_but_newest = [&]() {
    if (s_wave)
      __builtin_amdgcn_s_waitcnt(0x0F73);  // vmcnt(3), expcnt(7), lgkmcnt(15)
    else
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
  };

  // ---- B conversion: thread -> row tid/4, 16-byte chunk tid%4
  const int cb_row = tid >> 2, cb_q = tid & 3;
  const int cb_src = SL_BP + cb_row * 32 + 8 * cb_q;
  const int cb_dst = SL_B + cb_row * 64 + 16 * (cb_q ^ swz(cb_row));
  auto convert_b = [&](int t) {
    uint8_t* slot = lds + (t & (I4_NSLOT - 1)) * SL_BYTES;
    const v2u w = *reinterpret_cast<const v2u*>(slot + cb_src);
    *reinterpret_cast<v4u*>(slot + cb_dst) = int4x16_to_fp8x16(w[0], w[1]);
  };

  // ---- fragment addresses within a slot.  Rows r and r+32 have the same
  // chunk swizzle, so tile row / column 1 is tile 0 plus a constant offset.
  const int ra0 = wm * 64 + l32, rb0 = wn * 64 + l32;
  const int fa0 = SL_A + ra0 * 64 + 16 * ((2 * h) ^ swz(ra0));
  const int fa1 = SL_A + ra0 * 64 + 16 * ((2 * h + 1) ^ swz(ra0));
  const int fb0 = SL_B + rb0 * 64 + 16 * ((2 * h) ^ swz(rb0));
  const int fb1 = SL_B + rb0 * 64 + 16 * ((2 * h + 1) ^ swz(rb0));
  const int fsa = SL_S + SL_SH * h + ra0 * 8;
  const int fsb = SL_S + SL_SH * h + (I4_BM + rb0) * 8;
  auto load_frags = [&](I4Frags& f, int t) {
    const uint8_t* slot = lds + (t & (I4_NSLOT - 1)) * SL_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const v4u a0 = *reinterpret_cast<const v4u*>(slot + fa0 + 2048 * i);
      const v4u a1 = *reinterpret_cast<const v4u*>(slot + fa1 + 2048 * i);
      f.af[i] = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                    (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      const v4u b0 = *reinterpret_cast<const v4u*>(slot + fb0 + 2048 * i);
      const v4u b1 = *reinterpret_cast<const v4u*>(slot + fb1 + 2048 * i);
      f.bf[i] = v8i{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                    (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
      f.sa[i] = *reinterpret_cast<const v4s*>(slot + fsa + 256 * i);
      f.sb[i] = *reinterpret_cast<const v4s*>(slot + fsb + 256 * i);
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  const v16f zero = acc[0][0];

  auto compute = [&](const I4Frags& f) {
    // software pipeline over the 4 tiles: the MFMAs of tile t+1 are issued
    // before the FMAs of tile t consume its P and S.
    v16f p[2], sc[2];
    p[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.af[0], f.bf[0], zero, 0, 0, 0,
                                                           I4_SCALE_BYTE, 0, I4_SCALE_BYTE);
    sc[0] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(f.sa[0], f.sb[0], zero, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      if (t + 1 < 4) {
        const int tr = (t + 1) >> 1, tc = (t + 1) & 1;
        p[nxt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.af[tr], f.bf[tc], zero, 0, 0, 0,
                                                                 I4_SCALE_BYTE, 0, I4_SCALE_BYTE);
        sc[nxt] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(f.sa[tr], f.sb[tc], zero, 0, 0, 0);
      }
      const int tr = t >> 1, tc = t & 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tr][tc][i] = fmaf(p[cur][i], sc[cur][i], acc[tr][tc][i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: stages 0..3 in flight; convert B of stages 0, 1
  for (int t = 0; t < I4_NSLOT; ++t)
    if (t < G) dma(t);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  lds_barrier();
  convert_b(0);
  if (G > 1) convert_b(1);
  lds_barrier();
  I4Frags f0, f1;
  load_frags(f0, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): slot 0 is read before it is refilled

  // ---- main loop, unrolled by two so the fragment sets are static
  auto step = [&](int t, I4Frags& cur, I4Frags& nxt) {
    if (t + 4 < G) dma(t + 4);
    if (t + 1 < G) load_frags(nxt, t + 1);
    compute(cur);
    if (t + 2 < G) convert_b(t + 2);
    if (t + 4 < G)
      wait_dma_all_but_newest();
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tail, nothing newer in flight
    lds_barrier();
  };
  for (int t = 0; t < G; t += 2) {
    step(t, f0, f1);
    if (t + 1 < G) step(t + 1, f1, f0);
  }

  const int64_t mbase = m0 + wm * 64;
  const int nbase = n0 + wn * 64;
  if (T != nullptr) lowrank_up_tiles<2, 2>(acc, rank, M, mbase, nbase, lane, T, lora_up);
  store_tiles<2, 2>(acc, M, N, mbase, nbase, lane, bias, out_f32 != 0, Y, false);
}

hipError_t launch_int4_forward(int rank, bool out_f32, int64_t M, int N, int K,
                               const uint8_t* xcodes, const float* xscales, const float* T,
                               const uint8_t* wcodes, const float* wscales,
                               const uint16_t* lora_up, const uint16_t* bias, void* Y,
                               void* workspace, hipStream_t s) {
  const int64_t G = K / 64;
  const int64_t Mp = pad_rows(M);
  uint8_t* p = reinterpret_cast<uint8_t*>(workspace);
  uint8_t* xf8 = p;
  p += align256((size_t)M * K);
  v2u* sx0 = reinterpret_cast<v2u*>(p);
  p += align256((size_t)G * Mp * 8);
  v2u* sx1 = reinterpret_cast<v2u*>(p);
  p += align256((size_t)G * Mp * 8);
  v2u* sw0 = reinterpret_cast<v2u*>(p);
  p += align256((size_t)G * N * 8);
  v2u* sw1 = reinterpret_cast<v2u*>(p);
  const int64_t gt = (G + 63) / 64;
  const int64_t n_code = (M * (K / 32) + 255) / 256;
  const int64_t n_sx = (Mp / 64) * gt;
  const int64_t n_sw = ((N + 63) / 64) * gt;
  const int64_t gx = std::max(n_code, std::max(n_sx, n_sw));
  hipLaunchKernelGGL(int4_prep_kernel, dim3((unsigned)gx, 3), dim3(256), 0, s, M, N, K, xcodes,
                     xscales, wscales, xf8, sx0, sx1, sw0, sw1);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + I4_BM - 1) / I4_BM) * (N / I4_BN);
  hipLaunchKernelGGL(int4_gemm_kernel, dim3((unsigned)tiles), dim3(I4_THREADS), 0, s, M, N, K,
                     rank, (int)out_f32, xf8, sx0, sx1, wcodes, sw0, sw1, T, lora_up, bias, Y);
  return hipGetLastError();
}

}  // namespace svdq
