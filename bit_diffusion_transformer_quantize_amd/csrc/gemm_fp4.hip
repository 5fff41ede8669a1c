// FP4-mode (MXFP4: E2M1 codes, E8M0 block scales) W4A4 GEMM of the SVDQuant
// linear on gfx950.
//
//   Y = sum_b 2^(ex[m][b] + ew[n][b]) sum_{k in b} fx[m][k] fw[n][k] + T L2 + bias
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
// the whole K accumulation stays in the MFMA: no per-group vector work.  The
// low-rank term is T L2 with T split into bf16 high and low parts (two
// v_mfma_f32_32x32x16_bf16 per 16 ranks, accumulating into acc).
//
// Everything the kernel reads comes from the operand images (image.h)
// through global->LDS DMA.  The kernel is persistent and walks a stream of
// stages over its tiles, as the INT4 kernel does: per tile P pre stages
// (the bias and one 16-rank slice of T and L2 each) and G/2 code stages of
// two 64-groups (X and W codes, 8 KB each per group, and their scale runs).
// Every wave issues exactly four 1 KB DMAs and one 256-byte DMA per stage,
// and the DMA engine runs two stages ahead across tile boundaries.
//
// Compute: a 512-thread workgroup computes 256 x 256 outputs; each of its 8
// waves owns 64 x 128 (2 x 4 tiles).  The weight is the A operand and the
// activations the B operand, so the epilogue stores 16 bytes per lane.  The fragments of the next group are
// read while the 8 MFMAs of the current one run; one barrier per stage.
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"
#include "image.h"
#include "kernels.h"

namespace svdq {

constexpr int F4_BM = 256;
constexpr int F4_BN = 256;
constexpr int F4_THREADS = 512;
constexpr int F4_GROUP_M = 2;
constexpr int F4_NSLOT = 4;
// code stage: two group halves of [X codes 8 KB][W codes 8 KB][X scales 512][W scales 512]
constexpr int F4_XS = 16 * F4_CBLOCK;
constexpr int F4_WS = F4_XS + 8 * F4_SBLOCK;
constexpr int F4_GRP = F4_WS + 8 * F4_SBLOCK;  // 17408 bytes per group
constexpr int F4_SLOT = 2 * F4_GRP;
// pre stage: T hi/lo blocks, L2 blocks, the bias run
constexpr int F4_PRE_L2 = (F4_BM / 32) * LR_XBLOCK;                // 16 KB
constexpr int F4_PRE_BIAS = F4_PRE_L2 + (F4_BN / 32) * LR_WBLOCK;  // 24 KB
static_assert(F4_PRE_BIAS + 1024 <= F4_SLOT, "pre-stage fits a slot");
constexpr int FP4_FMT = 4;  // f8f6f4 format code of E2M1
// vector memory operations of one full output tile's bf16 stores per wave
// (2 per 32x32 tile; the fp32 form issues more, which only waits longer)
constexpr int F4_NST = 2 * 2 * 4;

typedef __attribute__((address_space(3))) void lds_void_f4;

__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Global -> LDS DMA of 16 (dwordx4) or 4 (dword) bytes per lane with a
// scalar base; see the INT4 kernel for why these are asm blocks.
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

struct TileXY4 {
  int tm, tn;
};
__device__ __forceinline__ TileXY4 tile_xy4(int L, int num_m, int num_n) {
  const int band = L / (F4_GROUP_M * num_n);
  const int first_m = band * F4_GROUP_M;
  const int gm = min(num_m - first_m, F4_GROUP_M);
  const int in_band = L - band * F4_GROUP_M * num_n;
  return TileXY4{first_m + in_band % gm, in_band / gm};
}
// k-th tile of workgroup b (XCD-contiguous eighths when both counts allow)
__device__ __forceinline__ int tile_number4(int b, int k, int nwg, int ntiles) {
  if ((nwg & 7) == 0 && (ntiles & 7) == 0) {
    const int per = ntiles >> 3, nw = nwg >> 3;
    return (b & 7) * per + (b >> 3) + k * nw;
  }
  return b + k * nwg;
}
__device__ __forceinline__ int tiles_of4(int b, int nwg, int ntiles) {
  if ((nwg & 7) == 0 && (ntiles & 7) == 0) {
    const int per = ntiles >> 3, nw = nwg >> 3, w = b >> 3;
    return w < per ? (per - w + nw - 1) / nw : 0;
  }
  return b < ntiles ? (ntiles - b + nwg - 1) / nwg : 0;
}

// LR: the layer has a low-rank branch (rank > 0); the two forms are
// separate kernels so that traces tell the rank-0 launches apart.
template <bool LR>
__global__ __launch_bounds__(F4_THREADS) void fp4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ ximg,
    int64_t x_rt, int64_t x_sc, int64_t x_lr, const uint8_t* __restrict__ wimg, int64_t w_ct,
    int64_t w_sc, int64_t w_lr, int64_t w_bias, void* __restrict__ Y) {
  // the ring, then a 256-byte pad that only dummy DMAs write
  __shared__ __attribute__((aligned(1024))) uint8_t lds[F4_NSLOT * F4_SLOT + 256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int num_m = (int)(x_rt / (F4_BM / 32));
  const int num_n = (int)(w_ct / (F4_BN / 32));
  const int ntiles = num_m * num_n;
  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int my_tiles = tiles_of4(b, nwg, ntiles);
  if (my_tiles == 0) return;  // uniform per workgroup: no barrier is reached
  const int S = K >> 7;       // code stages per tile (G/2; K % 128 == 0)
  const int R16 = LR ? rank >> 4 : 0;
  // pre-stages per tile: the bias rides in the first, one 16-rank slice of
  // the low-rank branch in each of the first R16; at least two, so that the
  // first two code stages of a tile are among the positions issued ahead
  // of the previous tile's stores
  const int P = R16 > 2 ? R16 : 2;
  const int SPT = P + S;
  const int total = my_tiles * SPT;

  // ---- DMA, generic form: stage q of the stream (the heads and tails of
  // tiles).  1 KB chunk slots w + 8 i (i = 0..3) land at slot + dst(chunk);
  // one 256-byte piece per wave.
  //   code stage: chunk c -> group half c/16; in the half, 0..7 X codes,
  //     8..15 W codes; piece w -> group half w/4, X (w&2 == 0) or W scales,
  //     bytes 256 (w&1) of the 512-byte run
  //   pre stage: chunks 0..15 T hi/lo, 16..23 L2, 24 the bias run, 25..31
  //     repeat 18..24; the piece repeats the first 256 bytes of the bias run
  //     (a pre stage past the rank: everything is the bias run)
  const uint32_t voff16 = (uint32_t)(lane * 16);
  const uint32_t voff4 = (uint32_t)(lane * 4);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_f4*)lds;
  TileXY4 cur_t = tile_xy4(tile_number4(b, 0, nwg, ntiles), num_m, num_n);
  TileXY4 nxt_t = my_tiles > 1 ? tile_xy4(tile_number4(b, 1, nwg, ntiles), num_m, num_n) : cur_t;
  int cur_base = 0;  // stream position of the current tile's first stage
  auto dma_stage = [&](int q) {
    const int qq = min(q, total - 1);  // past the end: re-read the last stage
    int j = qq - cur_base;
    const bool in_next = j >= SPT;
    j = in_next ? j - SPT : j;
    const int tm = in_next ? nxt_t.tm : cur_t.tm;
    const int tn = in_next ? nxt_t.tn : cur_t.tn;
    const bool pre = j < P;
    const bool lr = pre && j < R16;
    const int g0 = pre ? 0 : 2 * (j - P);  // first group of the code stage
    const int jl = lr ? j : 0;
    const int64_t xrow = (int64_t)tm * (F4_BM / 32), wrow = (int64_t)tn * (F4_BN / 32);
    const uint8_t* tl = ximg + x_lr + ((int64_t)jl * x_rt + xrow) * LR_XBLOCK;
    const uint8_t* ll = wimg + w_lr + ((int64_t)jl * w_ct + wrow) * LR_WBLOCK;
    const uint8_t* bs = wimg + w_bias + wrow * BIAS_BLOCK;
    const uint32_t slot = lds_base + (uint32_t)((q & (F4_NSLOT - 1)) * F4_SLOT);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = wave + 8 * i;
      const int gh = c >> 4, cc = c & 15;
      const int g = g0 + gh;
      const uint8_t* csrc = cc < 8 ? ximg + ((int64_t)g * x_rt + xrow) * F4_CBLOCK + cc * 1024
                                   : wimg + ((int64_t)g * w_ct + wrow) * F4_CBLOCK + (cc - 8) * 1024;
      const int cdst = gh * F4_GRP + cc * 1024;
      const int pc = lr ? (c >= 25 ? c - 7 : c) : 24;
      const uint8_t* psrc = pc < 16 ? tl + pc * 1024 : (pc < 24 ? ll + (pc - 16) * 1024 : bs);
      dma16_f4(pre ? psrc : csrc, voff16, slot + (uint32_t)(pre ? pc * 1024 : cdst));
    }
    {
      const int gh = wave >> 2, side = (wave >> 1) & 1, half = wave & 1;
      const int g = g0 + gh;
      const uint8_t* ssrc = side == 0 ? ximg + x_sc + ((int64_t)g * x_rt + xrow) * F4_SBLOCK
                                      : wimg + w_sc + ((int64_t)g * w_ct + wrow) * F4_SBLOCK;
      const int sdst = gh * F4_GRP + (side == 0 ? F4_XS : F4_WS) + half * 256;
      dma4_f4(pre ? bs : ssrc + half * 256, voff4, slot + (uint32_t)(pre ? F4_PRE_BIAS : sdst));
    }
  };
  // ---- DMA, body form: a code stage of the current tile from running
  // pointers, moving the pieces the generic form gives this wave: X and W
  // chunk w of both groups of the stage and its scale piece.
  const int s_gh = wave >> 2, s_side = (wave >> 1) & 1, s_half = wave & 1;
  const uint32_t dx = (uint32_t)wave * 1024;
  const uint32_t dsc = (uint32_t)(s_gh * F4_GRP + (s_side == 0 ? F4_XS : F4_WS) + s_half * 256);
  const int64_t xg = x_rt * F4_CBLOCK, wg = w_ct * F4_CBLOCK;  // one group further
  const int64_t sg = (s_side == 0 ? x_rt : w_ct) * F4_SBLOCK;
  const uint8_t* xrun = ximg;  // X code chunk w of the target stage's first group
  const uint8_t* wrun = wimg;
  const uint8_t* srun = ximg;  // this wave's scale piece of the target stage
  auto dma_code = [&](int q) {
    const uint32_t slot = lds_base + (uint32_t)((q & (F4_NSLOT - 1)) * F4_SLOT);
    dma16_f4(xrun, voff16, slot + dx);
    dma16_f4(wrun, voff16, slot + dx + 8 * 1024);
    dma16_f4(xrun + xg, voff16, slot + F4_GRP + dx);
    dma16_f4(wrun + wg, voff16, slot + F4_GRP + dx + 8 * 1024);
    dma4_f4(srun, voff4, slot + dsc);
    xrun += 2 * xg;
    wrun += 2 * wg;
    srun += 2 * sg;
  };
  // Waits for this wave's DMA of the stage about to be read, naming how many
  // younger vector memory operations may still be in flight (they complete
  // in issue order): the next stage's five in the body of a tile; at the
  // first four stages (j = 0..3) up to three younger stages plus the
  // F4_NST output stores of the previous tile behind them (before the first
  // tile, F4_NST dummy DMAs into the pad stand in for them).
  // With P == 2 the first code stage (j = 2) waits until only the stores
  // may be outstanding, which covers position 3 too: the next stage's read
  // point then needs no wait.
  auto wait_stage = [] { __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); };
  auto wait_at = [&](int j) {
    if (j == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(15 + F4_NST));
    else if (j == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(10 + F4_NST));
    else if (j == 2 && P == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(F4_NST));
    else if (j < 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 + F4_NST));
    else wait_stage();
  };
  auto barrier = [] { asm volatile("s_barrier" ::: "memory"); };

  // ---- code fragments of a group half
  const int fa = (wm * 2) * F4_CBLOCK + lane * 16;
  const int fsa = F4_XS + (wm * 2) * F4_SBLOCK + lane;
  const int fb = 8 * F4_CBLOCK + (wn * 4) * F4_CBLOCK + lane * 16;
  const int fsb = F4_WS + (wn * 4) * F4_SBLOCK + lane;
  struct Frags {
    v4i a[2], b[4];
    int sa[2], sb[4];
  };
  // fragments of group gh (0, 1) of the stage at position q
  auto load_frags = [&](Frags& f, int q, int gh) {
    const uint8_t* sp = lds + (q & (F4_NSLOT - 1)) * F4_SLOT + gh * F4_GRP;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const v4u x = *reinterpret_cast<const v4u*>(sp + fa + tr * F4_CBLOCK);
      f.a[tr] = v4i{(int)x[0], (int)x[1], (int)x[2], (int)x[3]};
      f.sa[tr] = sp[fsa + tr * F4_SBLOCK];
    }
#pragma unroll
    for (int tc = 0; tc < 4; ++tc) {
      const v4u x = *reinterpret_cast<const v4u*>(sp + fb + tc * F4_CBLOCK);
      f.b[tc] = v4i{(int)x[0], (int)x[1], (int)x[2], (int)x[3]};
      f.sb[tc] = sp[fsb + tc * F4_SBLOCK];
    }
  };

  v16f acc[2][4];
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int tc = 0; tc < 4; ++tc)
        acc[tr][tc] = svdq_mfma_scale_e2m1(f.b[tc], f.a[tr], acc[tr][tc], FP4_FMT, FP4_FMT, 0,
                                           f.sb[tc], 0, f.sa[tr]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- pre-stage fragments
  const int pta = (wm * 2) * LR_XBLOCK + lane * 16;
  const int plb = F4_PRE_L2 + (wn * 4) * LR_WBLOCK + lane * 16;
  const int pbias = F4_PRE_BIAS + 2 * (wn * 4) * 32;

  // Reading position t issues position t + 2, except at the first two
  // positions of a tile: their two successors were issued at the end of the
  // previous tile (or here), before its output stores.
  dma_stage(0);
  dma_stage(1);
  dma_stage(2);
  dma_stage(3);
#pragma unroll
  for (int i = 0; i < F4_NST; ++i) dma4_f4(wimg, voff4, lds_base + F4_NSLOT * F4_SLOT);
  int q = 0;
  Frags f0, f1;
  // one code stage at position q: group 2s (f0) reads the first half of its
  // slot, group 2s+1 (f1) the second; with NEXT the next stage's wait,
  // barrier and DMA issue sit between them (GEN: the DMA issued, position
  // q + 3, is not a code stage of this tile and takes the generic form)
  // (BODY: a stage past the tile's fourth position, whose wait needs no
  // branch, so that the loop over such stages is one basic block)
  auto code_stage = [&](int q, int s, auto next_tag, auto gen_tag, auto body_tag) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool GEN = decltype(gen_tag)::value;
    constexpr bool BODY = decltype(body_tag)::value;
    load_frags(f1, q, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    if constexpr (NEXT) {
      if constexpr (BODY) wait_stage();
      else if (P + s + 1 >= 4) wait_stage();  // else covered by the first code stage's wait
      barrier();
      if constexpr (GEN) dma_stage(q + 3);
      else dma_code(q + 3);
      load_frags(f0, q + 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
  };
#pragma nounroll
  for (int k = 0; k < my_tiles; ++k) {
    {  // the body DMAs start at code stage 3 (groups 6, 7)
      const int64_t xrow = (int64_t)cur_t.tm * (F4_BM / 32), wrow = (int64_t)cur_t.tn * (F4_BN / 32);
      xrun = ximg + (6 * x_rt + xrow) * F4_CBLOCK + dx;
      wrun = wimg + (6 * w_ct + wrow) * F4_CBLOCK + dx;
      srun = s_side == 0 ? ximg + x_sc + ((6 + s_gh) * x_rt + xrow) * F4_SBLOCK
                         : wimg + w_sc + ((6 + s_gh) * w_ct + wrow) * F4_SBLOCK;
      srun += s_half * 256;
    }
#pragma nounroll
    for (int jp = 0; jp < P; ++jp, ++q) {
      wait_at(jp);
      barrier();
      if (jp >= 2) dma_stage(q + 2);
      const uint8_t* sp = lds + (q & (F4_NSLOT - 1)) * F4_SLOT;
      if (jp == 0) init_bias_t<2, 4>(acc, sp + pbias, lane);
      if (jp < R16) {
        v8bf thi[2], tlo[2], lb[4];
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          thi[tr] = *reinterpret_cast<const v8bf*>(sp + pta + tr * LR_XBLOCK);
          tlo[tr] = *reinterpret_cast<const v8bf*>(sp + pta + tr * LR_XBLOCK + 1024);
        }
#pragma unroll
        for (int tc = 0; tc < 4; ++tc)
          lb[tc] = *reinterpret_cast<const v8bf*>(sp + plb + tc * LR_WBLOCK);
#pragma unroll
        for (int tr = 0; tr < 2; ++tr)
#pragma unroll
          for (int tc = 0; tc < 4; ++tc) {
            acc[tr][tc] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], thi[tr], acc[tr][tc], 0, 0, 0);
            acc[tr][tc] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], tlo[tr], acc[tr][tc], 0, 0, 0);
          }
      }
    }
    // code stages
    wait_at(P);
    barrier();
    dma_stage(q + 2);
    load_frags(f0, q, 0);
    // code stage s reads position P + s + 1 and issues P + s + 3 (stage s + 3)
    using T_ = std::true_type;
    using F_ = std::false_type;
    int s = 0;
    // a stage whose next position is among the tile's first four
#pragma nounroll
    for (; s < 3 - P && s + 3 < S; ++s, ++q) code_stage(q, s, T_{}, F_{}, F_{});
#pragma nounroll
    for (; s + 3 < S; ++s, ++q) code_stage(q, s, T_{}, F_{}, T_{});
    // the last two stages with a successor issue beyond the tile's code
    // stages (S == 2: one, S == 1: none)
    if (S > 2) code_stage(q++, S - 3, T_{}, T_{}, F_{});
    if (S > 1) code_stage(q++, S - 2, T_{}, T_{}, F_{});
    code_stage(q, S - 1, F_{}, F_{}, F_{});
    ++q;

    const int64_t mbase = (int64_t)cur_t.tm * F4_BM + wm * 64;
    const int nbase = cur_t.tn * F4_BN + wn * 128;
    if (k + 1 < my_tiles) {
      // every wave is done with the last two stages' slots: fill them with
      // the next tile's third and fourth stages before the stores
      barrier();
      cur_base = (k + 1) * SPT;
      cur_t = nxt_t;
      if (k + 2 < my_tiles) nxt_t = tile_xy4(tile_number4(b, k + 2, nwg, ntiles), num_m, num_n);
      dma_stage(q + 2);
      dma_stage(q + 3);
    }
    store_tiles_t<2, 4>(acc, M, N, mbase, nbase, lane, out_f32 != 0, Y);
    // an edge tile may issue fewer stores than the waits above count on
    if (!(mbase + 64 <= M && nbase + 128 <= N)) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  // DMAs past the end land before LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

hipError_t launch_fp4_forward(bool out_f32, int64_t M, int N, int K, int rank,
                              const void* ximage, const void* wimage, void* Y, hipStream_t s) {
  const ActImage a = act_image(1, M, K, rank);
  const WeightImage w = weight_image(1, N, K, rank);
  const int64_t tiles = (a.RT / (F4_BM / 32)) * (w.CT / (F4_BN / 32));
  const int64_t grid = std::min<int64_t>(tiles, device_cus());
  if (rank > 0)
    hipLaunchKernelGGL(fp4_gemm_kernel<true>, dim3((unsigned)grid), dim3(F4_THREADS), 0, s, M, N, K, rank,
                     (int)out_f32, reinterpret_cast<const uint8_t*>(ximage), a.RT, (int64_t)a.scale,
                     (int64_t)a.lr, reinterpret_cast<const uint8_t*>(wimage), w.CT,
                     (int64_t)w.scale, (int64_t)w.lr, (int64_t)w.bias, Y);
  else
    hipLaunchKernelGGL(fp4_gemm_kernel<false>, dim3((unsigned)grid), dim3(F4_THREADS), 0, s, M, N, K, rank,
                     (int)out_f32, reinterpret_cast<const uint8_t*>(ximage), a.RT, (int64_t)a.scale,
                     (int64_t)a.lr, reinterpret_cast<const uint8_t*>(wimage), w.CT,
                     (int64_t)w.scale, (int64_t)w.lr, (int64_t)w.bias, Y);
  return hipGetLastError();
}

}  // namespace svdq
