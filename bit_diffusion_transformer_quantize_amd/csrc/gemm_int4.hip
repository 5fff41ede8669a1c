// INT4-mode W4A4 GEMM of the SVDQuant linear on gfx950.
//
//   Y = sum_g sx[m][g] sw[n][g] P_g[m][n] + T L2 + bias,
//   P_g = sum_{k in g} qx[m][k] qw[n][k]
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
// The low-rank term (the up-projection of the 16-bit branch, fused into the
// 4-bit kernel as on the apatero.com page, section "O que e Nunchaku e como
// acelera modelos Qwen") is T L2 with T split into bf16 high and low parts:
// two v_mfma_f32_32x32x16_bf16 per 16 ranks accumulate it straight into acc.
//
// Both operands come as images (image.h) laid out in MFMA lane order, and
// everything the kernel reads (codes, scale operands, T, L2, bias) reaches
// LDS through global->LDS DMA of contiguous runs.  The kernel is persistent:
// each workgroup walks a stream of stages over its tiles; per tile the
// stream holds P "pre" stages (the bias and one 16-rank slice of T and L2
// each) and then G code stages (one 64-group each).  Every stage is one LDS
// ring slot and every wave issues exactly four DMAs per stage, so the DMA
// engine simply runs two stages ahead, across tile boundaries: the next
// tile's bias, low-rank slices and first groups arrive while the current
// tile finishes.
//
// Compute: a 512-thread workgroup computes 256 x 192 outputs; each of its 8
// waves (two per SIMD) owns 64 x 96 (2 x 3 MFMA tiles).  The weight is the A
// operand and the activations the B operand of every MFMA, so a lane's
// accumulator holds one output row and quads of consecutive columns, which
// the epilogue stores 16 bytes at a time.  Within a group the
// MFMAs of tile t+1 are issued before the FMAs of tile t in the fixed order
// P MFMA, 8 FMAs, S MFMA, 8 FMAs, and each fragment register is reloaded for
// the next group right after its last MFMA.
// Tiles are ordered so that the workgroups of one XCD (own L2) walk a band
// of I4_GROUP_M row tiles of X across all weight columns.
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"
#include "image.h"
#include "kernels.h"

namespace svdq {

constexpr int I4_BM = 256;
constexpr int I4_BN = 192;
constexpr int I4_THREADS = 512;
constexpr int I4_SCALE_BYTE = 127 + 3;  // E2M3 field q has value q/8
constexpr int I4_GROUP_M = 2;           // tile rows walked together per XCD
constexpr int I4_NSLOT = 4;
constexpr int SLOT_A = (I4_BM / 32) * I4_BLOCK;               // 16 KB of X
constexpr int SLOT_BYTES = SLOT_A + (I4_BN / 32) * I4_BLOCK;  // + 12 KB of W
// pre-stage layout inside a slot: T hi/lo blocks, L2 blocks, the bias run
constexpr int PRE_L2 = (I4_BM / 32) * LR_XBLOCK;              // 16 KB
constexpr int PRE_BIAS = PRE_L2 + (I4_BN / 32) * LR_WBLOCK;   // 22 KB
static_assert(PRE_BIAS + 1024 <= SLOT_BYTES, "pre-stage fits a slot");
constexpr int FP6_FMT = 2;  // f8f6f4 format code of E2M3
// vector memory operations of one full output tile's bf16 stores per wave
// (2 per 32x32 tile; the fp32 form issues more, which only waits longer)
constexpr int I4_NST = 2 * 2 * 3;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4 with a
// scalar base): lane i reads sbase + voff and writes LDS bytes
// [lds_addr + 16 i, +16).  Written as a small asm block (it has no register
// outputs) so that the compiler neither drains it at barriers nor serialises
// consecutive DMAs; the kernel waits for it with explicit s_waitcnt vmcnt.
// The base is wave-uniform by construction; readfirstlane makes that
// explicit (each half zero-extended: readfirstlane returns a signed int).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// Global -> LDS DMA of 4 bytes per lane (global_load_lds_dword): lane i
// reads sbase + voff and writes LDS bytes [lds_addr + 4 i, +4).
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// Output tile coordinates of band-ordered tile number L.
struct TileXY {
  int tm, tn;
};

__device__ __forceinline__ TileXY tile_xy(int L, int num_m, int num_n) {
  const int band = L / (I4_GROUP_M * num_n);
  const int first_m = band * I4_GROUP_M;
  const int gm = min(num_m - first_m, I4_GROUP_M);
  const int in_band = L - band * I4_GROUP_M * num_n;
  return TileXY{first_m + in_band % gm, in_band / gm};
}

// Band-ordered tile number of the k-th tile of workgroup b: with the grid
// and the tile count both multiples of 8, the workgroups of XCD b%8 share a
// contiguous eighth of the tiles; otherwise tiles go round-robin.
__device__ __forceinline__ int tile_number(int b, int k, int nwg, int ntiles) {
  if ((nwg & 7) == 0 && (ntiles & 7) == 0) {
    const int per = ntiles >> 3, nw = nwg >> 3;
    return (b & 7) * per + (b >> 3) + k * nw;
  }
  return b + k * nwg;
}

__device__ __forceinline__ int tiles_of(int b, int nwg, int ntiles) {
  if ((nwg & 7) == 0 && (ntiles & 7) == 0) {
    const int per = ntiles >> 3, nw = nwg >> 3, w = b >> 3;
    return w < per ? (per - w + nw - 1) / nw : 0;
  }
  return b < ntiles ? (ntiles - b + nwg - 1) / nwg : 0;
}

// LR: the layer has a low-rank branch (rank > 0); the two forms are
// separate kernels so that traces tell the rank-0 launches apart.
template <bool LR>
__global__ __launch_bounds__(I4_THREADS) void int4_gemm_kernel(
    int64_t M, int N, int K, int rank, int out_f32, const uint8_t* __restrict__ ximg,
    int64_t x_rt, int64_t x_lr, const uint8_t* __restrict__ wimg, int64_t w_ct, int64_t w_lr,
    int64_t w_bias, void* __restrict__ Y) {
  // the ring, then a 256-byte pad that only dummy DMAs write
  __shared__ __attribute__((aligned(1024))) uint8_t lds[I4_NSLOT * SLOT_BYTES + 256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int num_m = (int)(x_rt / (I4_BM / 32));
  const int num_n = (int)(w_ct / (I4_BN / 32));
  const int ntiles = num_m * num_n;
  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int my_tiles = tiles_of(b, nwg, ntiles);
  if (my_tiles == 0) return;  // uniform per workgroup: no barrier is reached
  const int G = K >> 6;
  const int R16 = LR ? rank >> 4 : 0;
  // pre-stages per tile: the bias rides in the first, one 16-rank slice of
  // the low-rank branch in each of the first R16 (at least one).  A pre
  // stage has next to no work, so each one past what the branch needs
  // would only wait on the DMA stream at the head of the tile; the code
  // stages among a tile's first four positions wait with the counts of
  // those positions instead.
  const int P = R16 > 1 ? R16 : 1;
  const int SPT = P + G;            // stages per tile
  const int total = my_tiles * SPT;

  // ---- DMA, generic form: stream position q (the heads and tails of
  // tiles).  Wave w moves chunk slots w, w+8, w+16, w+24 of the stage (1 KB
  // each, landing at slot + 1 KB * chunk).
  //   code stage: chunks 0..15 X codes, 16..27 W codes, 28..31 repeat 16..19
  //   pre stage:  chunks 0..15 T hi/lo, 16..21 L2, 22 the bias run,
  //               23..31 repeat 14..22 (a pre stage past the rank: every
  //               chunk is the bias run)
  // A repeated chunk writes the same bytes to the same place.
  const uint32_t voff = (uint32_t)(lane * 16);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  TileXY cur_t = tile_xy(tile_number(b, 0, nwg, ntiles), num_m, num_n);
  TileXY nxt_t = my_tiles > 1 ? tile_xy(tile_number(b, 1, nwg, ntiles), num_m, num_n) : cur_t;
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
    const int g = pre ? 0 : j - P;
    const int jl = lr ? j : 0;
    const uint8_t* xc = ximg + ((int64_t)g * x_rt + tm * (I4_BM / 32)) * I4_BLOCK;
    const uint8_t* wc = wimg + ((int64_t)g * w_ct + tn * (I4_BN / 32)) * I4_BLOCK;
    const uint8_t* tl = ximg + x_lr + ((int64_t)jl * x_rt + tm * (I4_BM / 32)) * LR_XBLOCK;
    const uint8_t* ll = wimg + w_lr + ((int64_t)jl * w_ct + tn * (I4_BN / 32)) * LR_WBLOCK;
    const uint8_t* bs = wimg + w_bias + (int64_t)tn * (I4_BN / 32) * BIAS_BLOCK;
    const uint32_t slot = lds_base + (uint32_t)((q & (I4_NSLOT - 1)) * SLOT_BYTES);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = wave + 8 * i;
      // code stage
      const int cc = c >= 28 ? c - 12 : c;
      const uint8_t* csrc = cc < 16 ? xc + cc * 1024 : wc + (cc - 16) * 1024;
      // pre stage
      const int pc = lr ? (c >= 23 ? c - 9 : c) : 22;
      const uint8_t* psrc = pc < 16 ? tl + pc * 1024 : (pc < 22 ? ll + (pc - 16) * 1024 : bs);
      const uint8_t* src = pre ? psrc : csrc;
      const int dst = (pre ? pc : cc) * 1024;
      dma16(src, voff, slot + (uint32_t)dst);
    }
  };
  // ---- DMA, body form: a code stage of the current tile from running
  // pointers (xrun, wrun: the X and W code blocks of the target group),
  // moving the chunks the generic form gives this wave: X chunks w and
  // w + 8, W chunks w and c3.
  const int c3 = wave < 4 ? wave + 8 : wave - 4;
  const uint32_t dx0 = (uint32_t)wave * 1024, dx1 = dx0 + 8 * 1024;
  const uint32_t dw2 = SLOT_A + dx0, dw3 = SLOT_A + (uint32_t)c3 * 1024;
  const int64_t xstep = x_rt * I4_BLOCK, wstep = w_ct * I4_BLOCK;
  const uint8_t* xrun = ximg;
  const uint8_t* wrun = wimg;
  auto dma_code = [&](int q) {
    const uint32_t slot = lds_base + (uint32_t)((q & (I4_NSLOT - 1)) * SLOT_BYTES);
    dma16(xrun + dx0, voff, slot + dx0);
    dma16(xrun + dx1, voff, slot + dx1);
    dma16(wrun + dx0, voff, slot + dw2);
    dma16(wrun + (dw3 - SLOT_A), voff, slot + dw3);
    xrun += xstep;
    wrun += wstep;
  };
  // Waits for this wave's DMA of the stage about to be read.  Vector memory
  // operations of a wave complete in issue order on gfx9, so the wait names
  // how many younger operations may still be in flight: in the body of a
  // tile the next stage's four DMAs (vmcnt(4)); at the first four stages of
  // a tile (j = 0..3) up to three younger stages plus the I4_NST output
  // stores of the previous tile, issued behind them (before the first tile,
  // I4_NST dummy DMAs into the pad stand in for them).
  auto wait_stage = [] { __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); };
  // positions 2 and 3 (pre or code stages): one stage and the stores are younger
  auto wait_head2 = [] { __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 + I4_NST)); };
  auto wait_at = [&](int j) {
    if (j == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(12 + I4_NST));
    else if (j == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 + I4_NST));
    else if (j < 4) wait_head2();
    else wait_stage();
  };
  auto barrier = [] { asm volatile("s_barrier" ::: "memory"); };

  // ---- fragments within a slot (see the image layout)
  const int fa = (wm * 2) * I4_BLOCK + h * 768 + l32 * 16;
  const int fa8 = (wm * 2) * I4_BLOCK + h * 768 + 512 + l32 * 8;
  const int fsa = (wm * 2) * I4_BLOCK + 1536 + lane * 8;
  const int fb = SLOT_A + (wn * 3) * I4_BLOCK + h * 768 + l32 * 16;
  const int fb8 = SLOT_A + (wn * 3) * I4_BLOCK + h * 768 + 512 + l32 * 8;
  const int fsb = SLOT_A + (wn * 3) * I4_BLOCK + 1536 + lane * 8;

  v6i af[2], bf[3];
  v4s sa[2], sb[3];
  auto load_a = [&](const uint8_t* sp, int tr) {
    const v4u x = *reinterpret_cast<const v4u*>(sp + fa + tr * I4_BLOCK);
    const v2u y = *reinterpret_cast<const v2u*>(sp + fa8 + tr * I4_BLOCK);
    af[tr] = v6i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1]};
    sa[tr] = *reinterpret_cast<const v4s*>(sp + fsa + tr * I4_BLOCK);
  };
  auto load_b = [&](const uint8_t* sp, int tc) {
    const v4u x = *reinterpret_cast<const v4u*>(sp + fb + tc * I4_BLOCK);
    const v2u y = *reinterpret_cast<const v2u*>(sp + fb8 + tc * I4_BLOCK);
    bf[tc] = v6i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1]};
    sb[tc] = *reinterpret_cast<const v4s*>(sp + fsb + tc * I4_BLOCK);
  };
  auto slot_ptr = [&](int q) { return lds + (q & (I4_NSLOT - 1)) * SLOT_BYTES; };

  v16f zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero[i] = 0.f;
  v16f acc[2][3];
  v16f p[2], sc[2];

  // tile t of a wave = (t / 3, t % 3); its P and S live in p/sc[t & 1]
  auto mfma_p = [&](int t) {
    const int tr = t / 3, tc = t % 3, bb = t & 1;
    p[bb] = svdq_mfma_scale_e2m3(bf[tc], af[tr], zero, FP6_FMT, FP6_FMT,
                                 0, I4_SCALE_BYTE, 0, I4_SCALE_BYTE);
  };
  auto mfma_s = [&](int t) {
    const int tr = t / 3, tc = t % 3, bb = t & 1;
    sc[bb] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sb[tc], sa[tr], zero, 0, 0, 0);
  };
  // FMAs i0 .. i0+7 of tile t: acc += P * S
  auto fma_half = [&](int t, int i0) {
    const int tr = t / 3, tc = t % 3, bb = t & 1;
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) acc[tr][tc][i] = fmaf(p[bb][i], sc[bb][i], acc[tr][tc][i]);
  };
  // One step: the MFMAs of tile `next` (if any) interleaved with the FMAs of
  // tile `cur`, in the fixed order P MFMA, 8 FMAs, S MFMA, loads (of the
  // fragments both MFMAs just read for the last time), 8 FMAs.
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

  // One code group at stream position q.  NEXT: the next position is the
  // tile's next group, read progressively during this one (its wait,
  // barrier and DMA issue sit in step 1, after the first fragment has been
  // freed); otherwise this is the tile's last group.  The DMA it issues
  // (position q + 3, code group g + 3) takes the body form while that is a
  // code stage of this tile and the generic form otherwise.  The last group
  // instead ends the tile's use of the ring at step 1 (every fragment of
  // its stage is in registers once tile 2's MFMAs have issued: LDS reads
  // return in order), moves the DMA window to the next tile and issues that
  // tile's third and fourth positions, ahead of the output stores.
  // BODY: a group known to be neither among a tile's first four positions
  // nor one of its last three, so that its wait and DMA take the body forms
  // without a branch: the loop over such groups is one basic block, and the
  // compiler keeps each step's MFMAs where they are written instead of
  // sinking them past the barrier into the block that reads their results.
  auto group = [&](int q, int g, auto next_tag, auto body_tag, int k) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool BODY = decltype(body_tag)::value;
    const uint8_t* nsp = slot_ptr(q + 1);
    step(1, 0, [] {});
    step(2, 1, [&] {  // A tile row 0 is free
      if constexpr (NEXT) {
        if constexpr (BODY) {
          wait_stage();
          barrier();
          dma_code(q + 3);
        } else {
          if (P + g + 1 < 4) wait_head2();  // the next position is the tile's third or fourth
          else wait_stage();
          barrier();
          if (g + 3 < G) dma_code(q + 3);
          else dma_stage(q + 3);
        }
        load_a(nsp, 0);
      } else if (k + 1 < my_tiles) {
        barrier();
        cur_base = (k + 1) * SPT;
        cur_t = nxt_t;
        if (k + 2 < my_tiles) nxt_t = tile_xy(tile_number(b, k + 2, nwg, ntiles), num_m, num_n);
        dma_stage(q + 3);
        dma_stage(q + 4);
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

  // ---- pre-stage fragments: T hi/lo (A), L2 (B), the bias
  const int pta = (wm * 2) * LR_XBLOCK + lane * 16;
  const int plb = PRE_L2 + (wn * 3) * LR_WBLOCK + lane * 16;
  const int pbias = PRE_BIAS + 2 * (wn * 3) * 32;

  // ---- the stream.  Reading position t issues position t + 2, except at
  // the first two positions of a tile: their two successors were issued at
  // the end of the previous tile (or here), before its output stores.
  dma_stage(0);
  dma_stage(1);
  dma_stage(2);
  dma_stage(3);
#pragma unroll
  for (int i = 0; i < I4_NST; ++i) dma4(wimg, voff >> 2, lds_base + I4_NSLOT * SLOT_BYTES);
  int q = 0;  // next stream position to read
#pragma nounroll
  for (int k = 0; k < my_tiles; ++k) {
    // the body DMAs start at code group 3
    xrun = ximg + ((int64_t)3 * x_rt + cur_t.tm * (I4_BM / 32)) * I4_BLOCK;
    wrun = wimg + ((int64_t)3 * w_ct + cur_t.tn * (I4_BN / 32)) * I4_BLOCK;
    // pre-stages: the bias, then the low-rank slices accumulate into acc
#pragma nounroll
    for (int jp = 0; jp < P; ++jp, ++q) {
      wait_at(jp);
      barrier();
      if (jp >= 2) dma_stage(q + 2);  // positions 2, 3 were issued at the previous tile's end
      const uint8_t* sp = slot_ptr(q);
      if (jp == 0) init_bias_t<2, 3>(acc, sp + pbias, lane);
      if (jp < R16) {
        v8bf thi[2], tlo[2], lb[3];
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          thi[tr] = *reinterpret_cast<const v8bf*>(sp + pta + tr * LR_XBLOCK);
          tlo[tr] = *reinterpret_cast<const v8bf*>(sp + pta + tr * LR_XBLOCK + 1024);
        }
#pragma unroll
        for (int tc = 0; tc < 3; ++tc)
          lb[tc] = *reinterpret_cast<const v8bf*>(sp + plb + tc * LR_WBLOCK);
#pragma unroll
        for (int tr = 0; tr < 2; ++tr)
#pragma unroll
          for (int tc = 0; tc < 3; ++tc) {
            acc[tr][tc] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], thi[tr], acc[tr][tc], 0, 0, 0);
            acc[tr][tc] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], tlo[tr], acc[tr][tc], 0, 0, 0);
          }
      }
    }
    // the first code group: all its fragments, then its first tile's MFMAs
    wait_at(P);
    barrier();
    if (P >= 2) dma_stage(q + 2);  // with P = 1, position 3 is already in flight
    {
      const uint8_t* sp = slot_ptr(q);
      load_a(sp, 0);
      load_a(sp, 1);
      load_b(sp, 0);
      load_b(sp, 1);
      load_b(sp, 2);
    }
    mfma_p(0);
    mfma_s(0);
    // group g reads position P + g + 1 and issues P + g + 3 (code group g + 3)
    using T_ = std::true_type;
    using F_ = std::false_type;
    const int64_t mbase = (int64_t)cur_t.tm * I4_BM + wm * 64;
    const int nbase = cur_t.tn * I4_BN + wn * 96;
    int g = 0;
    // the groups whose next position is among the tile's first four
    // (g < 3 - P), the body, then the two groups whose DMA lies past the
    // tile's code groups, and the last
#pragma nounroll
    for (; g < 3 - P && g + 1 < G; ++g, ++q) group(q, g, T_{}, F_{}, k);
#pragma nounroll
    for (; g + 3 < G; ++g, ++q) group(q, g, T_{}, T_{}, k);
#pragma nounroll
    for (; g + 1 < G; ++g, ++q) group(q, g, T_{}, F_{}, k);
    group(q, g, F_{}, F_{}, k);
    ++q;

    store_tiles_t<2, 3>(acc, M, N, mbase, nbase, lane, out_f32 != 0, Y);
    // an edge tile may issue fewer stores than the waits above count on
    if (!(mbase + 64 <= M && nbase + 96 <= N)) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  // the DMAs past the end of the stream must land before LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cus[dev] > 0) return cus[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cus[dev] = n;
  return n;
}

hipError_t launch_int4_forward(bool out_f32, int64_t M, int N, int K, int rank,
                               const void* ximage, const void* wimage, void* Y, hipStream_t s) {
  const ActImage a = act_image(0, M, K, rank);
  const WeightImage w = weight_image(0, N, K, rank);
  const int64_t tiles = (a.RT / (I4_BM / 32)) * (w.CT / (I4_BN / 32));
  const int64_t grid = std::min<int64_t>(tiles, device_cus());
  if (rank > 0)
    hipLaunchKernelGGL(int4_gemm_kernel<true>, dim3((unsigned)grid), dim3(I4_THREADS), 0, s, M, N, K,
                     rank, (int)out_f32, reinterpret_cast<const uint8_t*>(ximage), a.RT,
                     (int64_t)a.lr, reinterpret_cast<const uint8_t*>(wimage), w.CT, (int64_t)w.lr,
                     (int64_t)w.bias, Y);
  else
    hipLaunchKernelGGL(int4_gemm_kernel<false>, dim3((unsigned)grid), dim3(I4_THREADS), 0, s, M, N, K,
                     rank, (int)out_f32, reinterpret_cast<const uint8_t*>(ximage), a.RT,
                     (int64_t)a.lr, reinterpret_cast<const uint8_t*>(wimage), w.CT, (int64_t)w.lr,
                     (int64_t)w.bias, Y);
  return hipGetLastError();
}

}  // namespace svdq
