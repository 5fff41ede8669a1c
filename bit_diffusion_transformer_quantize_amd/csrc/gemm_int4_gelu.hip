// The FLUX MLP up-projection with its epilogue fused to the next layer's
// activation pass (INT4 mode): the W4A4 GEMM of the up layer, then, instead
// of writing its bf16 output, per element GELU(tanh), the down layer's
// smoothing x / lambda_down, the down layer's per-group INT4 quantization
// written straight into the down layer's activation image, and the down
// layer's low-rank down-projection T = X_hat L1 as per-tile partial sums.
// This removes the bf16 intermediate (written by the up GEMM and read back
// by the down layer's activation pass) that a separate pass needs; the
// Nunchaku Lite page on axbrief.com ("The Trade-off Between Fused Kernels
// and Generality") describes fusing neighbouring steps of the block into one
// kernel to cut memory traffic, and the apatero.com page ("O que e Nunchaku
// e como acelera modelos Qwen") the low-rank branch sharing the quantization
// kernel's read of the activations.
//
// One 256 x 128 output tile per workgroup of 8 waves (4 row bands of 64 x
// 2 column halves of 64): each wave's 64 columns are exactly one 64-group of
// the down layer's K, so a row's absmax is a lane-pair maximum.  The main
// product per 32 x 32 tile and 64-group is the one of int4_gemm_kernel:
// one FP6 (E2M3) scaled MFMA on the exact codes, one bf16 outer-product MFMA
// of the split scales and one FMA per output, in group order after the bias
// and T L2, so the fp32 accumulator (and the bf16 up output, optionally
// written) is the same arithmetic as svdq_linear_forward's.
//
// Epilogue per 32-row tile: y -> bf16 RNE -> GELU (the band table of the
// activation pass) -> x_hat = bf16_RNE(fp32(x / lambda)) with the exact
// fp64-reciprocal quotient -> amax over the 64 columns (lane l and l ^ 32)
// -> s = fp32(amax / 7), codes of clamp(fp32(x_hat / s), -8, 7) as E2M3
// fields by the hardware conversion, after one lane-half exchange so that
// each lane holds the 32 consecutive columns of one K half; T partial =
// x_hat (in the accumulator layout, which is the B operand layout of the
// bf16 32x32x8 MFMA) times the tile's slice of L1, summed over the two
// column waves through LDS.  split over the column tiles, the partial sums
// are added in tile order by fg_finish_t_kernel into the image's T halves.
#include <algorithm>

#include <type_traits>

#include "gemm_common.h"
#include "gelu_table.h"
#include "image.h"
#include "kernels.h"

namespace svdq {

constexpr int FG_BM = 256;
constexpr int FG_BN = 128;
constexpr int FG_THREADS = 512;
constexpr int FG_NSLOT = 4;
constexpr int FG_SLOT_X = (FG_BM / 32) * I4_BLOCK;            // 16 KB
constexpr int FG_SLOT = FG_SLOT_X + (FG_BN / 32) * I4_BLOCK;  // 24 KB
constexpr int FG_RING = FG_NSLOT * FG_SLOT;                   // 96 KB
constexpr int FG_SCALE_BYTE = 127 + 3;
constexpr int FG_FP6 = 2;

typedef short v4s_fg __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_fg;

__device__ __forceinline__ void fg_dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// RD4 = number of 32-rank tiles of the down layer's rank (0 .. 4).
template <int RD4>
__global__ __launch_bounds__(FG_THREADS) void fg_gemm_kernel(
    int64_t M, int N, int K, int rank_up, const uint8_t* __restrict__ ximg, int64_t x_rt,
    int64_t x_lr, const uint8_t* __restrict__ wimg, int64_t w_ct, int64_t w_lr, int64_t w_bias,
    int rank_dn, const float* __restrict__ lambda_dn, const uint16_t* __restrict__ lora_dn,
    uint8_t* __restrict__ dimg, int64_t d_rt, float* __restrict__ tpart,
    uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[FG_RING];
  __shared__ uint16_t gtab[gelu_table::kEntries];
  __shared__ __attribute__((aligned(16))) double rlam[FG_BN];
  __shared__ __attribute__((aligned(16))) uint16_t l1s[(RD4 > 0 ? RD4 : 1) * 32 * FG_BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int G = K >> 6;

  // tile of this workgroup: the workgroups of one XCD (blockIdx % 8) take a
  // contiguous run of tiles in row-major order (shared activation rows)
  const int num_n = N / FG_BN;
  const int ntiles = (int)(x_rt / (FG_BM / 32)) * num_n;
  int L = blockIdx.x;
  if ((gridDim.x & 7) == 0) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (L >= ntiles) return;
  const int tm = L / num_n, tn = L - (L / num_n) * num_n;
  const int64_t row0 = (int64_t)tm * FG_BM;
  const int col0 = tn * FG_BN;

  // ---- the main product's stream: group g is one stage of a 4-slot DMA
  // ring: 16 KB of X codes (8 row blocks) then 8 KB of W codes (4 column
  // blocks), 24 chunks of 1 KB; wave w moves chunks w, w+8, w+16.  The first
  // three stages are issued first, then every other load of the tile, so
  // that their latencies overlap.
  const uint32_t voff = (uint32_t)(lane * 16);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_fg*)ring;
  const uint8_t* xg0 = ximg + (row0 / 32) * I4_BLOCK;
  const uint8_t* wg0 = wimg + (int64_t)(col0 / 32) * I4_BLOCK;
  const int64_t xstep = x_rt * I4_BLOCK, wstep = w_ct * I4_BLOCK;
  auto dma_stage = [&](int g) {
    const uint32_t slot = lds_base + (uint32_t)((g & (FG_NSLOT - 1)) * FG_SLOT);
    const uint8_t* xs = xg0 + (int64_t)g * xstep;
    const uint8_t* ws = wg0 + (int64_t)g * wstep;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = wave + 8 * i;
      const uint8_t* src = c < 16 ? xs + c * 1024 : ws + (c - 16) * 1024;
      fg_dma16(src, voff, slot + (uint32_t)(c * 1024));
    }
  };
  dma_stage(0);
  if (G > 1) dma_stage(1);
  if (G > 2) dma_stage(2);

  // bias of the wave's columns (in the accumulator's column order)
  v2u bias_w[2][4];
  {
    const uint8_t* bias = wimg + w_bias + (int64_t)(col0 / 32 + wn * 2) * BIAS_BLOCK;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bias_w[tc][q] = *reinterpret_cast<const v2u*>(bias + tc * BIAS_BLOCK + 2 * (8 * q + 4 * h));
  }
  // ---- tile constants in LDS: GELU band, lambda reciprocals, and the
  // tile's slice of L1 in the lane order of the T MFMA's A operand: fragment
  // (j4, cg) for ranks 32 j4 .. +31 and tile columns 8 cg .. +7 is 64 lanes
  // x 8 bytes, lane l holding rank 32 j4 + l%32, columns 8 cg + 4 (l/32) .. +3
  for (int i = tid; i < gelu_table::kEntries / 2; i += FG_THREADS)
    reinterpret_cast<uint32_t*>(gtab)[i] = reinterpret_cast<const uint32_t*>(kGeluBand.v)[i];
  if (tid < FG_BN) rlam[tid] = 1.0 / (double)lambda_dn[col0 + tid];
  if constexpr (RD4 > 0) {
    for (int i = tid; i < RD4 * (FG_BN / 8) * 64; i += FG_THREADS) {
      const int fl = i & 63, frag = i >> 6;
      const int j4 = frag / (FG_BN / 8), cg = frag - j4 * (FG_BN / 8);
      const int j = 32 * j4 + (fl & 31);
      v2u v = {0u, 0u};
      if (j < rank_dn)
        v = *reinterpret_cast<const v2u*>(lora_dn + (int64_t)j * N + col0 + 8 * cg + 4 * (fl >> 5));
      *reinterpret_cast<v2u*>(l1s + 4 * i) = v;
    }
  }
  __syncthreads();  // the tables are in LDS

  // ---- the accumulator: bias, then T L2 (bf16 hi/lo of T)
  v16f acc[2][2];
  {
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v2u w = bias_w[tc][q];
        const float b4[4] = {bf16_to_f32(w[0] & 0xFFFFu), bf16_to_f32(w[0] >> 16),
                             bf16_to_f32(w[1] & 0xFFFFu), bf16_to_f32(w[1] >> 16)};
#pragma unroll
        for (int tr = 0; tr < 2; ++tr)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tr][tc][4 * q + e] = b4[e];
      }
    for (int j = 0; j < (rank_up >> 4); ++j) {
      v8bf thi[2], tlo[2], lb[2];
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const uint8_t* tb = ximg + x_lr + ((int64_t)j * x_rt + row0 / 32 + wm * 2 + tr) * LR_XBLOCK;
        thi[tr] = *reinterpret_cast<const v8bf*>(tb + 16 * lane);
        tlo[tr] = *reinterpret_cast<const v8bf*>(tb + 1024 + 16 * lane);
      }
#pragma unroll
      for (int tc = 0; tc < 2; ++tc)
        lb[tc] = *reinterpret_cast<const v8bf*>(
            wimg + w_lr + ((int64_t)j * w_ct + col0 / 32 + wn * 2 + tc) * LR_WBLOCK + 16 * lane);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
          acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], thi[tr], acc[tr][tc], 0, 0, 0);
          acc[tr][tc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[tc], tlo[tr], acc[tr][tc], 0, 0, 0);
        }
    }
  }

  // ---- the main product over the code groups; a stage's wait counts the
  // younger stages still in flight (every older load has completed: the
  // low-rank MFMAs above waited for theirs)
  const int fa = (wm * 2) * I4_BLOCK + h * 768 + l32 * 16;
  const int fa8 = (wm * 2) * I4_BLOCK + h * 768 + 512 + l32 * 8;
  const int fsa = (wm * 2) * I4_BLOCK + 1536 + lane * 8;
  const int fb = FG_SLOT_X + (wn * 2) * I4_BLOCK + h * 768 + l32 * 16;
  const int fb8 = FG_SLOT_X + (wn * 2) * I4_BLOCK + h * 768 + 512 + l32 * 8;
  const int fsb = FG_SLOT_X + (wn * 2) * I4_BLOCK + 1536 + lane * 8;
  v16f zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero[i] = 0.f;

  // fragments: A (activation) rows t and B (weight) columns t of the wave,
  // each with its bf16 scale operand; one set, each fragment reloaded for the
  // next group right after its last use in the current one
  v6i af[2], bf[2];
  v4s_fg sa[2], sb[2];
  auto load_a = [&](const uint8_t* sp, int t) {
    const v4u x = *reinterpret_cast<const v4u*>(sp + fa + t * I4_BLOCK);
    const v2u y = *reinterpret_cast<const v2u*>(sp + fa8 + t * I4_BLOCK);
    af[t] = v6i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1]};
    sa[t] = *reinterpret_cast<const v4s_fg*>(sp + fsa + t * I4_BLOCK);
  };
  auto load_b = [&](const uint8_t* sp, int t) {
    const v4u x = *reinterpret_cast<const v4u*>(sp + fb + t * I4_BLOCK);
    const v2u y = *reinterpret_cast<const v2u*>(sp + fb8 + t * I4_BLOCK);
    bf[t] = v6i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1]};
    sb[t] = *reinterpret_cast<const v4s_fg*>(sp + fsb + t * I4_BLOCK);
  };
  auto slot_ptr = [&](int g) { return ring + (g & (FG_NSLOT - 1)) * FG_SLOT; };
  // wait until stage t has landed (this wave's part: the stages issued after
  // it, at most two, may still be in flight; the wave's earlier fragment
  // reads have returned), then every wave's part
  auto wait_stage = [&](int t) {
    const int after = min(2, G - 1 - t);
    if (after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  v16f p[2], sc[2];
  auto mf = [&](int t) {  // the MFMAs of tile t = (t / 2, t % 2) into buffer t & 1
    const int tr = t >> 1, tc = t & 1, bb = t & 1;
    p[bb] = svdq_mfma_scale_e2m3(bf[tc], af[tr], zero, FG_FP6, FG_FP6,
                                 0, FG_SCALE_BYTE, 0, FG_SCALE_BYTE);
    sc[bb] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sb[tc], sa[tr], zero, 0, 0, 0);
  };
  auto fm = [&](int t) {
    const int tr = t >> 1, tc = t & 1, bb = t & 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[tr][tc][i] = fmaf(p[bb][i], sc[bb][i], acc[tr][tc][i]);
  };

  // The stream: stage 0's fragments are read before the loop; in group g the
  // MFMAs of tiles 0 and 1 go first, then (g + 1 < G) the wait and barrier
  // for stage g + 1 and the DMA of stage g + 4 into the slot of stage g, and
  // each fragment of stage g + 1 is read as soon as its register is free.
  wait_stage(0);
  if (G > 3) dma_stage(3);
  load_a(slot_ptr(0), 0);
  load_a(slot_ptr(0), 1);
  load_b(slot_ptr(0), 0);
  load_b(slot_ptr(0), 1);
  // BODY: g + 4 < G, so the wait counts two younger stages and a DMA is
  // issued; the loop over such groups then has no branch and the compiler
  // keeps the MFMAs ahead of the barrier as written
  auto group = [&](int g, auto body_tag) {
    constexpr bool BODY = decltype(body_tag)::value;
    const bool more = BODY || g + 1 < G;
    const uint8_t* nsp = slot_ptr(g + 1);
    mf(0);
    mf(1);
    if (more) {
      if constexpr (BODY) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        dma_stage(g + 4);
      } else {
        wait_stage(g + 1);
        if (g + 4 < G) dma_stage(g + 4);
      }
      load_a(nsp, 0);  // row 0: last used by tile 1
    }
    fm(0);
    mf(2);
    if (more) load_b(nsp, 0);  // column 0: last used by tile 2
    fm(1);
    mf(3);
    if (more) {
      load_a(nsp, 1);
      load_b(nsp, 1);
    }
    fm(2);
    fm(3);
  };
  int g = 0;
#pragma nounroll
  for (; g + 4 < G; ++g) group(g, std::true_type{});
#pragma nounroll
  for (; g < G; ++g) group(g, std::false_type{});

  // ---- epilogue: the ring is free once every wave is past the last group
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("s_barrier" ::: "memory");

  float* xch = reinterpret_cast<float*>(ring);  // T exchange: [wm][j4][16][64]
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
    v16f tacc[RD4 > 0 ? RD4 : 1];
    const int64_t m = row0 + wm * 64 + tr * 32 + l32;  // this lane's row
    const bool mok = m < M;
    // (1) bf16 output of the up layer (optional)
    if (Y != nullptr && mok) {
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        uint16_t* yr = Y + m * N + col0 + wn * 64 + tc * 32 + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = pack_bf16x2(acc[tr][tc][4 * q], acc[tr][tc][4 * q + 1]);
          const uint32_t hi = pack_bf16x2(acc[tr][tc][4 * q + 2], acc[tr][tc][4 * q + 3]);
          *reinterpret_cast<v2u*>(yr + 8 * q) = v2u{lo, hi};
        }
      }
    }
    // (2) x_hat = bf16(fp32(GELU(bf16(y)) / lambda)), kept as bf16 bits and fp32
    uint32_t xb[2][16];
    float xf[2][16];
    float amax = 0.f;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int c = wn * 64 + tc * 32 + 8 * (i >> 2) + 4 * h + (i & 3);  // column in the tile
        const uint32_t yb = pack_bf16x2(acc[tr][tc][i], acc[tr][tc][i + 1]);
        const uint32_t gb = gelu_bf16x2(yb, gtab);
        const double2 rl = *reinterpret_cast<const double2*>(rlam + c);
        float q[2];
        q[0] = (float)((double)bf16_to_f32(gb & 0xFFFFu) * rl.x);
        q[1] = (float)((double)bf16_to_f32(gb >> 16) * rl.y);
        const v2f qv = {q[0], q[1]};
        const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(qv, v2bf));
        xb[tc][i] = mok ? (pk & 0xFFFFu) : 0u;
        xb[tc][i + 1] = mok ? (pk >> 16) : 0u;
        xf[tc][i] = __uint_as_float(xb[tc][i] << 16);
        xf[tc][i + 1] = __uint_as_float(xb[tc][i + 1] << 16);
        amax = fmaxf(amax, fmaxf(fabsf(xf[tc][i]), fabsf(xf[tc][i + 1])));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    // (3) T partial: rank tile j4 += L1 slice (A) x x_hat (B, accumulator layout)
    if constexpr (RD4 > 0) {
#pragma unroll
      for (int j4 = 0; j4 < RD4; ++j4) tacc[j4] = zero;
#pragma unroll
      for (int tc = 0; tc < 2; ++tc)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const v4s_fg xv = {(short)xb[tc][4 * s4], (short)xb[tc][4 * s4 + 1],
                             (short)xb[tc][4 * s4 + 2], (short)xb[tc][4 * s4 + 3]};
#pragma unroll
          for (int j4 = 0; j4 < RD4; ++j4) {
            const int cg = wn * 8 + tc * 4 + s4;
            const v4s_fg lv = *reinterpret_cast<const v4s_fg*>(l1s + 4 * ((j4 * (FG_BN / 8) + cg) * 64 + lane));
            tacc[j4] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(lv, xv, tacc[j4], 0, 0, 0);
          }
        }
    }
    // (4) INT4 codes of the group: cq = clamp(fp32(x_hat / s), -8, 7)
    const float s = amax / 7.0f;
    float cq[2][16];
    const double rs = s != 0.f ? 1.0 / (double)s : 0.0;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        cq[tc][i] = s != 0.f ? __builtin_amdgcn_fmed3f((float)((double)xf[tc][i] * rs), -8.0f, 7.0f)
                             : 0.f;
    // lane halves exchange: lane l < 32 gets the 32 columns of column tile 0
    // (K half 0), lane l >= 32 those of column tile 1 (K half 1); x_new holds
    // the columns 8 qd + 0..3, y_new 8 qd + 4..7
    float xn[16], yn[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cq[0][i]),
                                                       __float_as_uint(cq[1][i]), false, false);
      xn[i] = __uint_as_float(sw[0]);
      yn[i] = __uint_as_float(sw[1]);
    }
    v16f ev, od;  // column 2c -> ev[c], 2c + 1 -> od[c]
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      ev[4 * qd + 0] = xn[4 * qd + 0];
      od[4 * qd + 0] = xn[4 * qd + 1];
      ev[4 * qd + 1] = xn[4 * qd + 2];
      od[4 * qd + 1] = xn[4 * qd + 3];
      ev[4 * qd + 2] = yn[4 * qd + 0];
      od[4 * qd + 2] = yn[4 * qd + 1];
      ev[4 * qd + 3] = yn[4 * qd + 2];
      od[4 * qd + 3] = yn[4 * qd + 3];
    }
    const v6i f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
    const int64_t rt = (row0 + wm * 64 + tr * 32) / 32;
    const int gd = tn * 2 + wn;  // the down layer's group
    uint8_t* blk = dimg + ((int64_t)gd * d_rt + rt) * I4_BLOCK;
    *reinterpret_cast<v4u*>(blk + h * 768 + 16 * l32) =
        v4u{(uint32_t)f[0], (uint32_t)f[1], (uint32_t)f[2], (uint32_t)f[3]};
    *reinterpret_cast<v2u*>(blk + h * 768 + 512 + 8 * l32) = v2u{(uint32_t)f[4], (uint32_t)f[5]};
    const uint32_t shb = f32_to_bf16(s);
    const uint32_t slb = f32_to_bf16(s - bf16_to_f32(shb));
    *reinterpret_cast<v2u*>(blk + 1536 + 8 * lane) = h == 0 ? v2u{shb | (slb << 16), shb} : v2u{slb, 0u};

    // (5) T partial of these 32 rows: the two column waves of the row band
    // are added through LDS (every wave reaches both barriers)
    if constexpr (RD4 > 0) {
      if (wn == 1) {
#pragma unroll
        for (int j4 = 0; j4 < RD4; ++j4)
#pragma unroll
          for (int i = 0; i < 16; ++i) xch[((wm * RD4 + j4) * 16 + i) * 64 + lane] = tacc[j4][i];
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (wn == 0) {
        float* tp = tpart + ((int64_t)tn * x_rt * 32 + m) * rank_dn;
#pragma unroll
        for (int j4 = 0; j4 < RD4; ++j4)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = 32 * j4 + 8 * q + 4 * h;  // ranks j .. j + 3
            if (j < rank_dn) {
              v4f v;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                v[e] = tacc[j4][4 * q + e] + xch[((wm * RD4 + j4) * 16 + 4 * q + e) * 64 + lane];
              *reinterpret_cast<v4f*>(tp + j) = v;
            }
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
}

// T of the down layer from the partial sums of the nt column tiles, added in
// tile order, written as the image's bf16 hi/lo blocks (and as fp32 T when T
// is not null); one thread per (row, 8 consecutive ranks).
__global__ __launch_bounds__(256) void fg_finish_t_kernel(int64_t M, int64_t rows, int rank, int nt,
                                                          const float* __restrict__ tpart,
                                                          uint8_t* __restrict__ dimg, size_t d_lr,
                                                          int64_t d_rt, float* __restrict__ T) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c8n = rank / 8;
  if (idx >= rows * c8n) return;
  const int64_t m = idx / c8n;
  const int c8 = (int)(idx - m * c8n);
  const float* tp = tpart + m * rank + 8 * c8;
  v4f a = *reinterpret_cast<const v4f*>(tp), b = *reinterpret_cast<const v4f*>(tp + 4);
  for (int t = 1; t < nt; ++t) {
    const float* q = tp + (int64_t)t * rows * rank;
    const v4f x = *reinterpret_cast<const v4f*>(q), y = *reinterpret_cast<const v4f*>(q + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] += x[i];
      b[i] += y[i];
    }
  }
  if (T != nullptr && m < M) {
    *reinterpret_cast<v4f*>(T + m * rank + 8 * c8) = a;
    *reinterpret_cast<v4f*>(T + m * rank + 8 * c8 + 4) = b;
  }
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    hi[i] = h0 | (h1 << 16);
    lo[i] = f32_to_bf16(v[2 * i] - bf16_to_f32(h0)) | (f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1)) << 16);
  }
  uint8_t* blk = dimg + d_lr + ((int64_t)(c8 >> 1) * d_rt + (m >> 5)) * LR_XBLOCK;
  const int slot = 32 * (c8 & 1) + (int)(m & 31);
  *reinterpret_cast<v4u*>(blk + 16 * slot) = v4u{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<v4u*>(blk + 1024 + 16 * slot) = v4u{lo[0], lo[1], lo[2], lo[3]};
}

size_t gelu_quantize_workspace_bytes(int64_t M, int N_up, int rank_dn) {
  const ActImage a = act_image(0, M, 64, 0);
  return (size_t)(N_up / FG_BN) * (size_t)(a.RT * 32) * (size_t)rank_dn * 4;
}

hipError_t launch_gelu_quantize(int64_t M, int N, int K, int rank_up, const void* ximage,
                                const void* wimage, int rank_dn, const float* lambda_dn,
                                const uint16_t* lora_dn, void* dimage, uint16_t* Y, float* T,
                                void* workspace, hipStream_t s) {
  const ActImage a = act_image(0, M, K, rank_up);
  const WeightImage w = weight_image(0, N, K, rank_up);
  const ActImage d = act_image(0, M, N, rank_dn);
  const int64_t tiles = (a.RT / (FG_BM / 32)) * (N / FG_BN);
  const uint8_t* xi = reinterpret_cast<const uint8_t*>(ximage);
  const uint8_t* wi = reinterpret_cast<const uint8_t*>(wimage);
  uint8_t* di = reinterpret_cast<uint8_t*>(dimage);
  float* tp = reinterpret_cast<float*>(workspace);
  const int rd4 = (rank_dn + 31) / 32;
#define SVDQ_FG_CASE(R)                                                                           \
  case R:                                                                                         \
    hipLaunchKernelGGL((fg_gemm_kernel<R>), dim3((unsigned)tiles), dim3(FG_THREADS), 0, s, M, N, \
                       K, rank_up, xi, a.RT, (int64_t)a.lr, wi, w.CT, (int64_t)w.lr,            \
                       (int64_t)w.bias, rank_dn, lambda_dn, lora_dn, di, d.RT, tp, Y);           \
    break;
  switch (rd4) {
    SVDQ_FG_CASE(0) SVDQ_FG_CASE(1) SVDQ_FG_CASE(2) SVDQ_FG_CASE(3) SVDQ_FG_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef SVDQ_FG_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rank_dn == 0) return e;
  const int64_t n = d.RT * 32 * (rank_dn / 8);
  hipLaunchKernelGGL(fg_finish_t_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, M,
                     d.RT * 32, rank_dn, (int)(N / FG_BN), tp, di, d.lr, d.RT, T);
  return hipGetLastError();
}

}  // namespace svdq
