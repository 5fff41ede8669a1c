// Pieces shared by the W4A4 GEMM kernels: the 32x32 MFMA accumulator
// layout, the bf16 split of T, the bias and the output store.
#pragma once

#include "common.h"

namespace svdq {

// 32x32 MFMA accumulator layout (same for the i8, bf16 and f8f6f4 forms):
// lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}


// Eight fp32 values -> their bf16 high parts and bf16 low parts (of the
// fp32 remainder), both RNE (v_cvt_pk_bf16_f32): hi + lo is within 2^-16
// relative of the value.
__device__ __forceinline__ void split_bf16x8(const v4f& a, const v4f& b, v8bf& hi, v8bf& lo) {
  const float t[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const v2f x = {t[2 * j], t[2 * j + 1]};
    const v2bf h = __builtin_convertvector(x, v2bf);
    const v2f hf = __builtin_convertvector(h, v2f);
    const v2f r = {x[0] - hf[0], x[1] - hf[1]};
    const v2bf l = __builtin_convertvector(r, v2bf);
    hi[2 * j] = h[0];
    hi[2 * j + 1] = h[1];
    lo[2 * j] = l[0];
    lo[2 * j + 1] = l[1];
  }
}

// s_waitcnt immediate that waits for vector memory count <= n (gfx9
// encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt not waited on).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert(vmcnt_imm(4) == 0x0F74 && vmcnt_imm(24) == 0x4F78, "vmcnt encoding");

// Transposed accumulator: with the weight as the A operand and the
// activations as the B operand of the 32x32 MFMAs, lane l, element i of tile
// (tr, tc) holds output row mbase + 32 tr + l%32 and output column
// nbase + 32 tc + acc_row(i, l): each quad of elements covers four
// consecutive columns.
//
// Y[rows, cols] = acc for such tiles, bf16 (RNE) or fp32; rows >= M and
// 8-column chunks at or past N are skipped (N is a multiple of 8, so a chunk
// is entirely inside or outside).  bf16: the quads of the two lane halves
// are exchanged with v_permlane32_swap so that every lane holds and stores 8
// consecutive columns (16 bytes); fp32: every quad is one 16-byte store.
// The two 16-byte bf16 quads a lane stores for one transposed 32x32 tile:
// o[qp] holds columns 16 qp + 8 (lane/32) .. +7 of row lane%32 (RNE).
__device__ __forceinline__ void tile_quads_bf16(const v16f& a, v4u (&o)[2]) {
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const v2f x = {a[2 * j], a[2 * j + 1]};
    pk[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
  }
#pragma unroll
  for (int qp = 0; qp < 2; ++qp) {
    // quads 2 qp (dwords 4 qp, +1) and 2 qp + 1 (dwords 4 qp + 2, +3)
    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * qp], pk[4 * qp + 2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * qp + 1], pk[4 * qp + 3], false, false);
    o[qp] = v4u{s0[0], s1[0], s0[1], s1[1]};
  }
}

template <int TR, int TC, bool FULL>
__device__ __forceinline__ void store_tiles_t_as(const v16f (&acc)[TR][TC], int64_t M, int N,
                                                 int64_t mbase, int nbase, int lane, bool out_f32,
                                                 void* __restrict__ Y) {
  // the lane-dependent addresses are formed here, not hoisted into the
  // caller's loops where they would hold registers across the main loop
  asm volatile("" : "+v"(lane));
  const int h = lane >> 5;
#pragma unroll
  for (int tr = 0; tr < TR; ++tr) {
    const int64_t m = mbase + tr * 32 + (lane & 31);
    const bool mok = FULL || m < M;
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      const int n0 = nbase + tc * 32;
      if (out_f32) {
        float* yr = reinterpret_cast<float*>(Y) + m * N + n0 + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4f v = {acc[tr][tc][4 * q], acc[tr][tc][4 * q + 1], acc[tr][tc][4 * q + 2],
                         acc[tr][tc][4 * q + 3]};
          if (FULL || (mok && n0 + 8 * q < N)) *reinterpret_cast<v4f*>(yr + 8 * q) = v;
        }
      } else {
        uint16_t* yr = reinterpret_cast<uint16_t*>(Y) + m * N + n0;
        v4u o[2];
        tile_quads_bf16(acc[tr][tc], o);
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          const int c = 16 * qp + 8 * h;
          if (FULL || (mok && n0 + c < N)) *reinterpret_cast<v4u*>(yr + c) = o[qp];
        }
      }
    }
  }
}

template <int TR, int TC>
__device__ __forceinline__ void store_tiles_t(const v16f (&acc)[TR][TC], int64_t M, int N,
                                              int64_t mbase, int nbase, int lane, bool out_f32,
                                              void* __restrict__ Y) {
  if (mbase + TR * 32 <= M && nbase + TC * 32 <= N)  // wave-uniform
    store_tiles_t_as<TR, TC, true>(acc, M, N, mbase, nbase, lane, out_f32, Y);
  else
    store_tiles_t_as<TR, TC, false>(acc, M, N, mbase, nbase, lane, out_f32, Y);
}

// acc[tr][tc] = the bias of the columns a transposed accumulator holds, from
// a run of bf16 bias values in LDS whose first entry is column nbase.
template <int TR, int TC>
__device__ __forceinline__ void init_bias_t(v16f (&acc)[TR][TC], const uint8_t* bias_run,
                                            int lane) {
  asm volatile("" : "+v"(lane));
  const int h = lane >> 5;
#pragma unroll
  for (int tc = 0; tc < TC; ++tc)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v2u w = *reinterpret_cast<const v2u*>(bias_run + 2 * (32 * tc + 8 * q + 4 * h));
      const float b[4] = {bf16_to_f32(w[0] & 0xFFFFu), bf16_to_f32(w[0] >> 16),
                          bf16_to_f32(w[1] & 0xFFFFu), bf16_to_f32(w[1] >> 16)};
#pragma unroll
      for (int tr = 0; tr < TR; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tr][tc][4 * q + e] = b[e];
    }
}

}  // namespace svdq
