// Device-side helpers shared by the gfx950 kernels of libsvdq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// v_mfma_scale_f32_32x32x64_f8f6f4 with each operand as wide as its format
// reads: 4 registers of E2M1 codes, 6 of E2M3.  clang's builtin takes 8 for
// every format, so a narrower fragment would be padded with registers the
// instruction never reads; the LLVM intrinsic is overloaded on the operand
// width.  Arguments: A, B, C, format of A, format of B, A scale selector,
// A scales (E8M0, one byte per lane), B scale selector, B scales.
extern "C" __device__ v16f svdq_mfma_scale_e2m1(v4i a, v4i b, v16f c, int fmt_a, int fmt_b,
                                                int sel_a, int scale_a, int sel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");
extern "C" __device__ v16f svdq_mfma_scale_e2m3(v6i a, v6i b, v16f c, int fmt_a, int fmt_b,
                                                int sel_a, int scale_a, int sel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v6i32.v6i32");

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even.  Inputs here are
// finite; NaN is not special-cased.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> one dword of two bf16 (lo in bits 0..15), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// INT4 code of v for a nonzero scale s: clamp(rint(fp32(v / s)), -8, 7).
// The division is the IEEE-correctly-rounded fp32 quotient.
__device__ __forceinline__ int int4_code(float v, float s) {
  float q = __builtin_rintf(v / s);
  q = fminf(fmaxf(q, -8.0f), 7.0f);
  return (int)q;
}

// E2M1 magnitude index (0..7) of |y| < 8: nearest grid point of
// {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even index, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_index(float a) {
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return c;
}

// 4-bit E2M1 sign-magnitude code of y (sign taken from the sign bit, so -0
// keeps it).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  return e2m1_index(fabsf(y)) | ((__float_as_uint(y) >> 28) & 8u);
}

// E8M0 exponent for a block with absolute maximum a >= 0:
// e = clamp(floor(log2 a) - 2, -127, 127), e = -127 for a == 0.  floor(log2 a)
// is read from the exponent field; any a below 2^-125 clamps to -127.
__device__ __forceinline__ int e8m0_exponent(float a) {
  int eb = (int)((__float_as_uint(a) >> 23) & 0xFFu);
  if (eb == 0) return -127;
  int e = eb - 127 - 2;
  return e < -127 ? -127 : e;
}

// 2^k as fp32 for -126 <= k <= 127.
__device__ __forceinline__ float exp2i(int k) {
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// Nibble unpack of 8 two's-complement int4 codes (one dword, element 2j in
// the low nibble of byte j) into int8 lanes holding 16*q: `even` gets the
// even elements, `odd` the odd ones.  Products of two such bytes carry a
// factor 256, removed with the scale.
__device__ __forceinline__ void int4x8_to_int8x16(uint32_t w, uint32_t& even, uint32_t& odd) {
  even = (w << 4) & 0xF0F0F0F0u;
  odd = w & 0xF0F0F0F0u;
}

// Eight two's-complement int4 codes (one dword, element 2j in the low nibble
// of byte j) -> eight e4m3 bytes that hold q * 2^-9 exactly.  In e4m3 the
// subnormal range is linear: byte |q| (0..8, exponent field 0 or 1) is
// |q| * 2^-9, and bit 7 is the sign, so the byte is the sign-magnitude form of
// q.  For a nibble value x (0..15) that is x when x < 8 and 0x90 - x
// otherwise.  `even` receives elements 0,2,4,6 and `odd` elements 1,3,5,7.
// The per-byte "x >= 8" masks come from v_perm_b32, whose selectors 8..11
// replicate the top bit of bytes 1, 3, 5, 7 of its 64-bit source.
__device__ __forceinline__ void int4x8_to_fp8x8(uint32_t w, uint32_t& even, uint32_t& odd) {
  const uint32_t xe = w & 0x0F0F0F0Fu;
  const uint32_t xo = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t ue = w << 4;  // bit 3 of each byte -> bit 7
  const uint32_t me = __builtin_amdgcn_perm(ue << 8, ue, 0x090B080Au);
  const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  even = ((0x90909090u - xe) & me) | (xe & ~me);
  odd = ((0x90909090u - xo) & mo) | (xo & ~mo);
}

// 16 int4 codes (two dwords) -> 16 e4m3 bytes {even(w0), even(w1), odd(w0),
// odd(w1)}: the 16-byte chunk layout both operands of the INT4 GEMM use.
__device__ __forceinline__ v4u int4x16_to_fp8x16(uint32_t w0, uint32_t w1) {
  uint32_t e0, o0, e1, o1;
  int4x8_to_fp8x8(w0, e0, o0);
  int4x8_to_fp8x8(w1, e1, o1);
  return v4u{e0, e1, o0, o1};
}

// 32 int4 codes (16 bytes) -> two such 16-byte chunks.
__device__ __forceinline__ void int4x32_to_fp8x32(const v4u& w, v4u& lo, v4u& hi) {
  lo = int4x16_to_fp8x16(w[0], w[1]);
  hi = int4x16_to_fp8x16(w[2], w[3]);
}

}  // namespace svdq
