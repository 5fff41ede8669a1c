// E4M3 block-scale bytes of the NVFP4 format (E2M1 codes in blocks of 16
// along K, one FP8 E4M3 scale per block, one fp32 scale per tensor; NVIDIA's
// published layout, the FP4 format the Nunchaku Lite page on axbrief.com
// names in "The Mechanics of 4-Bit Efficiency and SVDQuant"), shared by the
// activation pass and the NVFP4 weight packer and GEMM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

// Byte of E4M3_RNE_sat(v) for v >= 0: nearest value of the E4M3 grid
// (normals (1 + m/8) 2^e for e = -6..8, subnormals m 2^-9), ties to the even
// mantissa, 448 for everything from 448 up.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);  // 0..8 (8 = 2^-6)
  const uint32_t b = __float_as_uint(v);
  int e = (int)(b >> 23) - 127;
  uint32_t q = (b >> 20) & 7u;
  const uint32_t rem = b & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
  if (q == 8u) {
    q = 0;
    ++e;
  }
  const uint32_t byte = ((uint32_t)(e + 7) << 3) | q;
  return byte > 0x7Eu ? 0x7Eu : byte;
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

}  // namespace svdq
