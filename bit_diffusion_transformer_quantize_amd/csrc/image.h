// Operand images: the layouts in which the GEMM kernels read both sides of
// the layer.  The activation image is written by svdq_quantize_act, the
// weight image ("prepared weight") by svdq_prepare_weight; the GEMM copies
// contiguous runs of them into LDS with global->LDS DMA and reads MFMA
// fragments lane-linearly.  All blocks are in MFMA lane order: lane l of a
// 32-row tile holds row l%32 and the K half (or rank half) l/32.
//
// Activation image (rows padded to a multiple of 256, padding rows zero):
//   INT4  code blocks  [G][RT][2048]   (G = K/64 groups, RT = Mp/32)
//           [0, 768)     K half 0: 16-byte heads at 16 r, 8-byte tails at
//                        512 + 8 r (the 32 6-bit E2M3 fields of row r)
//           [768, 1536)  K half 1, same layout
//           [1536, 2048) 8-byte bf16 scale operand per lane (X pattern)
//   FP4   code blocks  [G][RT][1024]   (lane l: 16 bytes of E2M1 codes)
//         scale blocks [G][RT][64]     (lane l: one E8M0 byte)
//   both  low-rank blocks (rank r > 0) [r/16][RT][2048]: per 16-rank slice,
//         64 lanes x 8 bf16 of hi(T) at 16 l, then 64 lanes x 8 bf16 of
//         lo(T) at 1024 + 16 l (lane l: row l%32, ranks 8 (l/32) .. +7).
//         partial sums (r > 0 and S > 1) [S][RT*32][r] fp32: the writing
//         pass splits K into S ranges of whole 64-groups (act_splits) and
//         a second pass adds the S partial T rows in order.
//
// Weight image (columns padded to the GEMM's tile width, padding zero):
//   INT4  code blocks [G][CT][2048] as above with the W scale pattern
//   FP4   code blocks [G][CT][1024], scale blocks [G][CT][64]
//   both  low-rank blocks (r > 0) [r/16][CT][1024]: lane l: column l%32,
//         8 bf16 of L2 for ranks 8 (l/32) .. +7 of the slice
//         bias blocks [CT][64]: 32 bf16 per 32-column tile (zero without a
//         bias), followed by 1024 bytes of zero padding (a DMA of one
//         workgroup's bias run may read past the last tile).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

constexpr int IMG_ROWS_PAD = 256;        // activation rows: multiple of 256
constexpr int I4_COLS_PAD = 192;         // INT4 weight columns: multiple of 192
constexpr int F4_COLS_PAD = 256;         // FP4 weight columns: multiple of 256
constexpr int I4_BLOCK = 2048;           // INT4 code block
constexpr int F4_CBLOCK = 1024;          // FP4 code block
constexpr int F4_SBLOCK = 64;            // FP4 scale block
constexpr int LR_XBLOCK = 2048;          // T hi + lo per (slice, 32 rows)
constexpr int LR_WBLOCK = 1024;          // L2 per (slice, 32 columns)
constexpr int BIAS_BLOCK = 64;           // 32 bf16
constexpr int BIAS_TAIL = 1024;          // zero padding after the bias blocks

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// K ranges of the pass that writes the activation image: enough (16 rows,
// K range) work items to fill the GPU (about 1024), each range at least 48
// whole 64-groups (so that every wave of a workgroup has several), at most
// 16 ranges.
__host__ __device__ inline int act_splits(int64_t M, int K) {
  const int64_t blocks = round_up(M, IMG_ROWS_PAD) / 16;
  int64_t s = (1024 + blocks - 1) / blocks;
  const int64_t by_k = (K / 64) / 48;
  s = s > by_k ? by_k : s;
  return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}

struct ActImage {
  int64_t RT;              // 32-row tiles (padded rows / 32)
  int S;                   // K ranges of the writing pass
  size_t code;             // offset of the code blocks (0)
  size_t scale;            // FP4: offset of the scale blocks
  size_t lr;               // offset of the low-rank blocks
  size_t tpart;            // offset of the partial T sums (r > 0 and S > 1)
  size_t bytes;            // total size
};

__host__ __device__ inline ActImage act_image(int mode, int64_t M, int K, int rank) {
  ActImage a;
  const int64_t G = K / 64;
  a.RT = round_up(M, IMG_ROWS_PAD) / 32;
  a.S = act_splits(M, K);
  a.code = 0;
  if (mode == 0) {
    a.scale = 0;
    a.lr = (size_t)(G * a.RT * I4_BLOCK);
  } else {
    a.scale = (size_t)(G * a.RT * F4_CBLOCK);
    a.lr = a.scale + (size_t)(G * a.RT * F4_SBLOCK);
  }
  a.tpart = a.lr + (size_t)(rank / 16) * (size_t)a.RT * LR_XBLOCK;
  a.bytes = a.tpart + (rank > 0 && a.S > 1 ? (size_t)a.S * (size_t)a.RT * 32 * rank * 4 : 0);
  return a;
}

struct WeightImage {
  int64_t CT;              // 32-column tiles (padded columns / 32)
  size_t code, scale, lr, bias, bytes;
};

__host__ __device__ inline WeightImage weight_image(int mode, int N, int K, int rank) {
  WeightImage w;
  const int64_t G = K / 64;
  w.CT = round_up(N, mode == 0 ? I4_COLS_PAD : F4_COLS_PAD) / 32;
  w.code = 0;
  if (mode == 0) {
    w.scale = 0;
    w.lr = (size_t)(G * w.CT * I4_BLOCK);
  } else {
    w.scale = (size_t)(G * w.CT * F4_CBLOCK);
    w.lr = w.scale + (size_t)(G * w.CT * F4_SBLOCK);
  }
  w.bias = w.lr + (size_t)(rank / 16) * (size_t)w.CT * LR_WBLOCK;
  w.bytes = w.bias + (size_t)w.CT * BIAS_BLOCK + BIAS_TAIL;
  return w;
}

}  // namespace svdq
