// AWQ W4A16 linear layer: 4-bit weights with per-(row, 64-group) scale and
// zero point, 16-bit activations (page "Nunchaku Lite ..." on axbrief.com,
// sections "The Mechanics of 4-Bit Efficiency and SVDQuant" and "The
// Trade-off Between Fused Kernels and Generality": the layer type assigned to
// modulation linears).  Two kernels:
//   awq_pack_kernel  -- offline: bf16 W -> codes, scales, zero points, every
//                       step one IEEE fp32 operation (bit-exact).
//   awq_gemv_kernel  -- run time, small M (a batch of modulation vectors):
//                       Y = X deq(W)^T + b, HBM-bound on the packed weight.
//
// GEMV design.  Each wave owns R consecutive output rows; lane l takes the
// 16-code units l, l+64, l+128 of a K-slab of 3072 codes, so one wave-wide
// 8-byte load reads 512 contiguous code bytes.  The activations of the slab
// stay in VGPRs as bf16 pairs for all R rows.  A unit's codes become bf16
// pairs (128 + q) with one AND/shift and a byte permute that inserts the
// exponent byte 0x43, and v_dot2c_f32_bf16 forms
//   A = sum (128 + q_k) x_k,   B = sum x_k   (B once per slab and lane),
// so a unit adds s * (A - (128 + z) B) = s * sum (q_k - z) x_k.  The products
// of bf16 pairs are exact; A and B carry fp32 rounding only.  Partial sums of
// the R rows x MC batch rows are reduced across the wave by halving the set
// of values at each exchange step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kAwqGroup = 64;
constexpr int kAwqRows = 4;     // output rows per wave
constexpr int kAwqUnits = 3;    // 16-code units per lane per slab
constexpr int kAwqWaves = 4;    // waves per workgroup
constexpr int kAwqSlabUnits = 64 * kAwqUnits;

// ---------------------------------------------------------------- packing --
// One thread per (row, group): min and max of the 64 weights, then
//   d = max(fp32(max - min), 1e-5), s = fp32(d / 15),
//   z = clamp(rint(fp32(-min / s)), 0, 15),
//   q = clamp(rint(fp32(w / s)) + z, 0, 15)   (rint: ties to even).
__global__ __launch_bounds__(256) void awq_pack_kernel(int N, int K, const uint16_t* __restrict__ W,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros) {
  const int G = K / kAwqGroup;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * G) return;
  const int64_t row = idx / G;
  const int g = (int)(idx - row * G);
  const v4u* src = reinterpret_cast<const v4u*>(W + row * K + (int64_t)g * kAwqGroup);
  v4u w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = src[i];
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_to_f32(w[i][j] & 0xFFFFu), b = bf16_to_f32(w[i][j] >> 16);
      mx = fmaxf(mx, fmaxf(a, b));
      mn = fminf(mn, fminf(a, b));
    }
  const float d = fmaxf(mx - mn, 1e-5f);
  const float s = d / 15.0f;
  const float z = fminf(fmaxf(__builtin_rintf(-mn / s), 0.0f), 15.0f);
  v4u out[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_to_f32(w[i][j] & 0xFFFFu), b = bf16_to_f32(w[i][j] >> 16);
      const float qa = fminf(fmaxf(__builtin_rintf(a / s) + z, 0.0f), 15.0f);
      const float qb = fminf(fmaxf(__builtin_rintf(b / s) + z, 0.0f), 15.0f);
      packed |= ((uint32_t)qa | ((uint32_t)qb << 4)) << (8 * j);
    }
    out[i >> 2][i & 3] = packed;
  }
  v4u* dst = reinterpret_cast<v4u*>(codes + row * (K / 2) + (int64_t)g * (kAwqGroup / 2));
  dst[0] = out[0];
  dst[1] = out[1];
  scales[idx] = s;
  zeros[idx] = (uint8_t)z;
}

// ------------------------------------------------------------------- GEMV --
// Eight bf16 activations (one dword pair per two) reordered to match the code
// pairs below: (x0, x2), (x4, x6), (x1, x3), (x5, x7).
__device__ __forceinline__ v4u awq_reorder_x(const v4u& x) {
  v4u r;
  r[0] = __builtin_amdgcn_perm(x[1], x[0], 0x05040100u);  // x0 | x2
  r[1] = __builtin_amdgcn_perm(x[3], x[2], 0x05040100u);  // x4 | x6
  r[2] = __builtin_amdgcn_perm(x[1], x[0], 0x07060302u);  // x1 | x3
  r[3] = __builtin_amdgcn_perm(x[3], x[2], 0x07060302u);  // x5 | x7
  return r;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b),
                                         c, false);
}

// Eight codes (one dword, element 2j in the low nibble of byte j) as bf16
// pairs 128 + q in the order of awq_reorder_x.
__device__ __forceinline__ v4u awq_codes_bf16(uint32_t w) {
  constexpr uint32_t kExp = 0x43434343u;
  const uint32_t ev = w & 0x0F0F0F0Fu;          // q0 q2 q4 q6
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // q1 q3 q5 q7
  v4u r;
  r[0] = __builtin_amdgcn_perm(kExp, ev, 0x04010400u);
  r[1] = __builtin_amdgcn_perm(kExp, ev, 0x04030402u);
  r[2] = __builtin_amdgcn_perm(kExp, od, 0x04010400u);
  r[3] = __builtin_amdgcn_perm(kExp, od, 0x04030402u);
  return r;
}

// Sum of V values over the 64 lanes of a wave.  At each exchange step a lane
// keeps half of its values and adds the partner's copy of them, so the whole
// set costs V - 1 + (6 - log2 V) exchanges.  Afterwards v[0] of lane l holds
// the total of value index l >> (6 - log2 V).
template <int V>
__device__ __forceinline__ void wave_reduce_set(float (&v)[V], int lane) {
  int bit = 5;
#pragma unroll
  for (int n = V; n > 1; n >>= 1, --bit) {
    const bool hi = (lane >> bit) & 1;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float keep = hi ? v[i + n / 2] : v[i];
      const float send = hi ? v[i] : v[i + n / 2];
      v[i] = keep + __shfl_xor(send, 1 << bit, 64);
    }
  }
#pragma unroll
  for (; bit >= 0; --bit) v[0] += __shfl_xor(v[0], 1 << bit, 64);
}

// The weight side of RB rows for this lane's U units: codes, scales and
// zero points, issued row by row so that a row's arithmetic can start while
// later rows are still arriving (loads retire in issue order).
template <int RB>
struct AwqBlock {
  v2u w[RB][kAwqUnits];
  float s[RB][kAwqUnits];
  // zero points and bias stay in their memory widths: a loop-carried value
  // widened at the load would make the loop wait for the prefetched block
  uint8_t z[RB][kAwqUnits];
  uint16_t b[RB];   // bf16 bias of the rows (raw; ignored without bias)
};

template <int RB, bool WITH_BIAS>
__device__ __forceinline__ void awq_load_block(AwqBlock<RB>& bk, int row0, int N, int K, int G,
                                               const int (&gu)[kAwqUnits],
                                               const uint8_t* __restrict__ codes,
                                               const float* __restrict__ scales,
                                               const uint8_t* __restrict__ zeros,
                                               const uint16_t* __restrict__ bias) {
  // without a bias the (ignored) value is read from the zero points, which
  // hold at least 2N bytes, so that the load needs no branch
  const uint16_t* bsrc = bias != nullptr ? bias : reinterpret_cast<const uint16_t*>(zeros);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int64_t row = min(row0 + r, N - 1);
    if constexpr (WITH_BIAS) bk.b[r] = bsrc[row];
#pragma unroll
    for (int u = 0; u < kAwqUnits; ++u)
      bk.w[r][u] = __builtin_nontemporal_load(
          reinterpret_cast<const v2u*>(codes + row * (K / 2) + (int64_t)gu[u] * 8));
#pragma unroll
    for (int u = 0; u < kAwqUnits; ++u) {
      bk.s[r][u] = scales[row * G + (gu[u] >> 2)];
      bk.z[r][u] = zeros[row * G + (gu[u] >> 2)];
    }
  }
}

// Activations of this lane's units for MC batch rows: raw loads, then the
// reordered bf16 pairs and their sums (zero for units past K and rows past M).
template <int MC>
struct AwqAct {
  v4u raw[kAwqUnits][MC][2];
  v4u xp[kAwqUnits][MC][2];
  float xs[kAwqUnits][MC];
};

template <int MC>
__device__ __forceinline__ void awq_load_act(AwqAct<MC>& ac, int m0, int M, int K,
                                             const int (&gu)[kAwqUnits],
                                             const uint16_t* __restrict__ X) {
#pragma unroll
  for (int u = 0; u < kAwqUnits; ++u)
#pragma unroll
    for (int mi = 0; mi < MC; ++mi) {
      const int m = min(m0 + mi, M - 1);
      const v4u* src = reinterpret_cast<const v4u*>(X + (int64_t)m * K + (int64_t)gu[u] * 16);
      ac.raw[u][mi][0] = src[0];
      ac.raw[u][mi][1] = src[1];
    }
}

template <int MC>
__device__ __forceinline__ void awq_prep_act(AwqAct<MC>& ac, int m0, int M,
                                             const bool (&valid)[kAwqUnits]) {
#pragma unroll
  for (int u = 0; u < kAwqUnits; ++u)
#pragma unroll
    for (int mi = 0; mi < MC; ++mi) {
      const bool live = valid[u] && m0 + mi < M;
      v4u a = ac.raw[u][mi][0], b = ac.raw[u][mi][1];
      if (!live) a = b = v4u{0u, 0u, 0u, 0u};
      ac.xp[u][mi][0] = awq_reorder_x(a);
      ac.xp[u][mi][1] = awq_reorder_x(b);
      float t = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t = dot2(a[j], 0x3F803F80u, t);
        t = dot2(b[j], 0x3F803F80u, t);
      }
      ac.xs[u][mi] = t;
    }
}

// acc[r][mi] += sum over this lane's units of s * (A - (128 + z) B).
template <int RB, int MC>
__device__ __forceinline__ void awq_block_dot(const AwqBlock<RB>& bk, const AwqAct<MC>& ac,
                                              float (&acc)[RB * MC]) {
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int u = 0; u < kAwqUnits; ++u) {
      const v4u c0 = awq_codes_bf16(bk.w[r][u][0]);
      const v4u c1 = awq_codes_bf16(bk.w[r][u][1]);
      // 128 + z as fp32: z in the mantissa bits 16..19 of 128.0f
      const float off = __uint_as_float(0x43000000u | ((uint32_t)bk.z[r][u] << 16));
#pragma unroll
      for (int mi = 0; mi < MC; ++mi) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a = dot2(c0[j], ac.xp[u][mi][0][j], a);
          a = dot2(c1[j], ac.xp[u][mi][1][j], a);
        }
        acc[r * MC + mi] = fmaf(bk.s[r][u], fmaf(-off, ac.xs[u][mi], a), acc[r * MC + mi]);
      }
    }
}

// Wave-wide sums of acc, plus the bias, stored by one lane per output.
// The bias comes either from the block's loads (brow, streaming kernel) or,
// with brow == nullptr, is read here after all other loads have landed.
template <int RB, int MC, bool F32>
__device__ __forceinline__ void awq_store(float (&acc)[RB * MC], const uint16_t* brow,
                                          const uint16_t* __restrict__ bias, int lane, int row0,
                                          int m0, int M, int N, void* __restrict__ Y) {
  wave_reduce_set<RB * MC>(acc, lane);
  constexpr int kShift = 6 - __builtin_ctz(RB * MC);
  const int idx = lane >> kShift;
  float bv = 0.0f;
  if (brow != nullptr) {
    uint32_t bsel = brow[0];
#pragma unroll
    for (int r = 1; r < RB; ++r) bsel = idx / MC == r ? (uint32_t)brow[r] : bsel;
    bv = bias != nullptr ? bf16_to_f32(bsel) : 0.0f;
  }
  const int row = row0 + idx / MC, m = m0 + idx % MC;
  if ((lane & ((1 << kShift) - 1)) != 0 || row >= N || m >= M) return;
  if (brow == nullptr && bias != nullptr) bv = bf16_to_f32(bias[row]);
  const float y = acc[0] + bv;
  if constexpr (F32)
    reinterpret_cast<float*>(Y)[(int64_t)m * N + row] = y;
  else
    reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + row] = (uint16_t)f32_to_bf16(y);
}

__device__ __forceinline__ void awq_units(int slab, int lane, int KU, int (&gu)[kAwqUnits],
                                          bool (&valid)[kAwqUnits]) {
#pragma unroll
  for (int u = 0; u < kAwqUnits; ++u) {
    const int unit = slab * kAwqSlabUnits + u * 64 + lane;
    valid[u] = unit < KU;
    gu[u] = valid[u] ? unit : KU - 1;   // clamped; its activations are zero
  }
}

// General K: one block of kAwqRows rows per wave, K in slabs of 3072 codes.
template <int MC, bool F32>
__global__ __launch_bounds__(kAwqWaves * 64) void awq_gemv_kernel(
    int M, int N, int K, const uint16_t* __restrict__ X, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint8_t* __restrict__ zeros,
    const uint16_t* __restrict__ bias, void* __restrict__ Y) {
  constexpr int R = kAwqRows;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kAwqWaves + wave) * R;
  if (row0 >= N) return;
  const int m0 = blockIdx.y * MC;
  const int KU = K / 16;   // 16-code units per row
  const int G = K / kAwqGroup;
  const int nslab = (KU + kAwqSlabUnits - 1) / kAwqSlabUnits;

  float acc[R * MC];
#pragma unroll
  for (int i = 0; i < R * MC; ++i) acc[i] = 0.0f;
  for (int slab = 0; slab < nslab; ++slab) {
    int gu[kAwqUnits];
    bool valid[kAwqUnits];
    awq_units(slab, lane, KU, gu, valid);
    // every load of the slab before any arithmetic: activations (cache hits)
    // first, then the weight side; the scheduling barrier keeps the compiler
    // from sinking loads to their first use
    AwqAct<MC> ac;
    AwqBlock<R> bk;
    awq_load_act<MC>(ac, m0, M, K, gu, X);
    awq_load_block<R, false>(bk, row0, N, K, G, gu, codes, scales, zeros, bias);
    __builtin_amdgcn_sched_barrier(0);
    awq_prep_act<MC>(ac, m0, M, valid);
    awq_block_dot<R, MC>(bk, ac, acc);
  }
  awq_store<R, MC, F32>(acc, nullptr, bias, lane, row0, m0, M, N, Y);
}

// K <= 3072 (one slab): each wave streams row blocks of RB rows, block
// w, w + W, w + 2W, ... (W = waves in the grid), with the activations held in
// registers throughout and the next block's loads in flight while the current
// block is computed.  Two register sets alternate; the loop is unrolled by two
// so that no set is copied while its loads are outstanding.
template <int MC, bool F32, int RB>
__global__ __launch_bounds__(kAwqWaves * 64) void awq_gemv_stream_kernel(
    int M, int N, int K, const uint16_t* __restrict__ X, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint8_t* __restrict__ zeros,
    const uint16_t* __restrict__ bias, void* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int nblk = (N + RB - 1) / RB;
  const int stride = gridDim.x * kAwqWaves;
  int blk = blockIdx.x * kAwqWaves + (threadIdx.x >> 6);
  if (blk >= nblk) return;
  const int m0 = blockIdx.y * MC;
  const int KU = K / 16;
  const int G = K / kAwqGroup;
  int gu[kAwqUnits];
  bool valid[kAwqUnits];
  awq_units(0, lane, KU, gu, valid);

  AwqAct<MC> ac;
  AwqBlock<RB> b0, b1;
  awq_load_act<MC>(ac, m0, M, K, gu, X);
  awq_load_block<RB, true>(b0, blk * RB, N, K, G, gu, codes, scales, zeros, bias);
  __builtin_amdgcn_sched_barrier(0);
  awq_prep_act<MC>(ac, m0, M, valid);

  auto finish = [&](const AwqBlock<RB>& bk, int b) {
    float acc[RB * MC];
#pragma unroll
    for (int i = 0; i < RB * MC; ++i) acc[i] = 0.0f;
    awq_block_dot<RB, MC>(bk, ac, acc);
    awq_store<RB, MC, F32>(acc, bk.b, bias, lane, b * RB, m0, M, N, Y);
  };
  // The prefetch is unconditional so that the wait counts are exact on every
  // path: past the last block it re-reads the block being computed (a cache
  // hit); each block's arithmetic appears once per loop body, so the
  // compiler cannot hoist it above the prefetch.
#pragma nounroll
  for (;;) {
    const int n1 = blk + stride;
    awq_load_block<RB, true>(b1, (n1 < nblk ? n1 : blk) * RB, N, K, G, gu, codes, scales, zeros, bias);
    __builtin_amdgcn_sched_barrier(0);
    finish(b0, blk);
    if (n1 >= nblk) break;
    blk = n1;
    const int n2 = blk + stride;
    awq_load_block<RB, true>(b0, (n2 < nblk ? n2 : blk) * RB, N, K, G, gu, codes, scales, zeros, bias);
    __builtin_amdgcn_sched_barrier(0);
    finish(b1, blk);
    if (n2 >= nblk) break;
    blk = n2;
  }
}

constexpr int kAwqStreamRows = 2;   // rows per block of the streaming kernel

// Resident workgroups per CU of the streaming kernel (from its register
// use), so that the grid is exactly one wave of workgroups.
template <int MC, bool F32>
int stream_wg_per_cu() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, awq_gemv_stream_kernel<MC, F32, kAwqStreamRows>, kAwqWaves * 64, 0) != hipSuccess)
      n = 1;
    v = std::max(1, n);
    cached.store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int MC, bool F32>
void launch_gemv_t(int64_t M, int N, int K, const uint16_t* X, const uint8_t* codes,
                   const float* scales, const uint8_t* zeros, const uint16_t* bias, void* Y,
                   hipStream_t s) {
  const unsigned gy = (unsigned)((M + MC - 1) / MC);
  // The streaming kernel wins once its waves have several blocks each, or
  // with a batch (more arithmetic per byte); a single-row GEMV of moderate
  // N is latency-bound and runs fastest with every block's loads issued at
  // once by the one-shot kernel.
  const int64_t nblk = (N + kAwqStreamRows - 1) / kAwqStreamRows;
  const int64_t resident = (int64_t)device_cus() * stream_wg_per_cu<MC, F32>();
  if (K <= kAwqSlabUnits * 16 && (MC > 1 || nblk > 8 * resident * kAwqWaves)) {
    const int64_t wgs = (nblk + kAwqWaves - 1) / kAwqWaves;
    const dim3 grid((unsigned)std::min(wgs, resident), gy);
    awq_gemv_stream_kernel<MC, F32, kAwqStreamRows><<<grid, kAwqWaves * 64, 0, s>>>(
        (int)M, N, K, X, codes, scales, zeros, bias, Y);
  } else {
    const dim3 grid((unsigned)((N + kAwqWaves * kAwqRows - 1) / (kAwqWaves * kAwqRows)), gy);
    awq_gemv_kernel<MC, F32><<<grid, kAwqWaves * 64, 0, s>>>((int)M, N, K, X, codes, scales,
                                                             zeros, bias, Y);
  }
}

template <int MC>
hipError_t launch_gemv(bool f32, int64_t M, int N, int K, const uint16_t* X,
                       const uint8_t* codes, const float* scales, const uint8_t* zeros,
                       const uint16_t* bias, void* Y, hipStream_t s) {
  if (f32)
    launch_gemv_t<MC, true>(M, N, K, X, codes, scales, zeros, bias, Y, s);
  else
    launch_gemv_t<MC, false>(M, N, K, X, codes, scales, zeros, bias, Y, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_awq_pack(int N, int K, const uint16_t* W, uint8_t* codes, float* scales,
                           uint8_t* zeros, hipStream_t s) {
  const int64_t threads = (int64_t)N * (K / kAwqGroup);
  awq_pack_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(N, K, W, codes, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_awq_linear(bool out_f32, int64_t M, int N, int K, const uint16_t* X,
                             const uint8_t* codes, const float* scales, const uint8_t* zeros,
                             const uint16_t* bias, void* Y, hipStream_t s) {
  if (M == 1) return launch_gemv<1>(out_f32, M, N, K, X, codes, scales, zeros, bias, Y, s);
  if (M == 2) return launch_gemv<2>(out_f32, M, N, K, X, codes, scales, zeros, bias, Y, s);
  return launch_gemv<4>(out_f32, M, N, K, X, codes, scales, zeros, bias, Y, s);
}

}  // namespace svdq
