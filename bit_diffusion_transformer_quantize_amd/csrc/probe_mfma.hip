// Measurement aid, built as its own library (libsvdq_probe.so) and used only
// by the benchmark: the dense matrix rate this GPU sustains for one MFMA
// instruction, and the shader clock while it does, so that the "fraction of
// peak" of the layer's kernels can be read against both the published peak
// and the rate measured on the same box; and the compute floor of the INT4
// GEMM's K loop (int4_group_kernel below).
//
// Every wave of a grid of `wgs` workgroups x 8 waves (two per SIMD) issues
// `iters` x 6 independent MFMAs of one kind back to back (six accumulator
// chains, so the matrix pipe is never idle on a dependency), and records its
// elapsed s_memtime (the shader clock) and its start and end s_memrealtime
// (a constant 100 MHz counter common to the whole GPU).  The host takes the
// FLOP/s over the span from the first wave's start to the last wave's end
// (the launch itself excluded) and the clock from the memtime/realtime
// ratio.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(512) void probe_kernel(int iters, float* sink,
                                                    unsigned long long* ticks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v8i a, b;
  v8bf ha, hb;
  for (int i = 0; i < 8; ++i) {
    a[i] = (lane * 7 + i * 13) & 0x0f0f0f0f;
    b[i] = (lane * 5 + i * 3) & 0x0f0f0f0f;
    ha[i] = (__bf16)(0.001f * (lane + i));
    hb[i] = (__bf16)(0.002f * (lane - i));
  }
  v16f acc[6];
  v16i iacc[6];
  for (int t = 0; t < 6; ++t)
    for (int i = 0; i < 16; ++i) {
      acc[t][i] = 0.f;
      iacc[t][i] = 0;
    }
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    a[0] ^= it & 1;  // keeps the instructions in the loop
#pragma unroll
    for (int t = 0; t < 6; ++t) {
      if constexpr (KIND == 0)  // FP6 (E2M3), 32x32x64, the INT4 path's product
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[t], 2, 2, 0, 127, 0, 127);
      else if constexpr (KIND == 1)  // FP4 (E2M1), 32x32x64
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[t], 4, 4, 0, 127, 0, 127);
      else if constexpr (KIND == 2)  // bf16 32x32x16
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha, hb, acc[t], 0, 0, 0);
      else  // int8 32x32x32
        iacc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a.lo, b.lo, iacc[t], 0, 0, 0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int t = 0; t < 6; ++t)
    for (int i = 0; i < 16; ++i) s += acc[t][i] + (float)iacc[t][i];
  sink[blockIdx.x * 512 + threadIdx.x] = s;
  if (lane == 0) {
    ticks[(blockIdx.x * 8 + wave) * 3] = t1 - t0;
    ticks[(blockIdx.x * 8 + wave) * 3 + 1] = r0;
    ticks[(blockIdx.x * 8 + wave) * 3 + 2] = r1;
  }
}

// The compute of one 64-group of the INT4 GEMM's K loop, as one wave of its
// 256 x 192 workgroup tile does it (2 x 3 tiles of 32 x 32, eight waves, two
// per SIMD), looped `iters` times without memory traffic:
//   mode 0: the six FP6 32x32x64 products P alone;
//   mode 1: the six bf16 32x32x8 scale outer products S alone;
//   mode 2: the 96 fp32 FMAs acc += P * S alone;
//   mode 3: all of it in the kernel's order: P and S of tile t + 1 issued
//           between the two halves of tile t's FMAs.
// One iteration is one group-stage of the workgroup tile per SIMD, so the
// K loop's compute floor is (group-stages per workgroup) x (time per
// iteration).  Timing as for probe_kernel.
typedef short v4s __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(512) void int4_group_kernel(int iters, float* sink,
                                                         unsigned long long* ticks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v8i af[2], bf[3];
  v4s sa[2], sb[3];
  for (int r = 0; r < 2; ++r) {
    for (int i = 0; i < 8; ++i) af[r][i] = (lane * 7 + i * 13 + r * 5) & 0x0f0f0f0f;
    for (int i = 0; i < 4; ++i) sa[r][i] = (short)(0x3f80 + ((lane + i + r) & 7));
  }
  for (int c = 0; c < 3; ++c) {
    for (int i = 0; i < 8; ++i) bf[c][i] = (lane * 5 + i * 3 + c * 11) & 0x0f0f0f0f;
    for (int i = 0; i < 4; ++i) sb[c][i] = (short)(0x3f80 + ((lane * 3 + i + c) & 7));
  }
  v16f zero, acc[6], p[2], sc[2];
  for (int i = 0; i < 16; ++i) zero[i] = 0.f;
  for (int t = 0; t < 6; ++t) acc[t] = zero;
  for (int t = 0; t < 2; ++t)
    for (int i = 0; i < 16; ++i) {
      p[t][i] = 1e-3f * (float)(i + t + lane);
      sc[t][i] = 1e-3f * (float)(i - t);
    }
  auto P = [&](int t, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[t % 3], af[t / 3], c, 2, 2, 0, 130, 0, 130);
  };
  auto Sm = [&](int t, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sb[t % 3], sa[t / 3], c, 0, 0, 0);
  };
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    af[0][0] ^= it & 1;  // keeps the instructions in the loop
    af[1][0] ^= it & 1;
    sa[0][0] ^= (short)(it & 1);
    sa[1][0] ^= (short)(it & 1);
    if constexpr (MODE == 0) {
#pragma unroll
      for (int t = 0; t < 6; ++t) acc[t] = P(t, acc[t]);
    } else if constexpr (MODE == 1) {
#pragma unroll
      for (int t = 0; t < 6; ++t) acc[t] = Sm(t, acc[t]);
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int t = 0; t < 6; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = fmaf(p[t & 1][i], sc[t & 1][i], acc[t][i]);
      p[0][0] += 1.f;
    } else {
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        const int n = (t + 1) % 6;
        p[n & 1] = P(n, zero);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t][i] = fmaf(p[t & 1][i], sc[t & 1][i], acc[t][i]);
        __builtin_amdgcn_sched_barrier(0);
        sc[n & 1] = Sm(n, zero);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 8; i < 16; ++i) acc[t][i] = fmaf(p[t & 1][i], sc[t & 1][i], acc[t][i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int t = 0; t < 6; ++t)
    for (int i = 0; i < 16; ++i) s += acc[t][i];
  for (int t = 0; t < 2; ++t)
    for (int i = 0; i < 16; ++i) s += p[t][i] + sc[t][i];
  sink[blockIdx.x * 512 + threadIdx.x] = s;
  if (lane == 0) {
    ticks[(blockIdx.x * 8 + wave) * 3] = t1 - t0;
    ticks[(blockIdx.x * 8 + wave) * 3 + 1] = r0;
    ticks[(blockIdx.x * 8 + wave) * 3 + 2] = r1;
  }
}

}  // namespace

extern "C" {

// kind: 0 FP6 32x32x64, 1 FP4 32x32x64, 2 bf16 32x32x16, 3 int8 32x32x32.
// sink: device float [wgs * 512]; ticks: device uint64 [wgs * 8 * 3].
// Returns 0, or the HIP error of the launch.
int svdq_probe_mfma(int kind, int wgs, int iters, float* sink, unsigned long long* ticks,
                    void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_kernel<0>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    case 1: hipLaunchKernelGGL(probe_kernel<1>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    case 2: hipLaunchKernelGGL(probe_kernel<2>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    case 3: hipLaunchKernelGGL(probe_kernel<3>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// mode 0..3 as int4_group_kernel; buffers as for svdq_probe_mfma.
int svdq_probe_int4_group(int mode, int wgs, int iters, float* sink, unsigned long long* ticks,
                          void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL(int4_group_kernel<0>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    case 1: hipLaunchKernelGGL(int4_group_kernel<1>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    case 2: hipLaunchKernelGGL(int4_group_kernel<2>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    case 3: hipLaunchKernelGGL(int4_group_kernel<3>, dim3(wgs), dim3(512), 0, s, iters, sink, ticks); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Flops of one MFMA of the kind (2 x M x N x K).
double svdq_probe_mfma_flops(int kind) {
  switch (kind) {
    case 0: case 1: return 2.0 * 32 * 32 * 64;
    case 2: return 2.0 * 32 * 32 * 16;
    case 3: return 2.0 * 32 * 32 * 32;
  }
  return 0.0;
}

}  // extern "C"
