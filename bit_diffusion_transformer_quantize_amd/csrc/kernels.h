// Host-side launchers of the gfx950 kernels (internal to libsvdq).  Every
// launcher assumes its arguments were validated by the C-ABI layer and
// returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

hipError_t launch_calibrate_lambda(int64_t M, int K, int N, const uint16_t* X,
                                   const uint16_t* W, float* lambda, hipStream_t s);

// Per-column absolute maxima of a bf16 [R][K] matrix, optionally combined
// with amax; lambda from two such maxima.
hipError_t launch_column_absmax(int64_t R, int K, const uint16_t* A, float* amax, bool accumulate,
                                hipStream_t s);
hipError_t launch_lambda_from_absmax(int K, const float* xmax, const float* wmax, float* lambda,
                                     hipStream_t s);

hipError_t launch_pack_weight(int mode, int rank, int N, int K, const uint16_t* W,
                              const float* lambda, const uint16_t* lora_down,
                              const uint16_t* lora_up, uint8_t* wcodes, void* wscales,
                              hipStream_t s);

// Bytes of the operand images (layouts in image.h).
size_t act_image_bytes(int mode, int64_t M, int K, int rank);
size_t weight_image_bytes(int mode, int N, int K, int rank);

// Any of xcodes (with xscales), T and ximage may be null.
hipError_t launch_quantize_act(int mode, int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down,
                               uint8_t* xcodes, void* xscales, float* T, void* ximage,
                               bool gelu, hipStream_t s);

hipError_t launch_lowrank_down(int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down, float* T,
                               bool gelu, hipStream_t s);

// The activation image from the row-major codes, scales and T (T null when
// rank == 0); the partial-sum region is not written.
hipError_t launch_act_image_from_codes(int mode, int64_t M, int K, int rank, const uint8_t* xcodes,
                                       const void* xscales, const float* T, void* ximage,
                                       hipStream_t s);

hipError_t launch_prepare_weight(int mode, int N, int K, int rank, const uint8_t* wcodes,
                                 const void* wscales, const uint16_t* lora_up,
                                 const uint16_t* bias, void* wimage, hipStream_t s);

hipError_t launch_int4_forward(bool out_f32, int64_t M, int N, int K, int rank,
                               const void* ximage, const void* wimage, void* Y, hipStream_t s);
hipError_t launch_fp4_forward(bool out_f32, int64_t M, int N, int K, int rank,
                              const void* ximage, const void* wimage, void* Y, hipStream_t s);

hipError_t launch_lowrank_up(int rank, bool out_f32, int64_t M, int N, const float* T,
                             const uint16_t* lora_up, void* Y, hipStream_t s);

// AWQ W4A16 (awq.hip).
hipError_t launch_awq_pack(int N, int K, const uint16_t* W, uint8_t* codes, float* scales,
                           uint8_t* zeros, hipStream_t s);
hipError_t launch_awq_linear(bool out_f32, int64_t M, int N, int K, const uint16_t* X,
                             const uint8_t* codes, const float* scales, const uint8_t* zeros,
                             const uint16_t* bias, void* Y, hipStream_t s);

// Q/K RMSNorm + rotary embedding of the QKV output, in place (qk_norm_rope.hip).
hipError_t launch_qk_norm_rope(int64_t M, int heads, int64_t ld, uint16_t* Y, const uint16_t* q_scale,
                               const uint16_t* k_scale, const float* cosv, const float* sinv,
                               float eps, hipStream_t s);

// NVFP4 variant.  The activation pass is the mode-2 quantize_act_kernel
// (quantize_act.hip: codes, scale bytes and, when rank > 0, T = X_hat L1 from
// the same registers); the rest is nvfp4.hip.
hipError_t launch_nvfp4_quantize_act(int64_t M, int K, int rank, const uint16_t* X,
                                     const float* lambda, const float* g,
                                     const uint16_t* lora_down, uint8_t* xcodes, uint8_t* xscales,
                                     float* T, hipStream_t s);
hipError_t launch_nvfp4_scale_from_absmax(int n, const float* amax, float* g, hipStream_t s);
hipError_t launch_nvfp4_pack_weight(int N, int K, int rank, const uint16_t* W, const float* lambda,
                                    const uint16_t* lora_down, const uint16_t* lora_up,
                                    uint8_t* codes, uint8_t* scales, float* g, hipStream_t s);
hipError_t launch_nvfp4_linear(bool out_f32, int64_t M, int N, int K, int rank,
                               const uint8_t* xcodes, const uint8_t* xscales, const float* gx,
                               const uint8_t* wcodes, const uint8_t* wscales, const float* gw,
                               const float* T, const uint16_t* lora_up, const uint16_t* bias,
                               void* Y, hipStream_t s);

// The MLP up-projection with the down layer's activation pass fused into
// its epilogue (gemm_int4_gelu.hip).
size_t gelu_quantize_workspace_bytes(int64_t M, int N_up, int rank_dn);
hipError_t launch_gelu_quantize(int64_t M, int N, int K, int rank_up, const void* ximage,
                                const void* wimage, int rank_dn, const float* lambda_dn,
                                const uint16_t* lora_dn, void* dimage, uint16_t* Y, float* T,
                                void* workspace, hipStream_t s);

// Randomized truncated SVD of the smoothed weight (lowrank_factors.hip).
size_t lowrank_factors_workspace_bytes(int N, int K, int rank);
// Size of the static workspace of svdq_lowrank_factors_noalloc (64 MiB), and
// the current device's copy of it.
constexpr size_t LOWRANK_STATIC_WORKSPACE = size_t(64) << 20;
hipError_t lowrank_static_workspace(void** ptr);
hipError_t launch_lowrank_factors(int N, int K, int rank, const uint16_t* W, const float* lambda,
                                  uint64_t seed, int power_iters, uint16_t* lora_down,
                                  uint16_t* lora_up, double* sigma, void* workspace,
                                  hipStream_t s);

// Compute units of the current device (cached per device).
int device_cus();

}  // namespace svdq
