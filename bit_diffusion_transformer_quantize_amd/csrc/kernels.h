// Host-side launchers of the gfx950 kernels (internal to libsvdq).  Every
// launcher assumes its arguments were validated by the C-ABI layer and
// returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

hipError_t launch_calibrate_lambda(int64_t M, int K, int N, const uint16_t* X,
                                   const uint16_t* W, float* lambda, hipStream_t s);

hipError_t launch_pack_weight(int mode, int rank, int N, int K, const uint16_t* W,
                              const float* lambda, const uint16_t* lora_down,
                              const uint16_t* lora_up, uint8_t* wcodes, void* wscales,
                              hipStream_t s);

hipError_t launch_quantize_act(int mode, int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down,
                               uint8_t* xcodes, void* xscales, float* T, hipStream_t s);

hipError_t launch_lowrank_down(int rank, int64_t M, int K, const uint16_t* X,
                               const float* lambda, const uint16_t* lora_down, float* T,
                               hipStream_t s);

// Device workspace the forward needs: the activation operand image.
size_t int4_workspace_bytes(int64_t M, int K);
size_t fp4_workspace_bytes(int64_t M, int K);

// Bytes of the prepared (kernel-layout) weight of each mode, and the
// launchers that build it from packed codes and scales.
size_t int4_weight_image_bytes(int N, int K);
size_t fp4_weight_image_bytes(int N, int K);
hipError_t launch_int4_prepare_weight(int N, int K, const uint8_t* wcodes, const float* wscales,
                                      void* wimage, hipStream_t s);
hipError_t launch_fp4_prepare_weight(int N, int K, const uint8_t* wcodes, const uint8_t* wscales,
                                     void* wimage, hipStream_t s);

hipError_t launch_int4_forward(int rank, bool out_f32, int64_t M, int N, int K,
                               const uint8_t* xcodes, const float* xscales, const float* T,
                               const void* wimage, const uint16_t* lora_up,
                               const uint16_t* bias, void* Y, void* workspace, hipStream_t s);

hipError_t launch_fp4_forward(int rank, bool out_f32, int64_t M, int N, int K,
                              const uint8_t* xcodes, const uint8_t* xscales, const float* T,
                              const void* wimage, const uint16_t* lora_up, const uint16_t* bias,
                              void* Y, void* workspace, hipStream_t s);

hipError_t launch_lowrank_up(int rank, bool out_f32, int64_t M, int N, const float* T,
                             const uint16_t* lora_up, void* Y, hipStream_t s);

}  // namespace svdq
