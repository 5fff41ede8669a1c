// C ABI of libsvdq: argument validation (before any HIP call), the gfx950
// capability check, and the kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/svdq.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

svdq_status check_desc(const svdq_desc* d) {
  if (d == nullptr) return SVDQ_ERR_ARG;
  if (d->mode != SVDQ_MODE_INT4 && d->mode != SVDQ_MODE_FP4) return SVDQ_ERR_ARG;
  if ((d->flags & ~(SVDQ_FLAG_OUT_F32 | SVDQ_FLAG_GELU_IN)) != 0u) return SVDQ_ERR_ARG;
  if (d->K <= 0 || d->K % 128 != 0 || d->K > (1 << 20)) return SVDQ_ERR_SHAPE;
  if (d->N <= 0 || d->N % 128 != 0 || d->N > (1 << 20)) return SVDQ_ERR_SHAPE;
  if (d->rank < 0 || d->rank > 256 || d->rank % 16 != 0) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

#define SVDQ_TRY_INNER(expr)           \
  do {                                 \
    const svdq_status st_ = (expr);    \
    if (st_ != SVDQ_OK) return st_;    \
  } while (0)

svdq_status check_rows(int64_t M) {
  if (M < 1 || M > (int64_t(1) << 31)) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

// Activation tensors are limited to 2^36 elements (kernels index 32-code
// chunks with 32-bit integers).
svdq_status check_rows_k(int64_t M, int32_t K) {
  SVDQ_TRY_INNER(check_rows(M));
  if (M * (int64_t)K > (int64_t(1) << 36)) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

// The images handed to the GEMM must be exactly the sizes the descriptor and
// M give (the kernels address them from desc and M alone, so this bounds
// every access to the bytes the caller owns).
svdq_status check_images(const svdq_desc* d, int64_t M, size_t ximage_bytes, size_t wimage_bytes) {
  if (ximage_bytes != svdq::act_image_bytes(d->mode, M, d->K, d->rank)) return SVDQ_ERR_ARG;
  if (wimage_bytes != svdq::weight_image_bytes(d->mode, d->N, d->K, d->rank)) return SVDQ_ERR_ARG;
  return SVDQ_OK;
}

// Required pointer: non-null and 16-byte aligned.
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
// Optional pointer: null, or 16-byte aligned.
bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }

svdq_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SVDQ_ERR_HIP;
  if (dev < 0) return SVDQ_ERR_HIP;
  if (dev < kMaxDevices) {
    const int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return SVDQ_OK;
    if (st == 2) return SVDQ_ERR_ARCH;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SVDQ_ERR_HIP;
  const bool ok = svdq_arch_supported(prop.gcnArchName) != 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? SVDQ_OK : SVDQ_ERR_ARCH;
}

svdq_status from_hip(hipError_t e) { return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP; }

#define SVDQ_TRY(expr)                 \
  do {                                 \
    const svdq_status st_ = (expr);    \
    if (st_ != SVDQ_OK) return st_;    \
  } while (0)

}  // namespace

extern "C" {

const char* svdq_status_string(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_ERR_ARG: return "SVDQ_ERR_ARG: null or misaligned pointer, or bad mode/flags";
    case SVDQ_ERR_SHAPE: return "SVDQ_ERR_SHAPE: size outside the supported limits";
    case SVDQ_ERR_ARCH: return "SVDQ_ERR_ARCH: current device is not gfx950";
    case SVDQ_ERR_HIP: return "SVDQ_ERR_HIP: HIP runtime error";
  }
  return "SVDQ_ERR_UNKNOWN";
}

int svdq_arch_supported(const char* name) {
  if (name == nullptr) return 0;
  if (std::strncmp(name, "gfx950", 6) != 0) return 0;
  const char c = name[6];
  return (c == '\0' || c == ':') ? 1 : 0;
}

const char* svdq_version(void) { return "0.1.0"; }

svdq_status svdq_calibrate_lambda(int64_t M, int32_t K, int32_t N, const uint16_t* X,
                                  const uint16_t* W, float* lambda, void* stream) {
  if (!ptr_ok(X) || !ptr_ok(W) || !ptr_ok(lambda)) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_rows(M));
  if (N < 1 || N > (1 << 24) || K <= 0 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_calibrate_lambda(M, K, N, X, W, lambda, (hipStream_t)stream));
}

svdq_status svdq_calibrate_absmax(int64_t R, int32_t K, const uint16_t* A, float* amax,
                                  int32_t accumulate, void* stream) {
  if (!ptr_ok(A) || !ptr_ok(amax)) return SVDQ_ERR_ARG;
  if (accumulate != 0 && accumulate != 1) return SVDQ_ERR_ARG;
  if (R < 1 || R > (int64_t(1) << 31) || K <= 0 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_column_absmax(R, K, A, amax, accumulate != 0, (hipStream_t)stream));
}

svdq_status svdq_lambda_from_absmax(int32_t K, const float* xmax, const float* wmax, float* lambda,
                                    void* stream) {
  if (!ptr_ok(xmax) || !ptr_ok(wmax) || !ptr_ok(lambda)) return SVDQ_ERR_ARG;
  if (K <= 0 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_lambda_from_absmax(K, xmax, wmax, lambda, (hipStream_t)stream));
}

svdq_status svdq_pack_weight(const svdq_desc* d, const uint16_t* W, const float* lambda,
                             const uint16_t* lora_down, const uint16_t* lora_up,
                             uint8_t* wcodes, void* wscales, void* stream) {
  SVDQ_TRY(check_desc(d));
  if (!ptr_ok(W) || !ptr_ok(lambda) || !ptr_ok(wcodes) || !ptr_ok(wscales)) return SVDQ_ERR_ARG;
  if (d->rank > 0) {
    if (!ptr_ok(lora_down) || !ptr_ok(lora_up)) return SVDQ_ERR_ARG;
  } else if (lora_down != nullptr || lora_up != nullptr) {
    return SVDQ_ERR_ARG;
  }
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_pack_weight(d->mode, d->rank, d->N, d->K, W, lambda, lora_down,
                                           lora_up, wcodes, wscales, (hipStream_t)stream));
}

namespace {
svdq_status check_factor_shape(int32_t N, int32_t K, int32_t rank) {
  if (N < 128 || N % 128 != 0 || N > (1 << 20)) return SVDQ_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  if ((int64_t)N * K > (int64_t(1) << 32)) return SVDQ_ERR_SHAPE;
  if (rank < 16 || rank > 128 || rank % 16 != 0) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}
}  // namespace

svdq_status svdq_lowrank_factors_workspace(int32_t N, int32_t K, int32_t rank, size_t* bytes) {
  SVDQ_TRY(check_factor_shape(N, K, rank));
  if (bytes == nullptr) return SVDQ_ERR_ARG;
  *bytes = svdq::lowrank_factors_workspace_bytes(N, K, rank);
  return SVDQ_OK;
}

svdq_status svdq_lowrank_factors(int32_t N, int32_t K, int32_t rank, const uint16_t* W,
                                 const float* lambda, uint64_t seed, int32_t power_iters,
                                 uint16_t* lora_down, uint16_t* lora_up, double* sigma,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  SVDQ_TRY(check_factor_shape(N, K, rank));
  if (power_iters < 0 || power_iters > 8) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(W) || !ptr_ok(lambda) || !ptr_ok(lora_down) || !ptr_ok(lora_up) || !opt_ok(sigma))
    return SVDQ_ERR_ARG;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SVDQ_ERR_ARG;
  if (workspace_bytes < svdq::lowrank_factors_workspace_bytes(N, K, rank)) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_lowrank_factors(N, K, rank, W, lambda, seed, power_iters, lora_down,
                                               lora_up, sigma, workspace, (hipStream_t)stream));
}

svdq_status svdq_lowrank_factors_noalloc(int32_t N, int32_t K, int32_t rank, const uint16_t* W,
                                         const float* lambda, uint64_t seed, int32_t power_iters,
                                         uint16_t* lora_down, uint16_t* lora_up, double* sigma,
                                         void* stream) {
  SVDQ_TRY(check_factor_shape(N, K, rank));
  if (power_iters < 0 || power_iters > 8) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(W) || !ptr_ok(lambda) || !ptr_ok(lora_down) || !ptr_ok(lora_up) || !opt_ok(sigma))
    return SVDQ_ERR_ARG;
  if (svdq::lowrank_factors_workspace_bytes(N, K, rank) > svdq::LOWRANK_STATIC_WORKSPACE)
    return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  void* ws = nullptr;
  SVDQ_TRY(from_hip(svdq::lowrank_static_workspace(&ws)));
  return from_hip(svdq::launch_lowrank_factors(N, K, rank, W, lambda, seed, power_iters, lora_down,
                                               lora_up, sigma, ws, (hipStream_t)stream));
}

svdq_status svdq_act_image_size(const svdq_desc* d, int64_t M, size_t* bytes) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (bytes == nullptr) return SVDQ_ERR_ARG;
  *bytes = svdq::act_image_bytes(d->mode, M, d->K, d->rank);
  return SVDQ_OK;
}

svdq_status svdq_quantize_act(const svdq_desc* d, int64_t M, const uint16_t* X,
                              const float* lambda, const uint16_t* lora_down, uint8_t* xcodes,
                              void* xscales, float* T, void* ximage, size_t ximage_bytes,
                              void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (!ptr_ok(X) || !ptr_ok(lambda)) return SVDQ_ERR_ARG;
  if (ximage_bytes != (ximage == nullptr ? 0 : svdq::act_image_bytes(d->mode, M, d->K, d->rank)))
    return SVDQ_ERR_ARG;
  if ((xcodes == nullptr) != (xscales == nullptr)) return SVDQ_ERR_ARG;
  if (!opt_ok(xcodes) || !opt_ok(xscales) || !opt_ok(T) || !opt_ok(ximage)) return SVDQ_ERR_ARG;
  if (xcodes == nullptr && T == nullptr && ximage == nullptr) return SVDQ_ERR_ARG;
  if (d->rank == 0) {
    if (lora_down != nullptr || T != nullptr) return SVDQ_ERR_ARG;
  } else {
    // the low-rank part of the image and T both come from lora_down
    if ((T != nullptr || ximage != nullptr) && !ptr_ok(lora_down)) return SVDQ_ERR_ARG;
    if (T == nullptr && ximage == nullptr && lora_down != nullptr) return SVDQ_ERR_ARG;
  }
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_quantize_act(d->mode, d->rank, M, d->K, X, lambda, lora_down,
                                            xcodes, xscales, T, ximage,
                                            (d->flags & SVDQ_FLAG_GELU_IN) != 0u,
                                            (hipStream_t)stream));
}

svdq_status svdq_weight_image_size(const svdq_desc* d, size_t* bytes) {
  SVDQ_TRY(check_desc(d));
  if (bytes == nullptr) return SVDQ_ERR_ARG;
  *bytes = svdq::weight_image_bytes(d->mode, d->N, d->K, d->rank);
  return SVDQ_OK;
}

svdq_status svdq_prepare_weight(const svdq_desc* d, const uint8_t* wcodes, const void* wscales,
                                const uint16_t* lora_up, const uint16_t* bias, void* wimage,
                                size_t wimage_bytes, void* stream) {
  SVDQ_TRY(check_desc(d));
  if (!ptr_ok(wcodes) || !ptr_ok(wscales) || !ptr_ok(wimage) || !opt_ok(bias)) return SVDQ_ERR_ARG;
  if (wimage_bytes != svdq::weight_image_bytes(d->mode, d->N, d->K, d->rank)) return SVDQ_ERR_ARG;
  if (d->rank > 0 ? !ptr_ok(lora_up) : lora_up != nullptr) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_prepare_weight(d->mode, d->N, d->K, d->rank, wcodes, wscales,
                                              lora_up, bias, wimage, (hipStream_t)stream));
}

svdq_status svdq_linear_forward(const svdq_desc* d, int64_t M, const void* ximage,
                                size_t ximage_bytes, const void* wimage, size_t wimage_bytes,
                                void* Y, void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  // outputs are limited to 2^46 elements (tile counts stay 32-bit)
  if (M > (int64_t(1) << 46) / d->N) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(ximage) || !ptr_ok(wimage) || !ptr_ok(Y)) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_images(d, M, ximage_bytes, wimage_bytes));
  const bool f32 = (d->flags & SVDQ_FLAG_OUT_F32) != 0u;
  SVDQ_TRY(check_device());
  if (d->mode == SVDQ_MODE_INT4)
    return from_hip(svdq::launch_int4_forward(f32, M, d->N, d->K, d->rank, ximage, wimage, Y,
                                              (hipStream_t)stream));
  return from_hip(svdq::launch_fp4_forward(f32, M, d->N, d->K, d->rank, ximage, wimage, Y,
                                           (hipStream_t)stream));
}

svdq_status svdq_linear_forward_packed(const svdq_desc* d, int64_t M, const void* ximage,
                                       size_t ximage_bytes, const uint8_t* wcodes,
                                       const void* wscales, const uint16_t* lora_up,
                                       const uint16_t* bias, void* wscratch,
                                       size_t wscratch_bytes, void* Y, void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (M > (int64_t(1) << 46) / d->N) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(ximage) || !ptr_ok(wcodes) || !ptr_ok(wscales) || !ptr_ok(wscratch) ||
      !ptr_ok(Y) || !opt_ok(bias))
    return SVDQ_ERR_ARG;
  if (d->rank > 0 ? !ptr_ok(lora_up) : lora_up != nullptr) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_images(d, M, ximage_bytes, wscratch_bytes));
  const bool f32 = (d->flags & SVDQ_FLAG_OUT_F32) != 0u;
  SVDQ_TRY(check_device());
  const hipStream_t s = (hipStream_t)stream;
  SVDQ_TRY(from_hip(svdq::launch_prepare_weight(d->mode, d->N, d->K, d->rank, wcodes, wscales,
                                                lora_up, bias, wscratch, s)));
  if (d->mode == SVDQ_MODE_INT4)
    return from_hip(svdq::launch_int4_forward(f32, M, d->N, d->K, d->rank, ximage, wscratch, Y, s));
  return from_hip(svdq::launch_fp4_forward(f32, M, d->N, d->K, d->rank, ximage, wscratch, Y, s));
}

namespace {
// The row-major form's workspace: the activation image, then (at a 256-byte
// boundary) the prepared weight.
size_t rowmajor_xbytes(const svdq_desc* d, int64_t M) {
  return (svdq::act_image_bytes(d->mode, M, d->K, d->rank) + 255) / 256 * 256;
}
}  // namespace

svdq_status svdq_linear_rowmajor_workspace_size(const svdq_desc* d, int64_t M, size_t* bytes) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (bytes == nullptr) return SVDQ_ERR_ARG;
  *bytes = rowmajor_xbytes(d, M) + svdq::weight_image_bytes(d->mode, d->N, d->K, d->rank);
  return SVDQ_OK;
}

svdq_status svdq_linear_forward_rowmajor(const svdq_desc* d, int64_t M, const uint8_t* xcodes,
                                         const void* xscales, const float* T,
                                         const uint8_t* wcodes, const void* wscales,
                                         const uint16_t* lora_up, const uint16_t* bias, void* Y,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (M > (int64_t(1) << 46) / d->N) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(xcodes) || !ptr_ok(xscales) || !ptr_ok(wcodes) || !ptr_ok(wscales) ||
      !ptr_ok(Y) || !ptr_ok(workspace) || !opt_ok(bias))
    return SVDQ_ERR_ARG;
  if (d->rank > 0 ? (!ptr_ok(T) || !ptr_ok(lora_up)) : (T != nullptr || lora_up != nullptr))
    return SVDQ_ERR_ARG;
  const size_t xb = rowmajor_xbytes(d, M);
  if (workspace_bytes < xb + svdq::weight_image_bytes(d->mode, d->N, d->K, d->rank))
    return SVDQ_ERR_ARG;
  const bool f32 = (d->flags & SVDQ_FLAG_OUT_F32) != 0u;
  SVDQ_TRY(check_device());
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* ximage = reinterpret_cast<uint8_t*>(workspace);
  uint8_t* wimage = ximage + xb;
  SVDQ_TRY(from_hip(svdq::launch_act_image_from_codes(d->mode, M, d->K, d->rank, xcodes, xscales,
                                                      T, ximage, s)));
  SVDQ_TRY(from_hip(svdq::launch_prepare_weight(d->mode, d->N, d->K, d->rank, wcodes, wscales,
                                                lora_up, bias, wimage, s)));
  if (d->mode == SVDQ_MODE_INT4)
    return from_hip(svdq::launch_int4_forward(f32, M, d->N, d->K, d->rank, ximage, wimage, Y, s));
  return from_hip(svdq::launch_fp4_forward(f32, M, d->N, d->K, d->rank, ximage, wimage, Y, s));
}

namespace {
// An INT4 up layer feeding an INT4 down layer whose input is GELU of the up
// layer's output (down->K == up->N), down rank at most 128.
svdq_status check_mlp_pair(const svdq_desc* up, const svdq_desc* down) {
  SVDQ_TRY(check_desc(up));
  SVDQ_TRY(check_desc(down));
  if (up->mode != SVDQ_MODE_INT4 || down->mode != SVDQ_MODE_INT4) return SVDQ_ERR_ARG;
  if ((down->flags & SVDQ_FLAG_GELU_IN) == 0u) return SVDQ_ERR_ARG;
  if ((up->flags & SVDQ_FLAG_OUT_F32) != 0u) return SVDQ_ERR_ARG;
  if (down->K != up->N) return SVDQ_ERR_SHAPE;
  if (down->rank > 128) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}
}  // namespace

svdq_status svdq_gelu_quantize_workspace_size(const svdq_desc* up, int64_t M,
                                              const svdq_desc* down, size_t* bytes) {
  SVDQ_TRY(check_mlp_pair(up, down));
  SVDQ_TRY(check_rows_k(M, up->K));
  SVDQ_TRY(check_rows_k(M, down->K));
  if (bytes == nullptr) return SVDQ_ERR_ARG;
  *bytes = svdq::gelu_quantize_workspace_bytes(M, up->N, down->rank);
  return SVDQ_OK;
}

svdq_status svdq_linear_forward_gelu_quantize(const svdq_desc* up, int64_t M, const void* ximage,
                                              size_t ximage_bytes, const void* wimage,
                                              size_t wimage_bytes, const svdq_desc* down,
                                              const float* lambda_down, const uint16_t* lora_down,
                                              void* ximage_down, size_t ximage_down_bytes,
                                              uint16_t* Y, float* T, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  SVDQ_TRY(check_mlp_pair(up, down));
  SVDQ_TRY(check_rows_k(M, up->K));
  SVDQ_TRY(check_rows_k(M, down->K));
  if (M > (int64_t(1) << 46) / up->N) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(ximage) || !ptr_ok(wimage) || !ptr_ok(lambda_down) || !ptr_ok(ximage_down) ||
      !opt_ok(Y) || !opt_ok(T) || !opt_ok(workspace))
    return SVDQ_ERR_ARG;
  SVDQ_TRY(check_images(up, M, ximage_bytes, wimage_bytes));
  if (ximage_down_bytes != svdq::act_image_bytes(down->mode, M, down->K, down->rank))
    return SVDQ_ERR_ARG;
  if (down->rank > 0) {
    if (!ptr_ok(lora_down) || workspace == nullptr) return SVDQ_ERR_ARG;
  } else if (lora_down != nullptr || T != nullptr) {
    return SVDQ_ERR_ARG;
  }
  if (workspace_bytes < svdq::gelu_quantize_workspace_bytes(M, up->N, down->rank))
    return SVDQ_ERR_ARG;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_gelu_quantize(M, up->N, up->K, up->rank, ximage, wimage,
                                             down->rank, lambda_down, lora_down, ximage_down, Y,
                                             T, workspace, (hipStream_t)stream));
}

svdq_status svdq_lowrank_down(const svdq_desc* d, int64_t M, const uint16_t* X,
                              const float* lambda, const uint16_t* lora_down, float* T,
                              void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (d->rank == 0) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(X) || !ptr_ok(lambda) || !ptr_ok(lora_down) || !ptr_ok(T)) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_lowrank_down(d->rank, M, d->K, X, lambda, lora_down, T,
                                            (d->flags & SVDQ_FLAG_GELU_IN) != 0u,
                                            (hipStream_t)stream));
}

svdq_status svdq_lowrank_up(const svdq_desc* d, int64_t M, const float* T,
                            const uint16_t* lora_up, void* Y, void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (d->rank == 0) return SVDQ_ERR_SHAPE;
  if (!ptr_ok(T) || !ptr_ok(lora_up) || !ptr_ok(Y)) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_lowrank_up(d->rank, (d->flags & SVDQ_FLAG_OUT_F32) != 0u, M,
                                          d->N, T, lora_up, Y, (hipStream_t)stream));
}

namespace {
svdq_status check_qk(int64_t M, int32_t heads, int64_t ld, const void* Y, const void* q_scale,
                     const void* k_scale, const void* cos, const void* sin, float eps) {
  if (!ptr_ok(Y) || !ptr_ok(q_scale) || !ptr_ok(k_scale) || !ptr_ok(cos) || !ptr_ok(sin))
    return SVDQ_ERR_ARG;
  if (!(eps > 0.0f) || eps > 3.4e38f) return SVDQ_ERR_ARG;
  if (M < 1 || M > (int64_t(1) << 31) || heads < 1 || heads > 2048) return SVDQ_ERR_SHAPE;
  if (ld < (int64_t)2 * heads * 128 || ld > (int64_t(1) << 24) || ld % 8 != 0) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}
}  // namespace

svdq_status svdq_qk_norm_rope(int64_t M, int32_t heads, int64_t ld, uint16_t* Y,
                              const uint16_t* q_scale, const uint16_t* k_scale, const float* cos,
                              const float* sin, float eps, void* stream) {
  SVDQ_TRY(check_qk(M, heads, ld, Y, q_scale, k_scale, cos, sin, eps));
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_qk_norm_rope(M, heads, ld, Y, q_scale, k_scale, cos, sin, eps,
                                            (hipStream_t)stream));
}

svdq_status svdq_linear_forward_qk(const svdq_desc* d, int64_t M, const void* ximage,
                                   size_t ximage_bytes, const void* wimage, size_t wimage_bytes,
                                   int32_t heads, const uint16_t* q_scale,
                                   const uint16_t* k_scale, const float* cos, const float* sin,
                                   float eps, void* Y, void* stream) {
  SVDQ_TRY(check_desc(d));
  SVDQ_TRY(check_rows_k(M, d->K));
  if (M > (int64_t(1) << 46) / d->N) return SVDQ_ERR_SHAPE;
  if ((d->flags & SVDQ_FLAG_OUT_F32) != 0u) return SVDQ_ERR_ARG;
  if (!ptr_ok(ximage) || !ptr_ok(wimage)) return SVDQ_ERR_ARG;
  SVDQ_TRY(check_images(d, M, ximage_bytes, wimage_bytes));
  SVDQ_TRY(check_qk(M, heads, d->N, Y, q_scale, k_scale, cos, sin, eps));
  SVDQ_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  if (d->mode == SVDQ_MODE_FP4)
    SVDQ_TRY(from_hip(svdq::launch_fp4_forward(false, M, d->N, d->K, d->rank, ximage, wimage, Y, st)));
  else
    SVDQ_TRY(from_hip(svdq::launch_int4_forward(false, M, d->N, d->K, d->rank, ximage, wimage, Y, st)));
  return from_hip(svdq::launch_qk_norm_rope(M, heads, d->N, static_cast<uint16_t*>(Y), q_scale,
                                            k_scale, cos, sin, eps, st));
}

namespace {
svdq_status check_nv_shape(int64_t M, int32_t N, int32_t K, int32_t rank) {
  if (K < 128 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  if (N < 128 || N % 128 != 0 || N > (1 << 20)) return SVDQ_ERR_SHAPE;
  if (M < 1 || M > (int64_t(1) << 31) || M * (int64_t)K > (int64_t(1) << 36)) return SVDQ_ERR_SHAPE;
  if (rank < 0 || rank > 256 || rank % 16 != 0) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}
}  // namespace

svdq_status svdq_nvfp4_scale_from_absmax(int32_t n, const float* amax, float* g, void* stream) {
  if (!ptr_ok(amax) || !ptr_ok(g)) return SVDQ_ERR_ARG;
  if (n < 1) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_nvfp4_scale_from_absmax(n, amax, g, (hipStream_t)stream));
}

svdq_status svdq_nvfp4_quantize_act(int64_t M, int32_t K, int32_t rank, const uint16_t* X,
                                    const float* lambda, const float* g,
                                    const uint16_t* lora_down, uint8_t* xcodes, uint8_t* xscales,
                                    float* T, void* stream) {
  if (!ptr_ok(X) || !ptr_ok(lambda) || !ptr_ok(g) || !ptr_ok(xcodes) || !ptr_ok(xscales))
    return SVDQ_ERR_ARG;
  if (rank > 0 ? (!ptr_ok(lora_down) || !ptr_ok(T)) : (lora_down != nullptr || T != nullptr))
    return SVDQ_ERR_ARG;
  SVDQ_TRY(check_nv_shape(M, 128, K, rank));
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_nvfp4_quantize_act(M, K, rank, X, lambda, g, lora_down, xcodes,
                                                  xscales, T, (hipStream_t)stream));
}

svdq_status svdq_nvfp4_pack_weight(int32_t N, int32_t K, int32_t rank, const uint16_t* W,
                                   const float* lambda, const uint16_t* lora_down,
                                   const uint16_t* lora_up, uint8_t* wcodes, uint8_t* wscales,
                                   float* g, void* stream) {
  if (!ptr_ok(W) || !ptr_ok(lambda) || !ptr_ok(wcodes) || !ptr_ok(wscales) || !ptr_ok(g))
    return SVDQ_ERR_ARG;
  if (rank > 0 ? (!ptr_ok(lora_down) || !ptr_ok(lora_up))
               : (lora_down != nullptr || lora_up != nullptr))
    return SVDQ_ERR_ARG;
  SVDQ_TRY(check_nv_shape(1, N, K, rank));
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_nvfp4_pack_weight(N, K, rank, W, lambda, lora_down, lora_up,
                                                 wcodes, wscales, g, (hipStream_t)stream));
}

svdq_status svdq_nvfp4_linear(int64_t M, int32_t N, int32_t K, int32_t rank,
                              const uint8_t* xcodes, const uint8_t* xscales, const float* g_x,
                              const uint8_t* wcodes, const uint8_t* wscales, const float* g_w,
                              const float* T, const uint16_t* lora_up, const uint16_t* bias,
                              uint32_t flags, void* Y, void* stream) {
  if ((flags & ~SVDQ_FLAG_OUT_F32) != 0u) return SVDQ_ERR_ARG;
  if (!ptr_ok(xcodes) || !ptr_ok(xscales) || !ptr_ok(g_x) || !ptr_ok(wcodes) || !ptr_ok(wscales) ||
      !ptr_ok(g_w) || !ptr_ok(Y) || !opt_ok(bias))
    return SVDQ_ERR_ARG;
  if (rank > 0 ? (!ptr_ok(T) || !ptr_ok(lora_up)) : (T != nullptr || lora_up != nullptr))
    return SVDQ_ERR_ARG;
  SVDQ_TRY(check_nv_shape(M, N, K, rank));
  if (M > (int64_t(1) << 46) / N) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_nvfp4_linear((flags & SVDQ_FLAG_OUT_F32) != 0u, M, N, K, rank,
                                            xcodes, xscales, g_x, wcodes, wscales, g_w, T, lora_up,
                                            bias, Y, (hipStream_t)stream));
}

svdq_status svdq_awq_pack_weight(int32_t N, int32_t K, const uint16_t* W, uint8_t* codes,
                                 float* scales, uint8_t* zeros, void* stream) {
  if (!ptr_ok(W) || !ptr_ok(codes) || !ptr_ok(scales) || !ptr_ok(zeros)) return SVDQ_ERR_ARG;
  if (N < 1 || N > (1 << 24) || K < 128 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  if ((int64_t)N * K > (int64_t(1) << 36)) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_awq_pack(N, K, W, codes, scales, zeros, (hipStream_t)stream));
}

svdq_status svdq_awq_linear(int64_t M, int32_t N, int32_t K, const uint16_t* X,
                            const uint8_t* codes, const float* scales, const uint8_t* zeros,
                            const uint16_t* bias, uint32_t flags, void* Y, void* stream) {
  if ((flags & ~SVDQ_FLAG_OUT_F32) != 0u) return SVDQ_ERR_ARG;
  if (!ptr_ok(X) || !ptr_ok(codes) || !ptr_ok(scales) || !ptr_ok(zeros) || !ptr_ok(Y) ||
      !opt_ok(bias))
    return SVDQ_ERR_ARG;
  if (M < 1 || M > 64) return SVDQ_ERR_SHAPE;
  if (N < 1 || N > (1 << 24) || K < 128 || K % 128 != 0 || K > (1 << 20)) return SVDQ_ERR_SHAPE;
  if ((int64_t)N * K > (int64_t(1) << 36)) return SVDQ_ERR_SHAPE;
  SVDQ_TRY(check_device());
  return from_hip(svdq::launch_awq_linear((flags & SVDQ_FLAG_OUT_F32) != 0u, M, N, K, X, codes,
                                          scales, zeros, bias, Y, (hipStream_t)stream));
}

}  // extern "C"
