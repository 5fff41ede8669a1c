/*
 * svdq.h -- C ABI of the SVDQuant W4A4 quantized linear layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (Nunchaku Lite page on axbrief.com, section "The Mechanics of
 * 4-Bit Efficiency and SVDQuant"; Nunchaku troubleshooting page on
 * apatero.com, section "O que e Nunchaku e como acelera modelos Qwen"):
 * a per-input-channel smoothing factor lambda moves activation outliers into
 * the weight, the smoothed weight W_hat = W diag(lambda) is split into a
 * 16-bit rank-r branch L1 L2 (from its SVD) and a residual R that is stored
 * in 4 bits, activations are quantized to 4 bits at run time, and
 *
 *     Y = deq(Q(X_hat) Q(R)^T) + (X_hat L1) L2 + bias,   X_hat = X / lambda.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     dense row-major, 16-byte aligned.  The caller allocates and frees every
 *     buffer; the library allocates nothing and keeps no pointer after it
 *     returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls validate on the host, enqueue their kernels on `stream` and
 *     return; buffers must stay valid until that work completes.
 *   - Validation runs before any HIP runtime call: on SVDQ_ERR_ARG or
 *     SVDQ_ERR_SHAPE nothing is enqueued and outputs are untouched.  A device
 *     that is not gfx950 gives SVDQ_ERR_ARCH.  A failed launch or an earlier
 *     sticky HIP error gives SVDQ_ERR_HIP.  Faults inside kernels are
 *     asynchronous and surface at the caller's next synchronisation.
 *   - No call aborts the process or throws.
 *
 * Data formats (fixed by this library; the pages leave them open)
 *   bf16   : uint16_t bit patterns.
 *   lambda : float32 [K].
 *   L1, L2 : the rank-r factors are passed in the weight layout of the two
 *            linear maps they form, like nn.Linear weights:
 *              lora_down = L1^T, bf16 [r][K]   (the K -> r map),
 *              lora_up   = L2^T, bf16 [N][r]   (the r -> N map).
 *   INT4   : codes are two's-complement nibbles -8..7, groups of 64 along K,
 *            one float32 scale per (row, group) = fp32(absmax / 7); a code is
 *            clamp(rint_half_even(fp32(v / scale)), -8, 7), 0 when scale = 0.
 *   FP4    : codes are E2M1 sign-magnitude nibbles (bit 3 = sign, magnitudes
 *            0, .5, 1, 1.5, 2, 3, 4, 6), blocks of 32 along K, one E8M0 byte
 *            per (row, block) = e + 127 with e = clamp(floor(log2 absmax) - 2,
 *            -127, 127) (byte 0 for an all-zero block); a code is the nearest
 *            grid point to v * 2^-e, ties to the even code, saturating at 6.
 *   Packing: two codes per byte, element 2j in the low nibble and 2j+1 in
 *            the high nibble; rows are contiguous: codes [rows][K/2],
 *            scales [rows][K/64] (INT4, float32) or [rows][K/32] (FP4, uint8).
 *   T      : float32 [M][r], the down-projection X_hat L1.
 *
 * Shape limits: 1 <= M <= 2^31, M*K <= 2^36, K % 128 == 0, N % 128 == 0,
 * K, N <= 2^20, rank % 16 == 0, 0 <= rank <= 256 (rank 0 = no low-rank
 * branch); svdq_linear_forward also needs M*N <= 2^46.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_MODE_INT4 = 0, /* int4 codes, group 64, fp32 scales            */
  SVDQ_MODE_FP4 = 1   /* E2M1 codes, block 32, E8M0 scales (MXFP4)    */
} svdq_mode;

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_ARG = 1,   /* null / misaligned pointer, bad mode or flags  */
  SVDQ_ERR_SHAPE = 2, /* a size outside the limits above               */
  SVDQ_ERR_ARCH = 3,  /* current device is not gfx950                  */
  SVDQ_ERR_HIP = 4    /* HIP runtime error (launch or sticky error)    */
} svdq_status;

/* Y is written as float32 instead of bf16. */
#define SVDQ_FLAG_OUT_F32 0x1u

/* The layer's input is GELU(X) with the tanh approximation, applied to the
 * bf16 X that svdq_quantize_act and svdq_lowrank_down read: the down
 * projection of a transformer MLP reading the up projection's output (the
 * FLUX MLP: up-projection, GELU(tanh), down-projection), with the GELU fused
 * into the activation pass instead of a pass of its own.  Per element, in
 * IEEE fp32 without fused multiply-add:
 *   z = clamp(B * (x + A * ((x * x) * x)), -104, 104),
 *       A = fp32(0.044715), B = fp32(-2 sqrt(2/pi));
 *   e^z: k = rint(z * fp32(1/ln 2)), r = (z - k * 0.693359375) - k * fp32(ln 2 - 0.693359375),
 *        p = Horner form of sum_{n=0..7} r^n / n! (each 1/n! rounded to fp32,
 *        innermost first), e^z = p * 2^k;
 *   GELU(x) = x / (1 + e^z), rounded to bf16 (RNE) before smoothing.
 * svdq_linear_forward ignores the flag. */
#define SVDQ_FLAG_GELU_IN 0x2u

/* Static description of one quantized linear layer. */
typedef struct {
  int32_t mode;   /* svdq_mode                                   */
  int32_t K;      /* input features                               */
  int32_t N;      /* output features                              */
  int32_t rank;   /* r, width of the 16-bit low-rank branch        */
  uint32_t flags; /* SVDQ_FLAG_*                                  */
} svdq_desc;

/* Human-readable name of a status code (static storage). */
const char* svdq_status_string(svdq_status s);

/* 1 if a device architecture name (hipDeviceProp_t::gcnArchName, e.g.
 * "gfx950:sramecc+:xnack-") is one this library runs on, else 0.  Pure host
 * function; the capability check the pages describe for 4-bit kernels
 * (axbrief.com page, section "Hardware Specialization and the Compression
 * Workflow"). */
int svdq_arch_supported(const char* gcn_arch_name);

/* Library version, e.g. "0.1.0". */
const char* svdq_version(void);

/* Offline calibration of the smoothing factor (apatero.com page, section
 * "O que e Nunchaku ...": outliers are moved from activations to weights).
 *   lambda[k] = fp32(sqrt(fp64(max_m |X[m][k]|) / fp64(max_n |W[n][k]|))),
 *   lambda[k] = 1 where either maximum is 0.
 * X: bf16 [M][K] calibration activations; W: bf16 [N][K]; lambda: out [K].
 * Limits: M >= 1, N >= 1, K % 128 == 0. */
svdq_status svdq_calibrate_lambda(int64_t M, int32_t K, int32_t N, const uint16_t* X,
                                  const uint16_t* W, float* lambda, void* stream);

/* Calibration over many batches (same page and section: the outlier
 * statistics the smoothing factor comes from).  The per-column absolute
 * maximum of a bf16 matrix A [R][K], combined with the running maximum in
 * amax when accumulate is 1 (0: amax is overwritten):
 *   amax[k] = max(accumulate ? amax[k] : 0, max_r |A[r][k]|)   (exact).
 * Call it once per calibration batch of activations (and once on W), then
 * svdq_lambda_from_absmax.  Limits: 1 <= R <= 2^31, K % 128 == 0,
 * K <= 2^20; accumulate is 0 or 1. */
svdq_status svdq_calibrate_absmax(int64_t R, int32_t K, const uint16_t* A, float* amax,
                                  int32_t accumulate, void* stream);

/* lambda[k] = fp32(sqrt(fp64(xmax[k]) / fp64(wmax[k]))), 1 where either
 * maximum is 0 (the rule of svdq_calibrate_lambda, from running maxima).
 * xmax, wmax, lambda: float32 [K]; K % 128 == 0, K <= 2^20. */
svdq_status svdq_lambda_from_absmax(int32_t K, const float* xmax, const float* wmax,
                                    float* lambda, void* stream);

/* NVFP4 variant (axbrief.com page, sections "The Mechanics of 4-Bit
 * Efficiency and SVDQuant" and "Hardware Specialization and the Compression
 * Workflow": NVFP4 is the pages' 4-bit float format; its layout is NVIDIA's
 * published one).  The same layer (smoothing, rank-r 16-bit branch, 4-bit
 * residual), with both operands in NVFP4:
 *   codes  : E2M1 nibbles as in SVDQ_MODE_FP4, [rows][K/2];
 *   scales : uint8 [rows][K/16], the E4M3 scale of each block of 16 along K
 *            (bias 7, subnormals m 2^-9, largest finite 448 = byte 0x7E);
 *   g      : one float32 per tensor (device memory), > 0.
 * Quantization of a row-major tensor V: t = fp32(6 g); per block a = max |v|,
 * s = E4M3_RNE_sat(fp32(a / t)) (nearest E4M3 value, ties to the even
 * mantissa, 448 from 448 up), d = fp32(s * g), code = the E2M1 code of
 * fp32(v / d) as in SVDQ_MODE_FP4 (all codes 0 when s = 0); value = code * s
 * * g.  The per-tensor scale is g = fp32(amax / 2688) (2688 = 6 * 448), 1
 * when amax = 0.  Codes and scales are bit-identical to this definition.
 * gfx950's block-scaled matrix instructions take only power-of-two scales
 * per 32 elements, so the GEMM dequantizes both operands to bf16 (exact:
 * code * s has at most 6 significant bits) and runs the bf16 matrix
 * instruction; it is slower than SVDQ_MODE_FP4 (MXFP4), which gfx950 runs
 * natively.  Shape limits: K, N multiples of 128, <= 2^20; 1 <= M <= 2^31,
 * M * K <= 2^36; rank % 16 == 0, 0 <= rank <= 256. */

/* g = fp32(max_i amax[i] / 2688), or 1 if the maximum is 0: the activation
 * scale from calibration maxima (e.g. svdq_calibrate_absmax of X_hat's
 * columns).  amax: float32 [n] device, n >= 1; g: float32 [1] device. */
svdq_status svdq_nvfp4_scale_from_absmax(int32_t n, const float* amax, float* g, void* stream);

/* X_hat = bf16_RNE(fp32(X / lambda)) quantized with the per-tensor scale *g
 * (device), and, when rank > 0, the down-projection T = X_hat L1 from the
 * same read of X (the fusion the apatero.com page describes in section "O
 * que e Nunchaku ...", as in svdq_quantize_act).
 * X: bf16 [M][K]; xcodes [M][K/2]; xscales uint8 [M][K/16]; lora_down bf16
 * [r][K] (= L1 transposed) and T float32 [M][r], both NULL when rank is 0.
 * rank % 16 == 0, 0 <= rank <= 256. */
svdq_status svdq_nvfp4_quantize_act(int64_t M, int32_t K, int32_t rank, const uint16_t* X,
                                    const float* lambda, const float* g,
                                    const uint16_t* lora_down, uint8_t* xcodes, uint8_t* xscales,
                                    float* T, void* stream);

/* Offline: the residual R of svdq_pack_weight (same arithmetic) quantized
 * with g = fp32(max |R| / 2688) (written to *g, device float).  W bf16
 * [N][K]; lora_down bf16 [r][K] and lora_up bf16 [N][r] (NULL when rank is
 * 0); wcodes [N][K/2]; wscales uint8 [N][K/16]. */
svdq_status svdq_nvfp4_pack_weight(int32_t N, int32_t K, int32_t rank, const uint16_t* W,
                                   const float* lambda, const uint16_t* lora_down,
                                   const uint16_t* lora_up, uint8_t* wcodes, uint8_t* wscales,
                                   float* g, void* stream);

/* Y = g_x g_w sum_b s_x[m][b] s_w[n][b] sum_{k in b} c_x[m][k] c_w[n][k]
 *     + T L2 + bias, written [M][N] as bf16 (RNE) or float32
 * (flags = SVDQ_FLAG_OUT_F32; other bits are SVDQ_ERR_ARG).  T: float32
 * [M][r] (svdq_nvfp4_quantize_act), lora_up bf16 [N][r] (both NULL when rank is
 * 0); bias bf16 [N] or NULL.  fp32 arithmetic: exact products of the
 * dequantized values, fp32 sums, T L2 through a bf16 hi/lo split of T. */
svdq_status svdq_nvfp4_linear(int64_t M, int32_t N, int32_t K, int32_t rank,
                              const uint8_t* xcodes, const uint8_t* xscales, const float* g_x,
                              const uint8_t* wcodes, const uint8_t* wscales, const float* g_w,
                              const float* T, const uint16_t* lora_up, const uint16_t* bias,
                              uint32_t flags, void* Y, void* stream);

/* Offline: the rank-r factors of the smoothed weight (apatero.com page,
 * section "O que e Nunchaku ...", and axbrief.com page, section "The
 * Mechanics ...": the 16-bit branch is the rank-r part of W_hat =
 * W diag(lambda) from its SVD), by a randomized truncated SVD.  The pages
 * leave the SVD's algorithm open; this library fixes it as the randomized
 * range finder with power iterations (Halko, Martinsson and Tropp, "Finding
 * structure with randomness", SIAM Review 2011, algorithms 4.4 and 5.1):
 *   W_hat[n][k] = fp32(W[n][k] * lambda[k]), then fp64 throughout;
 *   l = min(rank + 16, N, K) sketch columns;
 *   Omega[n][j] = -1 if bit (j mod 128) of the Philox4x32-10 block of counter
 *     (n, j / 128, 0, 0) and key (seed mod 2^32, seed / 2^32) is set, else +1
 *     (bit b of a block = bit b mod 32 of its word b / 32);
 *   Q = orth(W_hat^T Omega); power_iters times: Z = orth(W_hat Q),
 *     Q = orth(W_hat^T Z);
 *   B = W_hat Q; B^T B = V diag(s^2) V^T, eigenvalues in descending order
 *     (equal ones by index), each eigenvector's largest-magnitude component
 *     (the first if several) positive;
 *   lora_down = L1^T with L1 = Q V_r diag(sqrt s)       bf16 [rank][K],
 *   lora_up   = L2^T = B V_r diag(1 / sqrt s)            bf16 [N][rank]
 *     (1 in place of sqrt s when s = 0), each rounded fp64 -> fp32 -> bf16
 *     (RNE both times); sigma[i] = s_i (fp64 [rank], optional, NULL = not
 *     written);
 *   orth(Y) = shifted CholeskyQR2: twice Y <- Y L^-T with
 *     L L^T = Y^T Y + (1e-12 trace(Y^T Y) / l) I (a zero Y stays zero).
 * lora_down and lora_up are the inputs of svdq_pack_weight and
 * svdq_quantize_act of a layer with this rank.  The result is a deterministic
 * function of the inputs, equal to the definition up to fp64 rounding (the
 * bf16 factors then match it up to a rounding-boundary ulp).
 * Limits: N, K multiples of 128, <= 2^20, N*K <= 2^32; 16 <= rank <= 128,
 * rank % 16 == 0; 0 <= power_iters <= 8.  workspace: device memory of at
 * least svdq_lowrank_factors_workspace() bytes, 256-byte aligned, owned by
 * the caller, contents undefined afterwards (SVDQ_ERR_ARG if smaller). */
svdq_status svdq_lowrank_factors_workspace(int32_t N, int32_t K, int32_t rank, size_t* bytes);
svdq_status svdq_lowrank_factors(int32_t N, int32_t K, int32_t rank, const uint16_t* W,
                                 const float* lambda, uint64_t seed, int32_t power_iters,
                                 uint16_t* lora_down, uint16_t* lora_up, double* sigma,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* svdq_lowrank_factors for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same results, bit for bit, with the
 * workspace in a static device array of 64 MiB that the library holds on
 * each device it runs on until the process ends (no allocation, no workspace
 * argument).  Shapes whose svdq_lowrank_factors_workspace exceeds 64 MiB
 * (e.g. 3072 x 3072 at rank 32 fits, 9216 x 3072 does not) give
 * SVDQ_ERR_SHAPE before anything is enqueued; other arguments and errors as
 * for svdq_lowrank_factors.  All calls on one device share that array:
 * calls whose work overlaps on one device (different streams, or threads)
 * race and must be serialised by the caller. */
svdq_status svdq_lowrank_factors_noalloc(int32_t N, int32_t K, int32_t rank, const uint16_t* W,
                                         const float* lambda, uint64_t seed, int32_t power_iters,
                                         uint16_t* lora_down, uint16_t* lora_up, double* sigma,
                                         void* stream);

/* Offline weight packing (same two pages; the residual branch of W4A4).
 *   W_hat[n][k] = fp32(W[n][k] * lambda[k]);
 *   acc = 0; for i = 0..r-1: acc = fp32(acc + L1[k][i] * L2[i][n]);
 *   R[n][k] = fp32(W_hat[n][k] - acc);   (no fused multiply-add anywhere)
 *   R quantized row by row in desc->mode into wcodes [N][K/2] and wscales.
 * W: bf16 [N][K]; lora_down: bf16 [r][K]; lora_up: bf16 [N][r] (both NULL
 * when rank == 0).  Codes and scales are bit-identical to the definition. */
svdq_status svdq_pack_weight(const svdq_desc* desc, const uint16_t* W, const float* lambda,
                             const uint16_t* lora_down, const uint16_t* lora_up,
                             uint8_t* wcodes, void* wscales, void* stream);

/* Operand images.  The GEMM reads both sides of the layer as "images": the
 * codes and scales re-laid in the lane order of the gfx950 matrix
 * instructions, together with the low-rank factor (T on the activation
 * side, L2 on the weight side) and, on the weight side, the bias, so that
 * one kernel streams everything it needs with contiguous copies.  An image
 * depends only on desc and M; its size is given by the two size functions
 * below, and every call that reads or writes one takes its byte count and
 * returns SVDQ_ERR_ARG unless it is exactly that size (so no access can
 * leave the caller's buffer).  An image of the right size built for another
 * descriptor is not detected: the result is then meaningless, but still in
 * bounds.
 *
 * How the row-major ABI tensors map into the images (bit for bit; the
 * parity tests decode the images and compare them with these tensors):
 *   G = K/64 groups; rows are grouped in 32-row tiles (activation rows
 *   padded with zero rows to a multiple of 256, weight rows = output columns
 *   padded to a multiple of 192 (INT4) or 256 (FP4)); "slot" s = 0..63 of a
 *   tile stands for row s % 32 of the tile and K half h = s / 32 (elements
 *   64 g + 32 h .. +31 of the group).
 *   INT4 code block (g, tile), 2048 bytes, at (g * tiles + tile) * 2048:
 *     bytes 768 h + 16 r .. +15 and 768 h + 512 + 8 r .. +7 hold, as one
 *     little-endian 192-bit string, the 32 codes q of row r and K half h,
 *     element i in bits 6 i .. 6 i + 5 as the sign-magnitude field
 *     (q < 0 ? 0x20 : 0) | |q| (the E2M3 encoding of q / 8); in the
 *     activation image a code 0 may also appear as 0x20 (-0: the encoder
 *     keeps the sign of a value that rounds to zero), which adds nothing
 *     to the product either;
 *     bytes 1536 + 8 s .. +7: the scale of row s % 32 and group g as two
 *     bf16 halves hi = bf16_RNE(s), lo = bf16_RNE(s - hi):
 *       activation image: slot s < 32: {hi | lo << 16, hi}, s >= 32: {lo, 0};
 *       weight image:     slot s < 32: {hi | hi << 16, lo}, s >= 32: {lo, 0}
 *     (dwords; together they make the K slots of a bf16 outer product hold
 *     hi*hi, lo*hi, hi*lo and lo*lo).
 *   FP4 code block (g, tile), 1024 bytes: bytes 16 s .. +15 are the 32
 *     packed E2M1 codes of row s % 32, K half s / 32, exactly as in the
 *     row-major codes; FP4 scale block (g, tile), 64 bytes, after all code
 *     blocks: byte s is the E8M0 scale of that row and 32-element block.
 *   Activation low-rank blocks (rank > 0), after the code (and scale)
 *     blocks: per (16-rank slice j, tile) 2048 bytes; slot s: row s % 32,
 *     ranks 16 j + 8 (s / 32) .. +7: bytes 16 s .. +15 the 8 bf16
 *     hi = bf16_RNE(T), bytes 1024 + 16 s .. +15 the 8 bf16
 *     lo = bf16_RNE(T - hi), T being the fp32 down-projection that the T
 *     output of svdq_quantize_act holds.
 *   Partial sums (activation side, rank > 0): the pass that writes the image
 *     splits K into S ranges of whole 64-groups, S = max(1, min(16,
 *     (K/64)/48, ceil(1024 / (padded rows / 16)))); when S > 1 the image
 *     ends with S fp32 partial sums of T per padded row, which a second
 *     kernel adds in order.
 *   Weight low-rank blocks (rank > 0): per (16-rank slice j, 32-column tile)
 *     1024 bytes; slot s: column s % 32, bytes 16 s .. +15 the 8 bf16
 *     lora_up[n][16 j + 8 (s / 32) .. +7] (L2 transposed).
 *   Bias: 64 bytes (32 bf16) per 32-column tile, zero without a bias, then
 *     1024 bytes of zero padding.
 * Storage: an INT4 image keeps each 4-bit code in a 6-bit field, the
 * narrowest operand of the gfx950 matrix instructions that holds -8..7
 * exactly, plus the bf16 scale halves: 8 bits per weight element, against
 * 4.5 bits in the row-major codes and scales (the weight memory is 2x
 * smaller than bf16 rather than 3.6x).  Re-expanding nibbles inside the
 * GEMM would add VALU work to a loop whose time is already VALU and MFMA
 * issue.  FP4 images hold the 4-bit codes as they are (4.25 bits per
 * element, 3.8x smaller than bf16). */

/* Bytes of the activation image for M rows.  Pure host function. */
svdq_status svdq_act_image_size(const svdq_desc* desc, int64_t M, size_t* bytes);

/* Bytes of the prepared weight of a layer.  Pure host function. */
svdq_status svdq_weight_image_size(const svdq_desc* desc, size_t* bytes);

/* Run-time activation side, one kernel (apatero.com page, section "O que e
 * Nunchaku ...": the down-projection of the low-rank branch is fused into
 * the quantization kernel and shares its activations).
 *   X_hat[m][k] = bf16_RNE(fp32(X[m][k] / lambda[k]));
 *   X_hat quantized row by row in desc->mode (codes, scales);
 *   T[m][i] = sum_k X_hat[m][k] * L1[k][i]   (fp32 accumulation).
 * Outputs, each optional (NULL = not written), at least one present:
 *   xcodes [M][K/2] and xscales (both or neither): the codes and scales in
 *     the documented row-major layout;
 *   T [M][r] float32: the down-projection (needs lora_down);
 *   ximage: the activation image that svdq_linear_forward reads, of
 *     ximage_bytes = svdq_act_image_size(desc, M) bytes (0 when ximage is
 *     NULL; any other count is SVDQ_ERR_ARG); with rank > 0 it includes T,
 *     so lora_down is then required.
 * With rank == 0, lora_down and T must be NULL.  Codes and scales are
 * bit-identical to the definition; T is accurate to fp32 accumulation. */
svdq_status svdq_quantize_act(const svdq_desc* desc, int64_t M, const uint16_t* X,
                              const float* lambda, const uint16_t* lora_down, uint8_t* xcodes,
                              void* xscales, float* T, void* ximage, size_t ximage_bytes,
                              void* stream);

/* Offline: the prepared weight of a layer (the one-time packing of the
 * weights into the kernel layout, as the apatero.com page describes for the
 * fused 4-bit kernel) from the codes and scales of svdq_pack_weight, the
 * low-rank factor lora_up (bf16 [N][r]; required when rank > 0, NULL when
 * rank == 0) and the bias (bf16 [N], or NULL for none).  wimage: device
 * buffer of wimage_bytes = svdq_weight_image_size(desc) bytes (any other
 * count is SVDQ_ERR_ARG), written completely. */
svdq_status svdq_prepare_weight(const svdq_desc* desc, const uint8_t* wcodes,
                                const void* wscales, const uint16_t* lora_up,
                                const uint16_t* bias, void* wimage, size_t wimage_bytes,
                                void* stream);

/* The W4A4 GEMM with the up-projection and the bias fused (axbrief.com
 * page, section "The Mechanics ...": 4-bit weights and activations;
 * apatero.com page: the up-projection is fused into the 4-bit compute
 * kernel).  From the activation image of M rows and the prepared weight of
 * the same desc:
 *   INT4: Y0[m][n] = sum_g sx[m][g] sw[n][g] sum_{k in g} qx[m][k] qw[n][k]
 *   FP4 : Y0[m][n] = sum_b 2^(ex[m][b] + ew[n][b]) sum_{k in b} fx[m][k] fw[n][k]
 *   Y = Y0 + T L2 + bias (T L2 only when rank > 0), written [M][N] as bf16
 *   (RNE) or float32 (SVDQ_FLAG_OUT_F32).
 * Accuracy: the integer/E2M1 block sums are exact, the rest is fp32
 * arithmetic (INT4: the product of the two group scales carries a relative
 * error below 2^-15; T and L2 enter as bf16 hi/lo splits, within 2^-16).
 * ximage_bytes and wimage_bytes are the sizes of the two buffers and must
 * equal svdq_act_image_size(desc, M) and svdq_weight_image_size(desc)
 * (else SVDQ_ERR_ARG, before anything is enqueued).  One kernel; no
 * workspace. */
svdq_status svdq_linear_forward(const svdq_desc* desc, int64_t M, const void* ximage,
                                size_t ximage_bytes, const void* wimage, size_t wimage_bytes,
                                void* Y, void* stream);

/* The same layer from weights kept resident in their packed 4-bit form: the
 * row-major codes and scales of svdq_pack_weight (INT4: 4.5 bits per weight
 * with the fp32 group scales; FP4: 4.25), L2 and the bias, instead of a
 * prepared weight (INT4: 8 bits per weight).  This is the memory case of the
 * pages (axbrief.com page, section "The Mechanics ...": 4-bit weights; the
 * apatero.com page, section "O que e Nunchaku ...", on the 3.6x smaller
 * model).  The gfx950 matrix instructions have no 4-bit integer operand, so
 * each call first writes the prepared weight into wscratch (a device buffer
 * of wscratch_bytes = svdq_weight_image_size(desc) bytes, else SVDQ_ERR_ARG
 * before anything is enqueued), then runs svdq_linear_forward on it: two
 * kernels on the stream, Y bit-identical to svdq_prepare_weight followed by
 * svdq_linear_forward.  One scratch serves every layer whose image fits, one
 * call at a time per scratch (calls that overlap on one scratch race).
 * Arguments as for svdq_prepare_weight and svdq_linear_forward; wscratch
 * must not overlap the other buffers. */
svdq_status svdq_linear_forward_packed(const svdq_desc* desc, int64_t M, const void* ximage,
                                       size_t ximage_bytes, const uint8_t* wcodes,
                                       const void* wscales, const uint16_t* lora_up,
                                       const uint16_t* bias, void* wscratch,
                                       size_t wscratch_bytes, void* Y, void* stream);

/* The layer from the tensors of the row-major ABI: the activation codes and
 * scales of svdq_quantize_act (xcodes [M][K/2], xscales [M][K/64] float32
 * (INT4) or [M][K/32] uint8 (FP4)), its down-projection T (float32 [M][r]),
 * the weight codes and scales of svdq_pack_weight, lora_up (bf16 [N][r])
 * and the bias (bf16 [N] or NULL): the forward of the axbrief.com page,
 * section "The Mechanics of 4-Bit Efficiency and SVDQuant" (4-bit weights
 * and activations with a 16-bit low-rank branch), for callers that keep
 * these tensors rather than the operand images.  Each call writes the
 * activation image (codes, scales and T as above; a code 0 is written as
 * +0) and the prepared weight into `workspace`, a device buffer of at least
 * svdq_linear_rowmajor_workspace_size(desc, M) bytes (fewer is
 * SVDQ_ERR_ARG, before anything is enqueued), then runs the GEMM: three
 * kernels on the stream.  Y equals svdq_linear_forward on the images that
 * svdq_quantize_act and svdq_prepare_weight write for the same tensors (up
 * to the sign of an exact zero); T and lora_up are both required when
 * rank > 0 and both NULL when rank == 0.  The workspace must not overlap
 * the other buffers, and calls that share one overlap-free workspace run
 * one at a time (overlapping calls race). */
svdq_status svdq_linear_rowmajor_workspace_size(const svdq_desc* desc, int64_t M, size_t* bytes);
svdq_status svdq_linear_forward_rowmajor(const svdq_desc* desc, int64_t M, const uint8_t* xcodes,
                                         const void* xscales, const float* T,
                                         const uint8_t* wcodes, const void* wscales,
                                         const uint16_t* lora_up, const uint16_t* bias, void* Y,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* The MLP up-projection with the next layer's activation pass fused into
 * its epilogue (Nunchaku Lite page on axbrief.com, section "The Trade-off
 * Between Fused Kernels and Generality": neighbouring steps of the block
 * fused into one kernel to cut memory traffic; apatero.com page, section "O
 * que e Nunchaku ...": the low-rank down-projection shares the quantization
 * kernel's activations).  `up` is an INT4 layer, `down` the INT4 layer that
 * reads GELU of its output (down->K == up->N, down->flags has
 * SVDQ_FLAG_GELU_IN, down->rank <= 128).  In one pass over the up layer's
 * output tiles, with the up layer's images ximage / wimage (sizes as for
 * svdq_linear_forward):
 *   y = the up layer's output, rounded to bf16 exactly as
 *       svdq_linear_forward writes it (written to Y, bf16 [M][up->N], when Y
 *       is not NULL);
 *   x = GELU(y) as SVDQ_FLAG_GELU_IN defines it, then the down layer's
 *       activation pass on x: ximage_down (svdq_act_image_size(down, M) bytes)
 *       receives the same codes, scales and T halves that svdq_quantize_act
 *       of `down` on x writes into the image (T is fp32-accumulated in a
 *       different order: over 128-column tiles, then over the tiles), and T,
 *       when not NULL, fp32 [M][down->rank], the down-projection itself.
 * The bf16 intermediate is never written (unless Y asks for it) nor read.
 * lambda_down: float32 [up->N]; lora_down: bf16 [down->rank][up->N] (NULL,
 * like T, when down->rank is 0).  workspace: device memory of at least
 * svdq_gelu_quantize_workspace_size bytes (the per-tile partial sums of T;
 * contents undefined afterwards; 0 bytes and NULL allowed when down->rank
 * is 0).  Two launches on `stream` (the fused GEMM, then the sum of the T
 * partials).  Other arguments and errors as for svdq_linear_forward; an
 * up or down descriptor that is not INT4, or a down descriptor without
 * SVDQ_FLAG_GELU_IN, is SVDQ_ERR_ARG. */
svdq_status svdq_gelu_quantize_workspace_size(const svdq_desc* up, int64_t M,
                                              const svdq_desc* down, size_t* bytes);
svdq_status svdq_linear_forward_gelu_quantize(const svdq_desc* up, int64_t M, const void* ximage,
                                              size_t ximage_bytes, const void* wimage,
                                              size_t wimage_bytes, const svdq_desc* down,
                                              const float* lambda_down, const uint16_t* lora_down,
                                              void* ximage_down, size_t ximage_down_bytes,
                                              uint16_t* Y, float* T, void* workspace,
                                              size_t workspace_bytes, void* stream);

/* Unfused low-rank branch, for comparison with the fused schedule (the
 * apatero.com page quotes the overhead of running the rank-32 branch as
 * separate kernels).  svdq_lowrank_down re-reads X and writes
 * T = bf16_RNE(fp32(X / lambda)) L1 (fp32 [M][r]); svdq_lowrank_up adds
 * T L2 to an existing Y [M][N] (bf16 or float32 per desc->flags) in place. */
svdq_status svdq_lowrank_down(const svdq_desc* desc, int64_t M, const uint16_t* X,
                              const float* lambda, const uint16_t* lora_down, float* T,
                              void* stream);
svdq_status svdq_lowrank_up(const svdq_desc* desc, int64_t M, const float* T,
                            const uint16_t* lora_up, void* Y, void* stream);

/* Attention input after the QKV projection (axbrief.com page, section "The
 * Trade-off Between Fused Kernels and Generality": the fused engine takes
 * the QKV projection through the Q/K normalisation and the rotary
 * embedding; the pages leave the arithmetic open, and this library follows
 * the FLUX attention input).  Y: bf16 [M][ld], one row per token whose
 * first 2 * heads * 128 features are Q and K, heads of 128 features each
 * ([Q | K | V] for a QKV layer, ld = 3 * heads * 128; the rest of the row,
 * e.g. V or a fused MLP part, is not touched).  In place, for every token m
 * and every head of Q (scale q_scale) and of K (k_scale):
 *   x_hat[d] = x[d] * (1 / sqrt(sum_d x[d]^2 / 128 + eps)) * scale[d],
 *   out[2i]   = cos[m][i] x_hat[2i] - sin[m][i] x_hat[2i+1],
 *   out[2i+1] = sin[m][i] x_hat[2i] + cos[m][i] x_hat[2i+1],   i < 64,
 * in fp32, each output rounded to bf16 (RNE).
 * q_scale, k_scale: bf16 [128]; cos, sin: float32 [M][64] (the positional
 * angles belong to the model).  Limits: 1 <= M <= 2^31, 1 <= heads <= 2048,
 * 2 * heads * 128 <= ld <= 2^24, ld % 8 == 0; eps > 0 and finite (else
 * SVDQ_ERR_ARG).  Pointers as in the conventions above. */
svdq_status svdq_qk_norm_rope(int64_t M, int32_t heads, int64_t ld, uint16_t* Y,
                              const uint16_t* q_scale, const uint16_t* k_scale, const float* cos,
                              const float* sin, float eps, void* stream);

/* svdq_linear_forward of a layer whose output starts with Q and K (the QKV
 * projection, or a fused QKV + MLP projection), followed by the transform
 * of svdq_qk_norm_rope on its first 2 * heads * 128 columns (ld = N), on the
 * bf16 output: two launches on `stream` (the GEMM, then the in-place pass),
 * in INT4 and FP4 mode alike.  Output bf16 only (SVDQ_FLAG_OUT_F32 is
 * SVDQ_ERR_ARG); 2 * heads * 128 <= N; image sizes and other limits as
 * for svdq_linear_forward and svdq_qk_norm_rope. */
svdq_status svdq_linear_forward_qk(const svdq_desc* desc, int64_t M, const void* ximage,
                                   size_t ximage_bytes, const void* wimage, size_t wimage_bytes,
                                   int32_t heads, const uint16_t* q_scale,
                                   const uint16_t* k_scale, const float* cos, const float* sin,
                                   float eps, void* Y, void* stream);

/* AWQ W4A16 linear layer: 4-bit weights, 16-bit activations (axbrief.com
 * page, section "The Mechanics of 4-Bit Efficiency and SVDQuant": the
 * layer type that keeps activations in 16 bits; section "The Trade-off
 * Between Fused Kernels and Generality": it is assigned to the modulation
 * linear layers, whose input is one vector per image).  The pages leave the
 * format open; this library fixes it as
 *   codes  : uint8 [N][K/2], nibbles 0..15, element 2j in the low nibble;
 *   scales : float32 [N][K/64], one per (row, group of 64 along K);
 *   zeros  : uint8 [N][K/64], zero points 0..15;
 *   deq(W)[n][k] = scales[n][g] * (q[n][k] - zeros[n][g]),  g = k / 64.
 * Shape limits: 1 <= N <= 2^24, 128 <= K <= 2^20 with K % 128 == 0,
 * N*K <= 2^36, and for svdq_awq_linear 1 <= M <= 64 (a small-batch kernel:
 * it streams the packed weight once per 4 rows of X).  Layers that share
 * their input (the modulation maps of all blocks read the same conditioning
 * vector) can be packed as one weight with their rows concatenated and run
 * as one call.  Pointers follow the conventions above. */

/* Offline: asymmetric min-max quantization of a bf16 weight W [N][K] per
 * (row, group):
 *   d = max(fp32(max - min), 1e-5), s = fp32(d / 15),
 *   z = clamp(rint(fp32(-min / s)), 0, 15),
 *   q = clamp(rint(fp32(w / s)) + z, 0, 15)       (rint: ties to even).
 * Every step is one IEEE fp32 operation; codes, scales and zeros are
 * bit-identical to this definition.  W must be finite. */
svdq_status svdq_awq_pack_weight(int32_t N, int32_t K, const uint16_t* W, uint8_t* codes,
                                 float* scales, uint8_t* zeros, void* stream);

/* Y[m][n] = sum_k X[m][k] deq(W)[n][k] + bias[n] for X bf16 [M][K], written
 * [M][N] as bf16 (RNE) or float32 (flags = SVDQ_FLAG_OUT_F32; other bits are
 * SVDQ_ERR_ARG).  bias: bf16 [N] or NULL.  fp32 arithmetic: per 16 weights
 * the kernel forms sum (128 + q) x and sum x from exact bf16 products and
 * combines them with the group's scale and zero point. */
svdq_status svdq_awq_linear(int64_t M, int32_t N, int32_t K, const uint16_t* X,
                            const uint8_t* codes, const float* scales, const uint8_t* zeros,
                            const uint16_t* bias, uint32_t flags, void* Y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
