"""CPU oracle for the NVFP4 variant of the W4A4 layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it.

The pages name NVFP4 as the 4-bit float format of the FP4 path (Nunchaku Lite
page on axbrief.com, sections "The Mechanics of 4-Bit Efficiency and
SVDQuant" and "Hardware Specialization and the Compression Workflow";
Nunchaku troubleshooting page on apatero.com); they do not give its layout.
The reading taken is NVIDIA's published NVFP4 format: E2M1 elements in blocks
of 16 along K, each block with an FP8 E4M3 scale, and one fp32 scale g per
tensor.  Quantization of a tensor V with per-tensor scale g (fp32, > 0):
  t = fp32(6 g);
  per block of 16: a = max |v|;  s = E4M3_RNE_sat(fp32(a / t));
  d = fp32(s g);  code = E2M1_RNE_sat(fp32(v / d)) with v's sign, all codes 0
  (+0) when s = 0;
  dequantized value = code * s * g.
E4M3_RNE_sat: nearest value of the E4M3 grid (normals (1 + m/8) 2^e,
e = -6..8, subnormals m 2^-9, largest finite 448), ties to the even
mantissa, values above 448 to 448.  The per-tensor scale is
g = fp32(amax / 2688) (2688 = 6 * 448, so the largest block scale is about
448), g = 1 when amax = 0.  The main product of the layer is
  Y0[m, n] = g_x g_w sum_b s_x[m, b] s_w[n, b] sum_{k in b} c_x[m, k] c_w[n, k].
"""
from __future__ import annotations

import numpy as np

from .svdq_oracle import (E2M1_GRID, _e2m1_code, bf16_to_f32, pack_nibbles, residual,
                          smooth_act, smooth_weight, unpack_nibbles)

__all__ = ["NVFP4_BLOCK", "E4M3_MAX", "e4m3_encode", "e4m3_decode", "nvfp4_global_scale",
           "quantize_nvfp4", "decode_nvfp4", "nvfp4_quantize_act", "nvfp4_pack_weight",
           "nvfp4_forward", "nvfp4_forward_dequant"]

NVFP4_BLOCK = 16
E4M3_MAX = 448.0
_f = np.float32


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """E4M3 bytes (sign 0, 0x00..0x7E) -> fp64 values."""
    b = np.asarray(b, np.int64)
    e = (b >> 3) & 0xF
    m = b & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))


def _rne(x: np.ndarray) -> np.ndarray:
    return np.rint(x)   # numpy rounds half to even


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Bytes of E4M3_RNE_sat(v) for v >= 0 (fp32 or fp64 values)."""
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.int64)
    sat = v >= E4M3_MAX
    sub = v < 2.0 ** -6
    # subnormal range: step 2^-9; q = 8 is the smallest normal, byte 8 as well
    out[sub] = _rne(v[sub] * 2.0 ** 9).astype(np.int64)
    nm = ~sat & ~sub
    f, ex = np.frexp(v[nm])                 # v = f 2^ex, f in [0.5, 1)
    e = ex - 1
    q = _rne((v[nm] * np.exp2(-e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    b = ((e + 7) << 3) | q
    out[nm] = np.minimum(b, 0x7E)           # above 448 only by rounding: saturate
    out[sat] = 0x7E
    return out.astype(np.uint8)


def nvfp4_global_scale(amax: float) -> np.float32:
    """g = fp32(amax / 2688), or 1 when amax is 0."""
    a = np.float32(amax)
    return np.float32(a / np.float32(6.0 * E4M3_MAX)) if a > 0 else np.float32(1.0)


def quantize_nvfp4(V: np.ndarray, g) -> tuple:
    """Codes uint8 [rows, K] (4-bit sign-magnitude E2M1) and E4M3 block-scale
    bytes uint8 [rows, K/16] of V (fp32 [rows, K]) with per-tensor scale g."""
    V = np.asarray(V, np.float32)
    rows, K = V.shape
    assert K % NVFP4_BLOCK == 0
    g = np.float32(g)
    t = np.float32(np.float32(6.0) * g)
    Vb = V.reshape(rows, K // NVFP4_BLOCK, NVFP4_BLOCK)
    a = np.abs(Vb).max(axis=2)
    with np.errstate(over="ignore"):
        sbf = (a / t).astype(np.float32)
    sb = e4m3_encode(sbf)
    sval = e4m3_decode(sb).astype(np.float32)
    d = (sval * g).astype(np.float32)
    nz = sval > 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (Vb / np.where(nz, d, np.float32(1.0))[:, :, None]).astype(np.float32)
    codes = _e2m1_code(y.astype(np.float64))
    codes = np.where(nz[:, :, None], codes, np.uint8(0)).astype(np.uint8)
    return codes.reshape(rows, K), sb


def decode_nvfp4(packed: np.ndarray, sbytes: np.ndarray, g) -> np.ndarray:
    """Dequantized fp64 values c * s * g of packed codes and scale bytes."""
    n = unpack_nibbles(packed).astype(np.int64)
    c = np.where(n & 8, -E2M1_GRID[n & 7], E2M1_GRID[n & 7])
    s = np.repeat(e4m3_decode(sbytes), NVFP4_BLOCK, axis=1)
    return c * s * float(np.float32(g))


def nvfp4_quantize_act(X_bf16, lam, g_x):
    """Activation side: X_hat = bf16_RNE(fp32(X / lambda)) (as in the other
    modes), quantized with the calibrated per-tensor scale g_x.  Returns
    (packed codes [M, K/2], scale bytes [M, K/16], X_hat bf16 bits)."""
    Xh = smooth_act(X_bf16, lam)
    codes, sb = quantize_nvfp4(bf16_to_f32(Xh), g_x)
    return pack_nibbles(codes), sb, Xh


def nvfp4_pack_weight(W_bf16, lam, L1_bf16, L2_bf16):
    """Weight side: the residual R of W_hat and the low-rank part, quantized
    with g_w = nvfp4_global_scale(max |R|).  Returns (packed codes, scale
    bytes, g_w)."""
    R = residual(smooth_weight(W_bf16, lam), L1_bf16, L2_bf16)
    g_w = nvfp4_global_scale(float(np.abs(R).max()))
    codes, sb = quantize_nvfp4(R, g_w)
    return pack_nibbles(codes), sb, g_w


def _codes_f32(packed):
    n = unpack_nibbles(packed).astype(np.int64)
    return np.where(n & 8, -E2M1_GRID[n & 7], E2M1_GRID[n & 7]).astype(np.float32)


def nvfp4_forward(xc, xs, g_x, T, wc, ws, g_w, L2_bf16, bias_bf16):
    """Y = g_x g_w sum_b s_x s_w (sum_{k in b} c_x c_w) + T L2 + bias in fp64.
    E2M1 products are multiples of 1/4 and a block sum is at most 576 in
    magnitude, so fp32 BLAS gives the inner sums exactly."""
    fx, fw = _codes_f32(xc), _codes_f32(wc)
    sx, sw = e4m3_decode(xs), e4m3_decode(ws)
    Y = np.zeros((fx.shape[0], fw.shape[0]), np.float64)
    for b in range(fx.shape[1] // NVFP4_BLOCK):
        sl = slice(b * NVFP4_BLOCK, (b + 1) * NVFP4_BLOCK)
        P = (fx[:, sl] @ fw[:, sl].T).astype(np.float64)
        Y += (sx[:, b][:, None] * sw[:, b][None, :]) * P
    Y *= float(np.float32(g_x)) * float(np.float32(g_w))
    if T is not None and L2_bf16 is not None and np.asarray(L2_bf16).shape[0] > 0:
        Y = Y + np.asarray(T, np.float64) @ bf16_to_f32(L2_bf16).astype(np.float64)
    if bias_bf16 is not None:
        Y = Y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return Y


def nvfp4_forward_dequant(xc, xs, g_x, T, wc, ws, g_w, L2_bf16, bias_bf16):
    """Second formulation: both operands dequantized to fp64, one matmul."""
    Y = decode_nvfp4(xc, xs, g_x) @ decode_nvfp4(wc, ws, g_w).T
    if T is not None and L2_bf16 is not None and np.asarray(L2_bf16).shape[0] > 0:
        Y = Y + np.asarray(T, np.float64) @ bf16_to_f32(L2_bf16).astype(np.float64)
    if bias_bf16 is not None:
        Y = Y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return Y
