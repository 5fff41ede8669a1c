"""CPU oracle for the SVDQuant W4A4 quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it.

It is a plain, slow, step-by-step numpy implementation of what the layer
computes, in fp64 where the mathematics is exact and with the explicit fp32 /
bf16 roundings that the packed codes and scales depend on.

Sources (cited by page title and section):
  [Apatero, "O que e Nunchaku"] -- page "Problemas do Nunchaku Qwen e como
      corrigi-los em 2025" (apatero.com), section "O que e Nunchaku e como
      acelera modelos Qwen": outliers are first moved from activations into the
      weights, then a high-precision low-rank branch obtained by SVD absorbs
      the weight outliers; the down-projection is fused into the quantization
      kernel and the up-projection into the 4-bit compute kernel.
  [Axbrief, "Mechanics"] -- page "Nunchaku Lite: the 50% VRAM reduction now
      integrated into Diffusers" (axbrief.com), section "The Mechanics of
      4-Bit Efficiency and SVDQuant": activation outliers are shifted toward
      the weights, the weight is split into a 16-bit low-rank branch and a
      4-bit residual branch, weights and activations both 4-bit (W4A4);
      ``SVDQW4A4Linear`` replaces ``nn.Linear``.
  [Note, "INT4"] -- page (note.com build log, Japanese), part "SVDQ-FP4 on
      Blackwell", item "1. INT4": INT4 codes cover -8..+7 and a weight is
      approximated as code x scale.
  [Axbrief, "Hardware"] -- same page as [Axbrief, "Mechanics"], section
      "Hardware Specialization and the Compression Workflow": an int4 and a
      4-bit floating-point precision exist side by side.

Parameters the pages leave open, fixed here (each is a reading, listed with
its reason in the design notes):
  * smoothing lambda_j = fp32(sqrt(fp64(max_m|X_mj|) / fp64(max_n|W_nj|))),
    lambda_j = 1 where either maximum is 0; X_hat = X / lambda (per input
    channel), W_hat = W * lambda;
  * X_hat is ONE bf16 tensor, bf16_RNE(fp32(X / lambda)), feeding both the
    quantizer and the low-rank down-projection;
  * INT4: groups of 64 along K, scale s = fp32(absmax / 7), code
    q = clamp(rint_half_even(fp32(v / s)), -8, 7), q = 0 when s == 0;
    two's-complement nibbles, even k in the low nibble;
  * FP4: E2M1 codes in blocks of 32 along K with an E8M0 power-of-two scale,
    e = clamp(floor(log2 absmax) - 2, -127, 127), e = -127 for an all-zero
    block, value y = v * 2^-e rounded to the nearest E2M1 grid point (ties to
    the even code), saturating at 6; sign-magnitude nibbles (bit 3 = sign);
    scale byte = e + 127;
  * low-rank factors from the fp64 SVD of W_hat^T with the singular values
    split evenly: L1 = bf16(U_r sqrt(S_r)) (K x r), L2 = bf16(sqrt(S_r) V_r^T)
    (r x N); rounding fp64 -> fp32 (RN) -> bf16 (RNE);
  * residual R = fp32(W_hat - acc), acc accumulated in fp32 over i = 0..r-1 in
    order, acc = fp32(acc + L1[k,i] * L2[i,n]) (bf16 x bf16 products are exact
    in fp32).
"""
from __future__ import annotations

import numpy as np

INT4_GROUP = 64
FP4_BLOCK = 32
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "calibrate_lambda", "column_absmax", "lambda_from_absmax",
    "smooth_weight",
    "lowrank_factors", "residual", "quantize_int4", "quantize_fp4",
    "pack_nibbles", "unpack_nibbles", "decode_int4", "decode_fp4",
    "pack_weight", "smooth_act", "quantize_act", "forward", "forward_dequant",
    "to_bf16_out",
]


# --------------------------------------------------------------------------
# bf16 <-> fp32 (bf16 is carried as uint16 bit patterns; numpy has no bf16)
# --------------------------------------------------------------------------
def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening: the bf16 bit pattern is the top half of the fp32 one."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, to nearest, ties to even (NaN -> quiet NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16).astype(np.uint16) & 0x8000) | 0x7FC0
    return r


# --------------------------------------------------------------------------
# Offline side: smoothing factor, smoothed weight, SVD branch, residual
# [Apatero, "O que e Nunchaku"]; [Axbrief, "Mechanics"]
# --------------------------------------------------------------------------
def column_absmax(A_bf16: np.ndarray, prev=None) -> np.ndarray:
    """max_m |A[m, j]| per column (fp32, exact), combined with a previous
    running maximum when given: the statistic calibration keeps over many
    batches of activations."""
    a = np.abs(bf16_to_f32(A_bf16)).max(axis=0).astype(np.float32)
    return a if prev is None else np.maximum(a, np.asarray(prev, np.float32))


def lambda_from_absmax(ax: np.ndarray, aw: np.ndarray) -> np.ndarray:
    """lambda_j = fp32(sqrt(fp64(ax_j) / fp64(aw_j))), 1 where either is 0."""
    ax = np.asarray(ax, np.float64)
    aw = np.asarray(aw, np.float64)
    ok = (ax > 0) & (aw > 0)
    lam = np.ones(ax.shape, dtype=np.float32)
    lam[ok] = np.sqrt(ax[ok] / aw[ok]).astype(np.float32)
    return lam


def calibrate_lambda(X_bf16: np.ndarray, W_bf16: np.ndarray) -> np.ndarray:
    """Per-input-channel smoothing factor (alpha = 1/2).

    lambda_j = fp32(sqrt(ax_j / aw_j)) with ax_j = max_m |X[m, j]| and
    aw_j = max_n |W[n, j]|, division and square root in fp64; lambda_j = 1
    where ax_j or aw_j is 0.  Dividing X by lambda and multiplying W by it
    moves magnitude from activation channels into weight columns while
    leaving X W^T unchanged.
    """
    return lambda_from_absmax(column_absmax(X_bf16), column_absmax(W_bf16))


def smooth_weight(W_bf16: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """W_hat[n, k] = fp32(W[n, k] * lambda_k): one fp32 rounding."""
    return (bf16_to_f32(W_bf16) * np.asarray(lam, np.float32)[None, :]).astype(np.float32)


def lowrank_factors(W_hat: np.ndarray, r: int):
    """Rank-r 16-bit branch from the SVD of the smoothed weight.

    W_hat^T (K x N) = U S V^T in fp64; L1 = bf16(U_r sqrt(S_r)) is K x r and
    L2 = bf16(sqrt(S_r) V_r^T) is r x N, so that L1 L2 ~ W_hat^T.  Returns
    (L1, L2, S) with L1/L2 as bf16 bit patterns and S the fp64 singular values.
    """
    U, S, Vt = np.linalg.svd(np.asarray(W_hat, np.float64).T, full_matrices=False)
    if r == 0:
        K, N = W_hat.shape[1], W_hat.shape[0]
        return np.zeros((K, 0), np.uint16), np.zeros((0, N), np.uint16), S
    rs = np.sqrt(S[:r])
    L1 = f32_to_bf16((U[:, :r] * rs[None, :]).astype(np.float32))
    L2 = f32_to_bf16((rs[:, None] * Vt[:r, :]).astype(np.float32))
    return L1, L2, S


def residual(W_hat: np.ndarray, L1_bf16: np.ndarray, L2_bf16: np.ndarray) -> np.ndarray:
    """R[n, k] = fp32(W_hat[n, k] - acc[n, k]) with
    acc = fp32(acc + L1[k, i] * L2[i, n]) for i = 0 .. r-1 in order."""
    W_hat = np.asarray(W_hat, np.float32)
    acc = np.zeros_like(W_hat)
    L1 = bf16_to_f32(L1_bf16)
    L2 = bf16_to_f32(L2_bf16)
    for i in range(L1.shape[1]):
        prod = np.multiply.outer(L2[i, :], L1[:, i]).astype(np.float32)  # exact
        acc = (acc + prod).astype(np.float32)
    return (W_hat - acc).astype(np.float32)


# --------------------------------------------------------------------------
# 4-bit quantizers  [Note, "INT4"]; [Axbrief, "Hardware"]
# --------------------------------------------------------------------------
def quantize_int4(V: np.ndarray):
    """Symmetric per-group INT4 quantization along the last axis.

    For each group of 64: a = max|v|, s = fp32(a / 7), q = 0 if s == 0 else
    clamp(rint(fp32(v / s)), -8, 7) with rint rounding half to even.
    Returns (codes int8 [rows, K], scales fp32 [rows, K/64]).
    """
    V = np.asarray(V, np.float32)
    rows, K = V.shape
    assert K % INT4_GROUP == 0
    Vg = V.reshape(rows, K // INT4_GROUP, INT4_GROUP)
    a = np.abs(Vg).max(axis=2)
    s = (a / np.float32(7.0)).astype(np.float32)
    q = np.zeros(Vg.shape, np.float32)
    nz = s != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (Vg / np.where(nz, s, np.float32(1.0))[:, :, None]).astype(np.float32)
    q = np.where(nz[:, :, None], np.clip(np.rint(quot), -8, 7), 0)
    return q.astype(np.int8).reshape(rows, K), s


def _e2m1_code(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 grid point to |y| (ties to the even code), sign in bit 3."""
    mag = np.abs(y)[..., None]
    d = np.abs(mag - E2M1_GRID)
    cand = d == d.min(axis=-1, keepdims=True)
    idx = np.arange(8)
    even = np.where(cand & (idx % 2 == 0), idx, 99).min(axis=-1)
    anyc = np.where(cand, idx, 99).min(axis=-1)
    code = np.where(even < 99, even, anyc).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 3)


def quantize_fp4(V: np.ndarray, chunk_rows: int = 256):
    """MXFP4-style quantization along the last axis: blocks of 32 share an
    E8M0 scale 2^e with e = clamp(floor(log2 a) - 2, -127, 127) (a = max|v|,
    e = -127 when a == 0), and each v becomes the E2M1 code of v * 2^-e.
    Returns (codes uint8 4-bit sign-magnitude [rows, K], scale bytes uint8
    [rows, K/32] holding e + 127)."""
    V = np.asarray(V, np.float32)
    rows, K = V.shape
    assert K % FP4_BLOCK == 0
    codes = np.empty((rows, K), np.uint8)
    sbytes = np.empty((rows, K // FP4_BLOCK), np.uint8)
    for r0 in range(0, rows, chunk_rows):
        Vb = V[r0:r0 + chunk_rows].reshape(-1, K // FP4_BLOCK, FP4_BLOCK).astype(np.float64)
        a = np.abs(Vb).max(axis=2)
        _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
        e = np.where(a > 0, np.clip(ex - 1 - 2, -127, 127), -127).astype(np.int64)
        y = np.ldexp(Vb, -e[:, :, None])          # exact in fp64
        codes[r0:r0 + chunk_rows] = _e2m1_code(y).reshape(-1, K)
        sbytes[r0:r0 + chunk_rows] = (e + 127).astype(np.uint8)
    return codes, sbytes


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2j in the low nibble, 2j+1 high."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: uint8 nibbles (0..15), element order restored."""
    p = np.asarray(packed, np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def decode_int4(packed: np.ndarray) -> np.ndarray:
    """Packed two's-complement nibbles -> int64 codes in -8..7."""
    n = unpack_nibbles(packed).astype(np.int64)
    return np.where(n >= 8, n - 16, n)


def decode_fp4(packed: np.ndarray) -> np.ndarray:
    """Packed E2M1 sign-magnitude nibbles -> fp64 values (before scaling)."""
    n = unpack_nibbles(packed).astype(np.int64)
    v = E2M1_GRID[n & 7]
    return np.where(n & 8, -v, v)


# --------------------------------------------------------------------------
# The three library operations
# --------------------------------------------------------------------------
def pack_weight(W_bf16, lam, L1_bf16, L2_bf16, mode: str):
    """Offline weight side: W_hat = W * lambda, R = W_hat - L1 L2 (fp32, fixed
    order), then 4-bit quantization of R's rows.  Returns (packed codes
    uint8 [N, K/2], scales: fp32 [N, K/64] for int4, uint8 [N, K/32] for fp4)."""
    W_hat = smooth_weight(W_bf16, lam)
    R = residual(W_hat, L1_bf16, L2_bf16)
    if mode == "int4":
        q, s = quantize_int4(R)
        return pack_nibbles(q), s
    if mode == "fp4":
        c, s = quantize_fp4(R)
        return pack_nibbles(c), s
    raise ValueError(mode)


def smooth_act(X_bf16: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """X_hat = bf16_RNE(fp32(X / lambda)) as bf16 bit patterns."""
    q = (bf16_to_f32(X_bf16) / np.asarray(lam, np.float32)[None, :]).astype(np.float32)
    return f32_to_bf16(q)


def quantize_act(X_bf16, lam, L1_bf16, mode: str, gelu_in: bool = False):
    """Run-time activation side: smoothing, 4-bit quantization of X_hat and
    the low-rank down-projection T = X_hat L1 from the same X_hat.  With
    gelu_in the layer's input is bf16_RNE(GELU_tanh(X)) (the MLP-down layer
    reading the up-projection's output; the fp32 steps are in gelu_oracle).
    Returns (packed codes, scales, T fp64 [M, r] or None, X_hat bf16 bits)."""
    if gelu_in:
        from .gelu_oracle import gelu_bf16
        X_bf16 = gelu_bf16(X_bf16)
    Xh = smooth_act(X_bf16, lam)
    Xf = bf16_to_f32(Xh)
    if mode == "int4":
        q, s = quantize_int4(Xf)
        codes = pack_nibbles(q)
    elif mode == "fp4":
        c, s = quantize_fp4(Xf)
        codes = pack_nibbles(c)
    else:
        raise ValueError(mode)
    T = None
    if L1_bf16 is not None and np.asarray(L1_bf16).shape[1] > 0:
        T = Xf.astype(np.float64) @ bf16_to_f32(L1_bf16).astype(np.float64)
    return codes, s, T, Xh


def _main_product_int4(xc, xs, wc, ws):
    """Y0[m, n] = sum_g sx[m, g] sw[n, g] (sum_{k in g} qx[m, k] qw[n, k]).
    The inner sums are integers below 2^24 in magnitude, so fp32 BLAS gives
    them exactly; the scaling and the sum over groups run in fp64."""
    qx = decode_int4(xc).astype(np.float32)
    qw = decode_int4(wc).astype(np.float32)
    G = qx.shape[1] // INT4_GROUP
    Y0 = np.zeros((qx.shape[0], qw.shape[0]), np.float64)
    for g in range(G):
        sl = slice(g * INT4_GROUP, (g + 1) * INT4_GROUP)
        P = (qx[:, sl] @ qw[:, sl].T).astype(np.float64)
        Y0 += (np.asarray(xs, np.float64)[:, g][:, None]
               * np.asarray(ws, np.float64)[:, g][None, :]) * P
    return Y0


def _main_product_fp4(xc, xs, wc, ws):
    """Y0[m, n] = sum_b 2^(ex[m, b] + ew[n, b]) (sum_{k in b} fx[m, k] fw[n, k]).
    E2M1 products are multiples of 1/4 and a block sum is at most 1152 in
    magnitude, so fp32 BLAS gives the inner sums exactly."""
    fx = decode_fp4(xc).astype(np.float32)
    fw = decode_fp4(wc).astype(np.float32)
    B = fx.shape[1] // FP4_BLOCK
    ex = np.asarray(xs, np.int64) - 127
    ew = np.asarray(ws, np.int64) - 127
    Y0 = np.zeros((fx.shape[0], fw.shape[0]), np.float64)
    for b in range(B):
        sl = slice(b * FP4_BLOCK, (b + 1) * FP4_BLOCK)
        P = (fx[:, sl] @ fw[:, sl].T).astype(np.float64)
        Y0 += np.ldexp(P, ex[:, b][:, None] + ew[:, b][None, :])
    return Y0


def forward(xcodes, xscales, T, wcodes, wscales, L2_bf16, bias_bf16, mode: str):
    """Y = deq(Q(X_hat) Q(R)^T) + T L2 + bias, all in fp64 (returns fp64)."""
    if mode == "int4":
        Y = _main_product_int4(xcodes, xscales, wcodes, wscales)
    elif mode == "fp4":
        Y = _main_product_fp4(xcodes, xscales, wcodes, wscales)
    else:
        raise ValueError(mode)
    if T is not None and L2_bf16 is not None and np.asarray(L2_bf16).shape[0] > 0:
        Y = Y + np.asarray(T, np.float64) @ bf16_to_f32(L2_bf16).astype(np.float64)
    if bias_bf16 is not None:
        Y = Y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return Y


def forward_dequant(xcodes, xscales, T, wcodes, wscales, L2_bf16, bias_bf16, mode: str):
    """Second formulation of ``forward``: dequantize both operands to fp64
    first, then one fp64 matmul."""
    if mode == "int4":
        dx = decode_int4(xcodes) * np.repeat(np.asarray(xscales, np.float64), INT4_GROUP, axis=1)
        dw = decode_int4(wcodes) * np.repeat(np.asarray(wscales, np.float64), INT4_GROUP, axis=1)
    else:
        dx = decode_fp4(xcodes) * np.repeat(np.ldexp(1.0, np.asarray(xscales, np.int64) - 127),
                                            FP4_BLOCK, axis=1)
        dw = decode_fp4(wcodes) * np.repeat(np.ldexp(1.0, np.asarray(wscales, np.int64) - 127),
                                            FP4_BLOCK, axis=1)
    Y = dx @ dw.T
    if T is not None and L2_bf16 is not None and np.asarray(L2_bf16).shape[0] > 0:
        Y = Y + np.asarray(T, np.float64) @ bf16_to_f32(L2_bf16).astype(np.float64)
    if bias_bf16 is not None:
        Y = Y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return Y


def to_bf16_out(Y: np.ndarray) -> np.ndarray:
    """The bf16 output the layer returns: fp64 -> fp32 (RN) -> bf16 (RNE)."""
    return f32_to_bf16(np.asarray(Y, np.float64).astype(np.float32))
