"""CPU oracle for the AWQ W4A16 linear layer (4-bit weights, 16-bit activations).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it.

Source: page "Nunchaku Lite: the 50% VRAM reduction now integrated into
Diffusers" (axbrief.com), sections "The Mechanics of 4-Bit Efficiency and
SVDQuant" (``AWQW4A16Linear`` replaces ``nn.Linear`` for 4-bit weights with
16-bit activations) and "The Trade-off Between Fused Kernels and Generality"
(modulation linear layers are assigned AWQ W4A16).

The pages give no format details; fixed here (a reading, listed in the design
notes): asymmetric 4-bit codes 0..15 per (row, group of 64 along K) with an
fp32 scale and a zero point 0..15, from the group's minimum and maximum:
  d = fp32(max - min), d = max(d, 1e-5) (a constant group still gets a
  nonzero step), s = fp32(d / 15), z = clamp(rint(fp32(-min / s)), 0, 15),
  q = clamp(rint(fp32(w / s)) + z, 0, 15)   (rint: half to even),
and the weight is taken as s * (q - z).  Every step is one IEEE fp32
operation, so codes, scales and zero points are reproducible bit for bit.
The layer is Y = X . deq(W)^T + b, computed here in fp64.
"""
from __future__ import annotations

import numpy as np

from .svdq_oracle import bf16_to_f32, pack_nibbles, unpack_nibbles

AWQ_GROUP = 64

__all__ = ["AWQ_GROUP", "awq_quantize", "awq_dequant", "awq_forward", "awq_forward_dequant"]


def awq_quantize(W_bf16: np.ndarray):
    """Pack a bf16 weight [N][K] (uint16 bit patterns).

    Returns (codes uint8 [N][K/2] packed nibbles 0..15 with element 2j in the
    low nibble, scales fp32 [N][K/64], zeros uint8 [N][K/64])."""
    W = bf16_to_f32(W_bf16)
    N, K = W.shape
    assert K % AWQ_GROUP == 0
    G = K // AWQ_GROUP
    Wg = W.reshape(N, G, AWQ_GROUP)
    mx = Wg.max(axis=2)
    mn = Wg.min(axis=2)
    d = (mx - mn).astype(np.float32)
    d = np.maximum(d, np.float32(1e-5))
    s = (d / np.float32(15.0)).astype(np.float32)
    z = np.clip(np.rint((-mn / s).astype(np.float32)), 0, 15)
    q = np.clip(np.rint((Wg / s[:, :, None]).astype(np.float32)) + z[:, :, None], 0, 15)
    codes = pack_nibbles(q.reshape(N, K).astype(np.int16))
    return codes, s, z.astype(np.uint8)


def awq_dequant(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """deq(W)[n][k] = s[n][g] * (q[n][k] - z[n][g]) in fp64."""
    q = unpack_nibbles(codes).astype(np.float64)
    N, K = q.shape
    G = K // AWQ_GROUP
    qg = q.reshape(N, G, AWQ_GROUP)
    w = np.asarray(scales, np.float64)[:, :, None] * (qg - np.asarray(zeros, np.float64)[:, :, None])
    return w.reshape(N, K)


def awq_forward(X_bf16, codes, scales, zeros, bias_bf16=None) -> np.ndarray:
    """Y[m][n] = sum_g s[n][g] * sum_{k in g} (q[n][k] - z[n][g]) x[m][k] + b[n],
    in fp64 (per-group form)."""
    X = bf16_to_f32(X_bf16).astype(np.float64)
    M, K = X.shape
    q = unpack_nibbles(codes).astype(np.float64)
    N = q.shape[0]
    G = K // AWQ_GROUP
    Y = np.zeros((M, N), np.float64)
    for g in range(G):
        sl = slice(g * AWQ_GROUP, (g + 1) * AWQ_GROUP)
        inner = X[:, sl] @ (q[:, sl] - np.asarray(zeros, np.float64)[:, g][:, None]).T
        Y += inner * np.asarray(scales, np.float64)[:, g][None, :]
    if bias_bf16 is not None:
        Y += bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return Y


def awq_forward_dequant(X_bf16, codes, scales, zeros, bias_bf16=None) -> np.ndarray:
    """The same layer as X . deq(W)^T + b (dequantize, then one product)."""
    X = bf16_to_f32(X_bf16).astype(np.float64)
    Y = X @ awq_dequant(codes, scales, zeros).T
    if bias_bf16 is not None:
        Y += bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return Y
