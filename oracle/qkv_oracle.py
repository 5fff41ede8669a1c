"""CPU oracle for the attention-input transform after the QKV projection:
per-head RMSNorm of Q and K, then rotary position embedding (RoPE).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it.

The Nunchaku Lite page (axbrief.com, section "The Trade-off Between Fused
Kernels and Generality") names the fused engine's kernel that takes the QKV
projection through the Q/K normalisation and the rotary embedding; the pages
do not give the arithmetic.  The reading taken is the FLUX attention input
(public FLUX.1 architecture): the projection output of one token is
[Q | K | V], each of H heads of D = 128 features;
  RMSNorm of one head h of Q (and of K, with its own scale):
      q_hat[d] = q[d] / sqrt(mean_d(q[d]^2) + eps) * scale_q[d];
  RoPE on adjacent pairs (2i, 2i+1) of every head with the token's angles:
      out[2i]   = cos[m][i] q_hat[2i] - sin[m][i] q_hat[2i+1],
      out[2i+1] = sin[m][i] q_hat[2i] + cos[m][i] q_hat[2i+1];
V passes through.  cos and sin are inputs ([M][D/2]), since the positional
frequencies belong to the model, not to the layer.  This oracle computes in
fp64 and returns fp64 values.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rms_norm_heads", "rope_pairs", "qk_norm_rope", "HEAD_DIM"]

HEAD_DIM = 128


def rms_norm_heads(X: np.ndarray, scale: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of every head: X [M][H*D] (any float), scale [D]."""
    X = np.asarray(X, np.float64)
    M, HD = X.shape
    D = scale.shape[0]
    Xh = X.reshape(M, HD // D, D)
    ms = np.mean(Xh * Xh, axis=2, keepdims=True)
    return (Xh / np.sqrt(ms + eps) * np.asarray(scale, np.float64)[None, None, :]).reshape(M, HD)


def rope_pairs(X: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs of every head: X [M][H*D], cos/sin [M][D/2]."""
    X = np.asarray(X, np.float64)
    M, HD = X.shape
    half = cos.shape[1]
    Xp = X.reshape(M, HD // (2 * half), half, 2)
    c = np.asarray(cos, np.float64)[:, None, :]
    s = np.asarray(sin, np.float64)[:, None, :]
    out = np.empty_like(Xp)
    out[..., 0] = c * Xp[..., 0] - s * Xp[..., 1]
    out[..., 1] = s * Xp[..., 0] + c * Xp[..., 1]
    return out.reshape(M, HD)


def qk_norm_rope(Y: np.ndarray, heads: int, q_scale, k_scale, cos, sin, eps: float = 1e-6):
    """Y [M][3 H D] (the QKV output, any float) -> (Q, K, V) fp64 [M][H D] each:
    Q and K normalised per head and rotated, V unchanged."""
    Y = np.asarray(Y, np.float64)
    HD = heads * HEAD_DIM
    assert Y.shape[1] == 3 * HD
    Q = rope_pairs(rms_norm_heads(Y[:, :HD], q_scale, eps), cos, sin)
    K = rope_pairs(rms_norm_heads(Y[:, HD:2 * HD], k_scale, eps), cos, sin)
    return Q, K, Y[:, 2 * HD:].copy()
