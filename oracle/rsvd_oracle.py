"""CPU oracle for the rank-r factors of the smoothed weight by randomized SVD.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it.

The 16-bit branch is the rank-r part of W_hat = W diag(lambda) from its SVD
(Nunchaku troubleshooting page on apatero.com, section "O que e Nunchaku e
como acelera modelos Qwen"; Nunchaku Lite page on axbrief.com, section "The
Mechanics of 4-Bit Efficiency and SVDQuant").  The pages do not say how the
SVD is computed; this is the randomized range finder with power iterations of
Halko, Martinsson and Tropp ("Finding structure with randomness", SIAM Review
2011, algorithms 4.4 and 5.1), with l = r + p sketch columns:

  Omega [N][l]: Rademacher signs, sign (n, j) = bit (j mod 128) of the
      128-bit block Philox4x32-10(counter = (n, j div 128, 0, 0),
      key = (seed_lo, seed_hi)) (bit b of the block = bit b mod 32 of word
      b div 32), bit set -> -1 (Salmon, Moraes, Dror and Shaw, "Parallel
      random numbers: as easy as 1, 2, 3", SC 2011);
  Q = orth(W_hat^T Omega);  q times: Z = orth(W_hat Q), Q = orth(W_hat^T Z);
  B = W_hat Q [N][l];  B^T B = V diag(s^2) V^T (eigenvalues descending,
      equal ones in index order; each eigenvector's sign is chosen so that its
      component of largest magnitude, the first one if several, is positive);
  L1 = Q V_r diag(sqrt s_r) [K][r],  L2^T = B V_r diag(1/sqrt s_r) [N][r],
so that L1 L2 = Q Q^T-projected W_hat^T restricted to the top r directions,
with the balanced sqrt(s) split; both factors are rounded to bf16 (RNE).
orth() is shifted CholeskyQR2 (two rounds of G = Y^T Y + 1e-12 trace(G)/l I,
R = chol(G), Y R^-1; a zero Y is returned unchanged).  This oracle runs every
step in fp64.
"""
from __future__ import annotations

import numpy as np

from .svdq_oracle import bf16_to_f32, f32_to_bf16

__all__ = ["philox4x32_10", "rademacher", "rsvd_factors", "rsvd_factors_f64", "orth_cholqr2",
           "RSVD_OVERSAMPLE", "RSVD_SHIFT"]

RSVD_OVERSAMPLE = 16
_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """One Philox4x32 block with 10 rounds: 4 x uint32 counter, 2 x uint32 key."""
    c0, c1, c2, c3 = (int(v) & _MASK for v in ctr)
    k0, k1 = (int(v) & _MASK for v in key)
    for rnd in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> 32, p0 & _MASK
        hi1, lo1 = p1 >> 32, p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if rnd < 9:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
    return c0, c1, c2, c3


def rademacher(N: int, l: int, seed: int) -> np.ndarray:
    """Omega [N][l] of +-1 (fp64)."""
    key = (seed & _MASK, (seed >> 32) & _MASK)
    om = np.empty((N, l), np.float64)
    for n in range(N):
        for blk in range((l + 127) // 128):
            words = philox4x32_10((n, blk, 0, 0), key)
            for b in range(min(128, l - 128 * blk)):
                om[n, 128 * blk + b] = -1.0 if (words[b >> 5] >> (b & 31)) & 1 else 1.0
    return om


RSVD_SHIFT = 1e-12


def orth_cholqr2(Y: np.ndarray) -> np.ndarray:
    """Shifted CholeskyQR2: two rounds of Y <- Y R^-1 with
    R^T R = Y^T Y + shift I, shift = 1e-12 trace(Y^T Y) / l (the shift keeps
    the factorization defined when the sketch is rank-deficient, as in
    shifted CholeskyQR; with full rank its effect is of that relative size)."""
    for _ in range(2):
        G = Y.T @ Y
        tr = np.trace(G)
        if tr == 0.0:                               # a zero Y stays zero
            return Y
        G = G + (RSVD_SHIFT * tr / G.shape[0]) * np.eye(G.shape[0])
        R = np.linalg.cholesky(G).T                 # upper triangular
        Y = np.linalg.solve(R.T, Y.T).T             # Y R^-1
    return Y


def rsvd_factors_f64(What: np.ndarray, r: int, seed: int, power_iters: int = 2,
                     oversample: int = RSVD_OVERSAMPLE):
    """fp64 (L1 [K][r], L2^T [N][r], s [r]) of an fp64 matrix What [N][K]."""
    N, K = What.shape
    l = min(r + oversample, min(N, K))
    Om = rademacher(N, l, seed)
    Q = orth_cholqr2(What.T @ Om)
    for _ in range(power_iters):
        Z = orth_cholqr2(What @ Q)
        Q = orth_cholqr2(What.T @ Z)
    B = What @ Q
    ev, V = np.linalg.eigh(B.T @ B)
    order = np.argsort(-ev, kind="stable")
    ev, V = ev[order], V[:, order]
    big = np.argmax(np.abs(V), axis=0)
    V = V * np.where(V[big, np.arange(V.shape[1])] < 0, -1.0, 1.0)[None, :]
    s = np.sqrt(np.maximum(ev[:r], 0.0))
    rs = np.sqrt(s)
    L1 = (Q @ V[:, :r]) * rs[None, :]
    up = (B @ V[:, :r]) / np.where(rs > 0, rs, 1.0)[None, :]
    return L1, up, s


def rsvd_factors(W_bf16, lam, r: int, seed: int, power_iters: int = 2,
                 oversample: int = RSVD_OVERSAMPLE):
    """(lora_down = L1^T bf16 [r][K], lora_up = L2^T bf16 [N][r], s [r] fp64)
    of W_hat = fp32(W * lambda)."""
    W = bf16_to_f32(W_bf16)
    What = (W * np.asarray(lam, np.float32)[None, :]).astype(np.float32).astype(np.float64)
    L1, up, s = rsvd_factors_f64(What, r, seed, power_iters, oversample)
    return f32_to_bf16(L1.T.astype(np.float32)), f32_to_bf16(up.astype(np.float32)), s
