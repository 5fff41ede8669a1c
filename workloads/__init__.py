"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module only draws random tensors: activations X, weights W and bias b,
with the shapes and outlier structure of the FLUX-sized workloads the method is
demonstrated on (the Nunchaku pages describe FLUX.1-dev and Qwen-Image
transformers; no checkpoints or calibration data exist here, so these draws
stand in for them). It holds none of the method's arithmetic: no smoothing,
no SVD, no quantization. Both the CPU oracle and the GPU path take their inputs
from here.

Recipe (shared by every workload):
  * one ``torch.Generator`` seeded with ``seed``; draws happen in the order
    X, X-outlier channel indices (randperm), X-outlier factors, W,
    W-outlier column indices (randperm), bias;
  * values are drawn in fp32, scaled, then rounded to bf16 (RNE, torch's cast);
  * X ~ N(0, 1) with ``x_outliers`` input channels multiplied by a per-channel
    factor (a constant, or one U(lo, hi) draw per channel);
  * W ~ N(0, 0.02) with ``w_outliers`` input columns multiplied by
    ``w_factor``;
  * bias ~ N(0, 0.01).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple, Union

import numpy as np
import torch

Factor = Union[float, Tuple[float, float]]


@dataclasses.dataclass(frozen=True)
class LinearSpec:
    """One quantized linear layer: Y[M, N] = X[M, K] . W[N, K]^T + b."""
    name: str
    M: int
    K: int
    N: int
    rank: int
    mode: str                      # "int4", "fp4", or "awq" (W4A16, rank 0)
    x_outliers: int
    x_factor: Factor
    w_outliers: int = 0
    w_factor: float = 1.0


def _round_count(frac: float, k: int) -> int:
    return int(round(frac * k))


# Workloads (shapes from the FLUX.1-dev transformer: hidden 3072, QKV 9216,
# MLP 12288, 1024x1024 latent with 2x2 patches = 4096 image tokens, 512 text).
TINY = LinearSpec("tiny_256x512x512_r16", 256, 512, 512, 16, "int4",
                  x_outliers=4, x_factor=50.0)
FLUX_QKV = LinearSpec("flux_qkv_4096x3072x9216_r32", 4096, 3072, 9216, 32, "int4",
                      x_outliers=_round_count(0.01, 3072), x_factor=(20.0, 100.0),
                      w_outliers=_round_count(0.005, 3072), w_factor=10.0)
FLUX_MLP_UP = LinearSpec("flux_mlp_up_4608x3072x12288_r32", 4608, 3072, 12288, 32, "int4",
                         x_outliers=_round_count(0.01, 3072), x_factor=(20.0, 100.0),
                         w_outliers=_round_count(0.005, 3072), w_factor=10.0)
# The down projection's activations are GELU(up output); only W is drawn here.
FLUX_MLP_DOWN = LinearSpec("flux_mlp_down_4608x12288x3072_r32", 4608, 12288, 3072, 32, "int4",
                           x_outliers=0, x_factor=1.0,
                           w_outliers=_round_count(0.005, 12288), w_factor=10.0)
FLUX_FUSED_FP4 = LinearSpec("flux_fused_qkv_mlp_fp4_4608x3072x21504_r32", 4608, 3072, 21504, 32,
                            "fp4", x_outliers=_round_count(0.01, 3072), x_factor=50.0)

SPECS = {s.name: s for s in (TINY, FLUX_QKV, FLUX_MLP_UP, FLUX_MLP_DOWN, FLUX_FUSED_FP4)}


def block_chain_specs(rank: int = 128):
    """The eight quantized linears of one FLUX double-stream block at batch 2:
    image stream M = 2*4096, text stream M = 2*512; per stream qkv 3072->9216,
    out-proj 3072->3072, MLP up 3072->12288, MLP down 12288->3072.  The MLP
    down layer's input is GELU(MLP up output) at run time."""
    out = []
    for stream, M in (("img", 8192), ("txt", 1024)):
        for lname, K, N in (("qkv", 3072, 9216), ("out", 3072, 3072),
                            ("up", 3072, 12288), ("down", 12288, 3072)):
            down = lname == "down"
            out.append(LinearSpec(f"block_{stream}_{lname}", M, K, N, rank, "int4",
                                  x_outliers=0 if down else _round_count(0.01, K),
                                  x_factor=1.0 if down else (20.0, 100.0),
                                  w_outliers=_round_count(0.005, K), w_factor=10.0))
    return out


def modulation_specs(M: int = 1):
    """The AWQ W4A16 modulation linears of one FLUX.1 forward: their input is
    one conditioning vector per image (M = batch).  Hidden size 3072; each of
    the 19 double-stream blocks has an image and a text modulation map
    3072 -> 6*3072, each of the 38 single-stream blocks 3072 -> 3*3072, and
    the output norm 3072 -> 2*3072.  Returns [(spec, count)]."""
    kw = dict(rank=0, mode="awq", x_outliers=0, x_factor=1.0,
              w_outliers=_round_count(0.005, 3072), w_factor=10.0)
    return [(LinearSpec(f"mod_double_{M}x3072x18432", M, 3072, 18432, **kw), 38),
            (LinearSpec(f"mod_single_{M}x3072x9216", M, 3072, 9216, **kw), 38),
            (LinearSpec(f"mod_norm_out_{M}x3072x6144", M, 3072, 6144, **kw), 1)]


def draw(spec: LinearSpec, seed: int = 0, M: Optional[int] = None):
    """Draw (X, W, bias) as bf16 CPU tensors for ``spec``.

    ``M`` overrides the token count (the rows of X are drawn first, so a
    smaller M gives a different X but the same recipe).  X is None-free even
    for down layers; callers replace it by GELU(up output) where the recipe
    says so.
    """
    M = spec.M if M is None else M
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(M, spec.K, generator=g, dtype=torch.float32)
    if spec.x_outliers:
        idx = torch.randperm(spec.K, generator=g)[: spec.x_outliers]
        if isinstance(spec.x_factor, tuple):
            lo, hi = spec.x_factor
            f = lo + (hi - lo) * torch.rand(spec.x_outliers, generator=g, dtype=torch.float32)
        else:
            f = torch.full((spec.x_outliers,), float(spec.x_factor))
        X[:, idx] *= f
    W = 0.02 * torch.randn(spec.N, spec.K, generator=g, dtype=torch.float32)
    if spec.w_outliers:
        widx = torch.randperm(spec.K, generator=g)[: spec.w_outliers]
        W[:, widx] *= spec.w_factor
    b = 0.01 * torch.randn(spec.N, generator=g, dtype=torch.float32)
    return X.to(torch.bfloat16), W.to(torch.bfloat16), b.to(torch.bfloat16)


def spectral_weight(N: int, K: int, seed: int = 0, terms: int = 192, decay: float = 1.0,
                    noise: float = 0.002) -> torch.Tensor:
    """A bf16 weight [N][K] with a decaying spectrum, like trained projection
    weights (and unlike an i.i.d. Gaussian draw, whose singular values
    bunch together): sum_i s_i a_i b_i^T over ``terms`` Gaussian pairs with
    s_i = 0.02 (1 + i)^-decay, plus N(0, noise) per entry.  One generator
    seeded with ``seed``; draws in the order a, b, noise."""
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(N, terms, generator=g, dtype=torch.float32)
    b = torch.randn(terms, K, generator=g, dtype=torch.float32) / float(np.sqrt(K))
    s = 0.02 * (1.0 + torch.arange(terms, dtype=torch.float32)) ** -decay
    W = (a * s[None, :]) @ b + noise * torch.randn(N, K, generator=g, dtype=torch.float32)
    return W.to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 array of its bit patterns (no arithmetic)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor (no arithmetic)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
