"""CPU oracle for the GELU(tanh) prologue of the MLP-down layer's quantize pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it.

The FLUX MLP is up-projection, GELU with the tanh approximation, then
down-projection (the MLP pair of the FLUX-shaped workloads).  Fusing the GELU
into the quantization pass of the down layer needs the activation function
fixed to the last fp32 operation, because its bf16-rounded output decides the
4-bit codes.  The definition used on both sides (a reading: the pages name
the MLP, not this arithmetic):

  GELU_tanh(x) = 0.5 x (1 + tanh(s (x + a x^3))),  s = sqrt(2/pi), a = 0.044715
               = x / (1 + exp(-2 s (x + a x^3)))      (0.5 (1 + tanh y) = 1 / (1 + e^-2y)),

the second form having no cancellation for negative x.  In fp32, one IEEE
operation per step and no fused multiply-add:
  x2 = x*x; x3 = x2*x; u = x + A*x3; z = clamp(B*u, -104, 104);
  e = exp_f32(z); h = x / (1 + e);   the output is bf16_RNE(h),
with A = fp32(0.044715), B = fp32(-2 sqrt(2/pi)).
exp_f32 is Cody and Waite's argument reduction with a two-part ln 2 and a
degree-7 Taylor polynomial on the reduced argument:
  k = rint(z * L) (ties to even), r = (z - k*C1) - k*C2,
  p = 1 + r(1 + r(1/2 + r(1/6 + r(1/24 + r(1/120 + r(1/720 + r/5040))))))
      (Horner, innermost first; each 1/n! rounded to fp32),
  exp_f32(z) = p * 2^k   (exact scaling, gradual underflow, overflow to inf),
with L = fp32(1/ln 2), C1 = 0.693359375 (ln 2 to 10 significant bits, so
k*C1 is exact), C2 = fp32(ln 2 - C1).
"""
from __future__ import annotations

import math

import numpy as np

from .svdq_oracle import bf16_to_f32, f32_to_bf16

__all__ = ["exp_f32", "gelu_tanh_f32", "gelu_bf16", "gelu_tanh_f64"]

_f = np.float32
_L = _f(1.0 / math.log(2.0))
_C1 = _f(0.693359375)
_C2 = _f(math.log(2.0) - 0.693359375)
_A = _f(0.044715)
_B = _f(-2.0 * math.sqrt(2.0 / math.pi))
_INV_FACT = [_f(1.0 / math.factorial(n)) for n in range(8)]   # 1, 1, 1/2, ..., 1/5040


def exp_f32(z: np.ndarray) -> np.ndarray:
    """e^z in fp32 by the steps above; z fp32 with |z| <= 104."""
    z = np.asarray(z, np.float32)
    k = np.rint(z * _L).astype(np.float32)
    r = (z - k * _C1) - k * _C2
    p = _INV_FACT[7]
    for n in range(6, -1, -1):
        p = (p * r + _INV_FACT[n]).astype(np.float32)
    with np.errstate(over="ignore"):
        return np.ldexp(p, k.astype(np.int32)).astype(np.float32)


def gelu_tanh_f32(x: np.ndarray) -> np.ndarray:
    """GELU with the tanh approximation, fp32, by the steps above."""
    x = np.asarray(x, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        x2 = x * x
        x3 = x2 * x
        u = x + _A * x3
        z = np.clip(_B * u, _f(-104.0), _f(104.0)).astype(np.float32)
        e = exp_f32(z)
        return (x / (_f(1.0) + e)).astype(np.float32)


def gelu_bf16(X_bf16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of bf16_RNE(GELU_tanh(x)) for bf16 inputs."""
    return f32_to_bf16(gelu_tanh_f32(bf16_to_f32(X_bf16)))


def gelu_tanh_f64(x: np.ndarray) -> np.ndarray:
    """The textbook tanh form in fp64 (for pins only)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))
