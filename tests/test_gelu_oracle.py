"""Pins of the GELU(tanh) oracle (CPU): exp_f32 against the exponential, the
fp32 GELU against the textbook tanh form in fp64, exact special values and
the odd-part identity, and planted mistakes in copies of the arithmetic
that each fail a pin."""
import math

import numpy as np
import pytest

import oracle as O


def _gelu_variant(x, a=0.044715, b=-2.0 * math.sqrt(2.0 / math.pi), deg=7, c2=True):
    """A copy of the fp32 steps with one knob changed (for the mutation pins)."""
    f = np.float32
    x = np.asarray(x, f)
    with np.errstate(over="ignore", invalid="ignore"):
        u = x + f(a) * (x * x * x)
        z = np.clip(f(b) * u, f(-104), f(104)).astype(f)
        k = np.rint(z * f(1 / math.log(2))).astype(f)
        r = (z - k * f(0.693359375)) - (k * f(math.log(2) - 0.693359375) if c2 else f(0))
        p = f(1 / math.factorial(deg))
        for n in range(deg - 1, -1, -1):
            p = (p * r + f(1 / math.factorial(n))).astype(f)
        e = np.ldexp(p, k.astype(np.int32)).astype(f)
        return (x / (f(1) + e)).astype(f)


def _check_gelu(g, x):
    """The pins a GELU implementation must meet on the grid x."""
    ref = O.gelu_tanh_f64(x.astype(np.float64))
    err = np.abs(g.astype(np.float64) - ref)
    big = np.abs(ref) >= 1e-3
    ok_rel = np.all(err[big] <= 2.0 ** -19 * np.abs(ref[big]))
    ok_abs = np.all(err <= 2.0 ** -20 * np.maximum(1.0, np.abs(x)))
    return ok_rel and ok_abs


X = np.linspace(-12, 12, 400_001).astype(np.float32)


def test_exp_against_the_exponential():
    z = np.linspace(-87, 88, 1_000_001).astype(np.float32)
    e = O.exp_f32(z).astype(np.float64)
    t = np.exp(z.astype(np.float64))
    assert np.max(np.abs(e - t) / t) <= 2 * 2.0 ** -24
    # exact at z = 0 and on powers of two of e's argument grid k ln 2 (r = 0 up to C2)
    assert O.exp_f32(np.float32(0.0)) == 1.0


def test_gelu_against_the_tanh_form():
    assert _check_gelu(O.gelu_tanh_f32(X), X)


def test_gelu_special_values_and_identity():
    g = O.gelu_tanh_f32(np.array([0.0, 10.0, 37.5, 1e13, 3e38], np.float32))
    assert np.array_equal(g, np.array([0.0, 10.0, 37.5, 1e13, 3e38], np.float32))
    neg = O.gelu_tanh_f32(np.array([-20.0, -1e13, -3e38], np.float32))
    assert np.all(neg == 0.0) and np.all(np.signbit(neg))
    # odd part: GELU(x) - GELU(-x) = x
    xs = np.linspace(0.0, 8.0, 10001).astype(np.float32)
    d = O.gelu_tanh_f32(xs).astype(np.float64) - O.gelu_tanh_f32(-xs).astype(np.float64)
    assert np.all(np.abs(d - xs) <= 2.0 ** -21 * np.maximum(1.0, xs))


def test_gelu_bf16_rounds_the_fp32_value():
    rng = np.random.default_rng(0)
    xb = (rng.standard_normal(4096).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    h = O.gelu_bf16(xb)
    assert np.array_equal(h, O.f32_to_bf16(O.gelu_tanh_f32(O.bf16_to_f32(xb))))


def test_variant_copy_matches_the_oracle():
    """The knob-free copy used below reproduces the oracle bit for bit, so a
    failing mutation is the planted change and nothing else."""
    assert np.array_equal(_gelu_variant(X).view(np.uint32), O.gelu_tanh_f32(X).view(np.uint32))


@pytest.mark.parametrize("kw", [dict(a=0.0447), dict(b=2.0 * math.sqrt(2.0 / math.pi)),
                                dict(deg=3), dict(c2=False)])
def test_mutations_fail_a_pin(kw):
    assert not _check_gelu(_gelu_variant(X, **kw), X)
