"""Pins of the AWQ W4A16 oracle (CPU): exact recovery of a weight that lies
on a 4-bit grid, the half-step error bound, the code and zero ranges, the
per-group form against dequantize-then-multiply, and a scalar brute force."""
import numpy as np
import pytest

import oracle as O


def _bits_f32(x):
    """fp32 values that are exact in bf16 -> bf16 bit patterns."""
    x = np.asarray(x, np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f32(b), x)
    return b


def test_exact_grid_is_recovered():
    """W = s0 (q - z0) with s0 a power of two and each group using codes 0
    and 15: the packer must return s0, z0 and q exactly."""
    rng = np.random.default_rng(0)
    N, K = 6, 256
    G = K // 64
    s0 = np.ldexp(1.0, rng.integers(-12, -2, (N, G))).astype(np.float32)
    z0 = rng.integers(0, 16, (N, G))
    q = rng.integers(0, 16, (N, G, 64))
    q[:, :, 0], q[:, :, 1] = 0, 15
    w = (s0[:, :, None] * (q - z0[:, :, None])).astype(np.float32).reshape(N, K)
    codes, s, z = O.awq_quantize(_bits_f32(w))
    assert np.array_equal(s, s0)
    assert np.array_equal(z, z0.astype(np.uint8))
    assert np.array_equal(O.unpack_nibbles(codes), q.reshape(N, K).astype(np.uint8))
    assert np.array_equal(O.awq_dequant(codes, s, z), w.astype(np.float64))


def test_half_step_bound_and_ranges():
    rng = np.random.default_rng(1)
    N, K = 32, 512
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    w[3, :64] = 0.0                     # constant group: floor of the step
    w[4, 64:128] = 0.5                  # positive constant group
    b = (w.view(np.uint32) >> 16).astype(np.uint16)
    wf = O.bf16_to_f32(b).astype(np.float64)
    codes, s, z = O.awq_quantize(b)
    q = O.unpack_nibbles(codes)
    assert q.max() <= 15 and z.max() <= 15
    assert np.all(s > 0)
    deq = O.awq_dequant(codes, s, z)
    step = np.repeat(s.astype(np.float64), 64, axis=1)
    # every weight between the group's min and max dequantizes within half
    # a step (plus the fp32 roundings of the quotient), except where the
    # zero point was clipped to the code range
    zc = np.repeat(z.astype(np.float64), 64, axis=1)
    ok_zone = (zc > 0) & (zc < 15)
    err = np.abs(deq - wf)
    assert np.all(err[ok_zone] <= 0.5 * step[ok_zone] * (1 + 1e-6) + 1e-12)
    # the constant zero group dequantizes to exactly zero
    assert np.all(deq[3, :64] == 0.0)


def test_forward_two_formulations_and_brute_force():
    rng = np.random.default_rng(2)
    M, N, K = 3, 5, 128
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    bb = (0.01 * rng.standard_normal(N)).astype(np.float32)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    bias = (bb.view(np.uint32) >> 16).astype(np.uint16)
    codes, s, z = O.awq_quantize(wb)
    Y1 = O.awq_forward(xb, codes, s, z, bias)
    Y2 = O.awq_forward_dequant(xb, codes, s, z, bias)
    assert np.allclose(Y1, Y2, rtol=1e-12, atol=1e-12)
    q = O.unpack_nibbles(codes)
    xf = O.bf16_to_f32(xb)
    bf = O.bf16_to_f32(bias)
    for m in range(M):
        for n in range(N):
            acc = float(bf[n])
            for k in range(K):
                g = k // 64
                acc += float(s[n, g]) * (int(q[n, k]) - int(z[n, g])) * float(xf[m, k])
            assert abs(acc - Y1[m, n]) <= 1e-12 * (1 + abs(acc))


@pytest.mark.parametrize("bad", ["levels16", "zero_sign", "no_floor"])
def test_mutations_fail_a_pin(bad):
    """A planted mistake in a copy of the packer breaks the exact-grid pin
    (the constant-group pin for the missing floor)."""
    rng = np.random.default_rng(0)
    N, K = 4, 128
    G = K // 64
    s0 = np.full((N, G), 2.0 ** -6, np.float32)
    z0 = rng.integers(1, 15, (N, G))
    q = rng.integers(0, 16, (N, G, 64))
    q[:, :, 0], q[:, :, 1] = 0, 15
    w = (s0[:, :, None] * (q - z0[:, :, None])).astype(np.float32).reshape(N, K)
    w[0, :64] = 0.0
    W = w.reshape(N, G, 64)

    def packer(Wg):
        mx, mn = Wg.max(axis=2), Wg.min(axis=2)
        d = (mx - mn).astype(np.float32)
        if bad != "no_floor":
            d = np.maximum(d, np.float32(1e-5))
        s = (d / np.float32(16.0 if bad == "levels16" else 15.0)).astype(np.float32)
        zq = (mn if bad == "zero_sign" else -mn) / s
        z = np.clip(np.rint(zq.astype(np.float32)), 0, 15)
        qq = np.clip(np.rint((Wg / s[:, :, None]).astype(np.float32)) + z[:, :, None], 0, 15)
        return s, z, qq

    with np.errstate(divide="ignore", invalid="ignore"):
        s, z, qq = packer(W)
    deq = s[:, :, None] * (qq - z[:, :, None])
    recovered = np.array_equal(deq[1:], W[1:].astype(np.float64)) and np.all(np.isfinite(deq[0]))
    assert not recovered
