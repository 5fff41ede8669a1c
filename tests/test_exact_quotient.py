"""The exact-quotient claim the activation pass rests on, checked on the CPU.

The pass forms fp32(a / b) for a bf16 numerator a and an fp32 divisor b (the
smoothing x / lambda, the INT4 code argument x_hat / s, the NVFP4 code
argument x_hat / fp32(s g)) as fp32(fp64(a) * fp64(1 / b)) instead of a
division per element.  That equals the correctly rounded fp32 quotient
because a / b (8 significant bits over 24) is never an fp32 rounding midpoint
unless it is exact, and otherwise lies about 2^-48 (relative) or more from
every midpoint, while the fp64 product is within 2^-52 of a / b.  This test
checks the identity directly against IEEE fp32 division (numpy's float32
divide is one correctly rounded operation) for every finite bf16 numerator
and a sample of divisors chosen where the argument is tightest: subnormal
divisors, all-ones significands, powers of two, INT4 scales fp32(m / 7) and
NVFP4 divisors fp32(s g) with s an E4M3 value.  The reciprocal must be the
correctly rounded fp64 1 / b (an IEEE division, as the kernels compute it):
one ulp off, the product misrounds quotients that are exact fp32 midpoints
in the subnormal range (power-of-two divisors, whose reciprocal is exact);
the last test pins that."""
import numpy as np


def _all_finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]                       # drop inf / NaN
    return (b << 16).view(np.float32)


def _divisors(rng) -> np.ndarray:
    parts = []
    # subnormals: the smallest ones, all-ones, random
    sub = np.concatenate([np.arange(1, 64, dtype=np.uint32), [0x7FFFFF, 0x400000, 0x000001],
                          rng.integers(1, 1 << 23, 1000, dtype=np.uint32)])
    parts.append(sub.astype(np.uint32).view(np.float32))
    # all-ones significands and powers of two at every exponent step of 4
    e = np.arange(1, 255, 4, dtype=np.uint32) << 23
    parts.append((e | 0x7FFFFF).view(np.float32))
    parts.append(e.view(np.float32))
    # random normal patterns across the whole range
    rnd = (rng.integers(1, 255, 3000, dtype=np.uint32) << 23) | rng.integers(0, 1 << 23, 3000,
                                                                               dtype=np.uint32)
    parts.append(rnd.view(np.float32))
    # INT4 group scales s = fp32(absmax / 7) for bf16 maxima
    am = _all_finite_bf16()
    am = np.abs(am[(am != 0)])
    parts.append((rng.choice(am, 1000) / np.float32(7.0)).astype(np.float32))
    # NVFP4: d = fp32(s g) with s an E4M3 value and g = fp32(amax / 2688)
    e4m3 = np.array([(1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7) if (c >> 3) else (c & 7) * 2.0 ** -9
                     for c in range(1, 127)], np.float64)
    g = (rng.uniform(1e-3, 1e3, 1000) / 2688.0).astype(np.float32)
    parts.append((rng.choice(e4m3, 1000).astype(np.float32) * g).astype(np.float32))
    d = np.concatenate(parts).astype(np.float32)
    return d[np.isfinite(d) & (d > 0)]


def test_fp64_reciprocal_product_is_the_fp32_quotient():
    rng = np.random.default_rng(2024)
    a32 = _all_finite_bf16()
    a64 = a32.astype(np.float64)
    divs = _divisors(rng)
    assert divs.size > 6000
    bad = 0
    with np.errstate(over="ignore", under="ignore", divide="ignore", invalid="ignore"):
        for i in range(0, divs.size, 64):
            b32 = divs[i:i + 64]
            ref = a32[None, :] / b32[:, None]                       # IEEE fp32 division
            r = 1.0 / b32.astype(np.float64)                        # correctly rounded fp64
            got = (a64[None, :] * r[:, None]).astype(np.float32)
            bad += int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
    assert bad == 0, f"{bad} quotients differ from the IEEE fp32 division"


def test_a_direct_fp32_reciprocal_would_not_do():
    """Negative control: fp32(a * fp32(1 / b)) (a reciprocal rounded to fp32)
    differs from the fp32 quotient for some of the same pairs, so the check
    above can tell a wrong scheme from the right one."""
    rng = np.random.default_rng(7)
    a32 = _all_finite_bf16()
    b32 = _divisors(rng)[:200]
    with np.errstate(over="ignore", under="ignore", divide="ignore", invalid="ignore"):
        ref = a32[None, :] / b32[:, None]
        got = a32[None, :] * (np.float32(1.0) / b32)[:, None]
    assert np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)) > 0


def test_a_reciprocal_one_ulp_low_misrounds_exact_subnormal_midpoints():
    """Why the reciprocal has to be correctly rounded: for b = 2^18, 1 / b is
    exact, a / b can be exactly half-way between two fp32 subnormals, and a
    reciprocal one fp64 ulp low pushes the product below the midpoint."""
    b = np.float32(2.0 ** 18)
    a = np.float32(1.5 * 2.0 ** -149 * 2.0 ** 18)       # a / b = 1.5 * 2^-149 exactly
    assert float(a) == 1.5 * 2.0 ** -131                  # a is a bf16 value (2 significant bits)
    with np.errstate(under="ignore"):
        ref = a / b                                       # ties to even: 2 * 2^-149
        r = 1.0 / np.float64(b)
        exact = np.float32(np.float64(a) * r)
        low = np.float32(np.float64(a) * np.nextafter(r, 0.0))
    assert exact.view(np.uint32) == ref.view(np.uint32) == 2
    assert low.view(np.uint32) == 1


def test_int4_scale_is_the_fp64_product_with_one_seventh():
    """The INT4 group scale s = fp32(amax / 7) is formed as the fp64 product of
    amax with the correctly rounded fp64 1/7 (an instance of the identity
    above, 7 being the divisor): equal for every finite bf16 amax."""
    am = np.abs(_all_finite_bf16())
    ref = am / np.float32(7.0)
    got = (am.astype(np.float64) * (1.0 / 7.0)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_int4_codes_need_neither_the_clamp_nor_an_exact_reciprocal_of_s():
    """For INT4 codes rint_even(clamp(fp32(x_hat / s), -8, 7)) with s = fp32(amax
    / 7) and |x_hat| <= amax: the clamp never acts (|fp32(x_hat / s)| < 7.0004),
    and a reciprocal of s up to 8 fp64 ulps off the correctly rounded one
    gives the same codes, so the kernel may take 1/s from the hardware
    reciprocal with Newton steps.  Every finite bf16 x_hat up to amax, for
    amax at the smallest subnormals, the largest finite values and a sample in
    between."""
    rng = np.random.default_rng(3)
    a32 = _all_finite_bf16()
    mags = np.unique(np.abs(a32[a32 != 0]))
    amaxes = np.concatenate([mags[:8], mags[-4:], rng.choice(mags, 48, replace=False)])
    worst = 0.0
    with np.errstate(over="ignore", under="ignore"):
        for amax in amaxes:
            s = np.float32(amax) / np.float32(7.0)
            x = a32[np.abs(a32) <= amax]
            q = x / s                                            # IEEE fp32 quotient
            worst = max(worst, float(np.max(np.abs(q))))
            ref = np.rint(np.clip(q, -8, 7))
            r = 1.0 / np.float64(s)
            for k in (-8, -3, -1, 1, 3, 8):
                rk = r
                for _ in range(abs(k)):
                    rk = np.nextafter(rk, np.inf if k > 0 else 0.0)
                got = np.rint((x.astype(np.float64) * rk).astype(np.float32))
                assert np.array_equal(got, ref), (float(amax), k)
    assert worst < 7.0004
