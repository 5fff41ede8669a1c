"""Exhaustive sweeps of the activation quantizers through the C ABI against
the oracle, bit for bit (codes, scales, and the decoded image).

FP4: for every block exponent e the image can hold (-127 .. 125) a set of
blocks whose maximum fixes e and whose other elements run through every bf16
value with magnitude in [2^(e-3), 2^(e+3)) (where the E2M1 decision is made)
plus signed zeros, the smallest subnormals and values far below the grid, so
every rounding tie, the saturation at 6 and the sign of zeros are exercised
at every scale.
INT4: groups with maximum 7 (scale exactly 1, so the code is the rounded
value itself) running through every bf16 value in [-7, 7], every tie
k + 1/2 included, and groups with maximum 3.5 (scale 1/2) and a random
fractional scale.

lambda is 1 and the rank 0, so X_hat = X and the outputs are the codes and
scales alone."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from image_decode import decode_act_image
from layer_util import np_

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bf16_values(lo_exp, hi_exp):
    """Every bf16 bit pattern with biased exponent in [lo_exp, hi_exp], both signs."""
    e = np.arange(max(lo_exp, 0), min(hi_exp, 254) + 1, dtype=np.uint32)
    m = np.arange(128, dtype=np.uint32)
    pos = ((e[:, None] << 7) | m[None, :]).ravel()
    return np.concatenate([pos, pos | 0x8000]).astype(np.uint16)


def _fp4_sweep_rows(K):
    """Rows of bf16 bits: blocks of 32, each [setter, 31 sweep values]."""
    blocks = []
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0040, 0x8040, 0x007F, 0x807F],
                        np.uint16)
    for e in range(-127, 126):
        setter = np.uint16(((e + 2 + 127) & 0xFF) << 7) if e > -127 else np.uint16(2 << 7)
        # e = -127: maximum 2^-125 (biased exponent 2)
        lo, hi = e + 127 - 3, e + 127 + 2          # biased exponents of [2^(e-3), 2^(e+3))
        if e == -127:
            lo, hi = 0, 2
        vals = np.concatenate([_bf16_values(lo, hi), specials])
        # keep every value at most the setter in magnitude
        mag = vals & 0x7FFF
        vals = vals[mag <= (setter & 0x7FFF)]
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((len(vals), 1), setter, np.uint16), vals], axis=1))
    b = np.concatenate(blocks)                                   # [nblocks][32]
    per_row = K // 32
    pad = (-len(b)) % per_row
    b = np.concatenate([b, np.zeros((pad, 32), np.uint16)])
    return b.reshape(-1, K)


def _int4_sweep_rows(K, rng):
    vals = _bf16_values(0, 129)                                  # |v| < 4 ... up to exponent 129
    f = O.bf16_to_f32(vals)
    vals = vals[np.isfinite(f) & (np.abs(f) <= 7.0)]
    groups = []
    for setter in (0x40E0, 0xC0E0, 0x4060):                      # 7.0, -7.0, 3.5
        lim = abs(float(O.bf16_to_f32(np.array([setter], np.uint16))[0]))
        v = vals[np.abs(O.bf16_to_f32(vals)) <= lim]
        pad = (-len(v)) % 63
        v = np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(-1, 63)
        groups.append(np.concatenate([np.full((len(v), 1), setter, np.uint16), v], axis=1))
    # random fractional scales: a random maximum, the rest below it
    r = rng.standard_normal((512, 64)).astype(np.float32) * np.float32(3.0)
    groups.append(O.f32_to_bf16(r))
    g = np.concatenate(groups)
    per_row = K // 64
    pad = (-len(g)) % per_row
    g = np.concatenate([g, np.zeros((pad, 64), np.uint16)])
    return g.reshape(-1, K)


def _run(mode, xb):
    from bit_diffusion_transformer_quantize_amd import svdq as S
    M, K = xb.shape
    lam = np.ones(K, np.float32)
    xc_o, xs_o, _, _ = O.quantize_act(xb, lam, None, mode)
    d = S.desc(mode, K, 128, 0)
    X = WL.from_bits(xb).to(DEV)
    xc, xs, _, ximg = S.svdq_quantize_act(d, X, torch.from_numpy(lam).to(DEV), None, codes=True)
    torch.cuda.synchronize()
    assert np.array_equal(np_(xs), xs_o), f"{mode} scales"
    got = np_(xc)
    bad = np.nonzero(got != xc_o)
    assert bad[0].size == 0, (f"{mode}: {bad[0].size} code bytes differ, first at row {bad[0][0]} "
                              f"byte {bad[1][0]}: got {got[bad][0]:#04x} want {xc_o[bad][0]:#04x}")
    img = decode_act_image(np_(ximg), mode, M, K, 0)
    assert np.array_equal(img["codes"][:M], xc_o), f"{mode} image codes"


def test_fp4_every_scale_and_value():
    xb = _fp4_sweep_rows(1024)
    print("[case] fp4 sweep", xb.shape, flush=True)
    _run("fp4", xb)


def test_int4_ties_and_every_value_below_seven():
    xb = _int4_sweep_rows(1024, np.random.default_rng(5))
    print("[case] int4 sweep", xb.shape, flush=True)
    _run("int4", xb)
