"""Pins of the NVFP4 oracle (CPU): E4M3 encoding against its decode table
and torch's float8_e4m3fn conversion, the block quantizer's invariants and
error bound, the two formulations of the product, and planted mistakes."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle.nvfp4_oracle as NV


def test_e4m3_round_trip_of_every_finite_code():
    b = np.arange(0, 0x7F, dtype=np.uint8)
    v = O.e4m3_decode(b)
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(O.e4m3_encode(v), b)


def test_e4m3_matches_torch_below_saturation():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(0, 448, 20000), np.exp(rng.uniform(-14, 6, 20000)),
                        (O.e4m3_decode(np.arange(0, 0x7E)) + O.e4m3_decode(np.arange(1, 0x7F))) / 2])
    v = v.astype(np.float32)
    v = v[v <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_e4m3_saturates_and_ties_to_even():
    assert np.array_equal(O.e4m3_encode(np.array([448.0, 460.0, 464.0, 1e30])), [0x7E] * 4)
    # 1 + 1/16 lies between 1 (m = 0) and 1.125 (m = 1): even mantissa wins
    assert O.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert O.e4m3_encode(np.array([1.1875]))[0] == 0x3A   # between m = 1 and m = 2


def test_global_scale():
    assert NV.nvfp4_global_scale(2688.0) == np.float32(1.0)
    assert NV.nvfp4_global_scale(0.0) == np.float32(1.0)


def _blocks(seed, rows=64, K=256):
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-3, 3, (rows, 1)))).astype(np.float32)
    V[3, 16:32] = 0.0                                   # a zero block
    return V


def test_quantizer_invariants_and_error_bound():
    V = _blocks(1)
    g = NV.nvfp4_global_scale(float(np.abs(V).max()))
    codes, sb = O.quantize_nvfp4(V, g)
    assert codes.max() <= 15 and sb.max() <= 0x7E
    s = O.e4m3_decode(sb)
    mag = O.E2M1_GRID[codes.reshape(64, -1, 16) & 7]
    # a zero block: scale 0 and all codes +0
    assert sb[3, 1] == 0 and not codes[3, 16:32].any()
    # blocks with a normal scale reach the top of the E2M1 grid
    normal = (sb >= 0x08) & (sb < 0x7E)
    assert np.all(mag.max(axis=2)[normal] == 6.0)
    # each value within half an E2M1 step of its block's grid, times d = s g
    d = (s.astype(np.float32) * g).astype(np.float32)
    y = V.reshape(64, -1, 16) / np.where(d > 0, d, 1)[:, :, None]
    c = np.where(codes.reshape(64, -1, 16) & 8, -mag, mag)
    half = np.where(np.abs(c) < 2, 0.25, np.where(np.abs(c) < 4, 0.5, 1.0))
    err = np.abs(y - c)
    ok = (err <= half * (1 + 1e-6)) | (np.abs(c) == 6) & (np.abs(y) >= 6)
    assert np.all(ok[d > 0])
    # signs are kept
    assert np.all((codes.reshape(64, -1, 16) >> 3)[(V.reshape(64, -1, 16) > 0)] == 0)


def test_two_formulations_of_the_product():
    rng = np.random.default_rng(2)
    X = _blocks(3, rows=40, K=128)
    W = _blocks(4, rows=24, K=128)
    gx = NV.nvfp4_global_scale(float(np.abs(X).max()))
    gw = NV.nvfp4_global_scale(float(np.abs(W).max()))
    xc, xs = O.quantize_nvfp4(X, gx)
    wc, ws = O.quantize_nvfp4(W, gw)
    xc, wc = O.pack_nibbles(xc), O.pack_nibbles(wc)
    T = rng.standard_normal((40, 16))
    L2 = O.f32_to_bf16(rng.standard_normal((16, 24)).astype(np.float32))
    b = O.f32_to_bf16(rng.standard_normal(24).astype(np.float32))
    Y1 = O.nvfp4_forward(xc, xs, gx, T, wc, ws, gw, L2, b)
    Y2 = O.nvfp4_forward_dequant(xc, xs, gx, T, wc, ws, gw, L2, b)
    assert np.allclose(Y1, Y2, rtol=1e-12, atol=1e-12 * np.abs(Y2).max())
    # the dequantized operands are no further from X than MXFP4's (blocks of
    # 16 with E4M3 scales against blocks of 32 with powers of two)
    Dx = O.decode_nvfp4(xc, xs, gx)
    mc, ms = O.quantize_fp4(X)
    Mx = O.decode_fp4(O.pack_nibbles(mc)) * np.repeat(np.ldexp(1.0, ms.astype(np.int64) - 127),
                                                      32, axis=1)
    assert np.linalg.norm(Dx - X) <= 1.05 * np.linalg.norm(Mx - X)
    assert np.linalg.norm(Dx - X) <= 0.12 * np.linalg.norm(X)


@pytest.mark.parametrize("bug", ["floor", "half_up"])
def test_mutations_fail_a_pin(bug, monkeypatch):
    monkeypatch.setattr(NV, "_rne", np.floor if bug == "floor" else (lambda x: np.floor(x + 0.5)))
    mid = ((O.e4m3_decode(np.arange(0, 0x7E)) + O.e4m3_decode(np.arange(1, 0x7F))) / 2)
    v = np.concatenate([np.random.default_rng(0).uniform(0, 448, 2000), mid]).astype(np.float32)
    got = NV.e4m3_encode(v)
    monkeypatch.undo()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(got, ref)
