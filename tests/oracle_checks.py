"""Pins for the CPU oracle: each check compares the oracle with something that
the pages or the mathematics fix independently of its code (hand-derived
fixtures, exact rational replays, closed forms, invariants, reductions to a
textbook routine, brute force).  Every check raises AssertionError on a
mismatch; ``test_oracle_pins.py`` runs them and ``test_oracle_mutations.py``
plants mistakes in the oracle and checks that at least one of them fails.

The oracle module is looked up at call time so that a patched attribute is
the one exercised.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import exact_fp as xf
import oracle.svdq_oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_to_bf16_bits(vals):
    return np.array([np.float32(v).view(np.uint32) >> 16 for v in vals], np.uint16)


# ---------------------------------------------------------------- bf16 RNE
def check_bf16_rne_vs_torch(n=1 << 20, seed=0):
    """Bit-twiddled RNE == torch's fp32 -> bf16 cast, on random fp32 patterns
    (all exponents, subnormals included) and on every exact tie pattern."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, 1 << 16, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, np.arange(0, 1 << 17, dtype=np.uint32)])
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f32_to_bf16(x)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"bf16 RNE mismatch at {x[bad[:5]]}"
    # widening is exact
    back = O.bf16_to_f32(got)
    assert np.array_equal(back, ref.astype(np.uint32).__lshift__(16).view(np.float32))


# ---------------------------------------------------------------- INT4
def check_int4_golden():
    g = _load("int4_groups.json")
    G = g["group"]
    for case in g["cases"]:
        vals = case["values"] + [0.0] * (G - len(case["values"]))
        q, s = O.quantize_int4(np.array([vals], np.float32))
        n = len(case["codes"])
        assert float(s[0, 0]) == case["scale"], (case["name"], s[0, 0])
        assert q[0, :n].tolist() == case["codes"], (case["name"], q[0, :n].tolist())


def _random_groups(rng, ngroups, G):
    out = []
    for i in range(ngroups):
        kind = i % 6
        if kind == 0:      # ordinary normals
            v = rng.standard_normal(G)
        elif kind == 1:    # subnormal range
            v = rng.standard_normal(G) * 2.0 ** -140
        elif kind == 2:    # all zero
            v = np.zeros(G)
        elif kind == 3:    # exact ties: absmax 7*2^j and values (k+1/2)*2^j
            j = int(rng.integers(-10, 10))
            v = (rng.integers(-7, 7, G) + 0.5) * 2.0 ** j
            v[0] = 7 * 2.0 ** j
        elif kind == 4:    # one outlier
            v = rng.standard_normal(G)
            v[int(rng.integers(G))] *= 300
        else:              # tiny groups that push the scale to the last subnormals
            v = rng.integers(-8, 9, G) * 2.0 ** -149
        out.append(np.asarray(v, np.float32))
    return np.stack(out)


def check_int4_replay(seed=0, ngroups=60, bf16_inputs=False):
    """Oracle codes and scales == an exact rational replay of the quantizer."""
    rng = np.random.default_rng(seed)
    V = _random_groups(rng, ngroups, 64)
    if bf16_inputs:
        V = O.bf16_to_f32(O.f32_to_bf16(V))
    q, s = O.quantize_int4(V.reshape(ngroups // 2, 128))
    q = q.reshape(ngroups, 64)
    s = s.reshape(ngroups)
    for i in range(ngroups):
        es, ec = xf.int4_group([float(x) for x in V[i]])
        assert Fraction(float(s[i])) == es, (i, float(s[i]), float(es))
        assert q[i].tolist() == ec, (i, q[i].tolist(), ec)


def check_int4_invariants(seed=0):
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    V[3, :64] = 0
    q, s = O.quantize_int4(V)
    qg = q.reshape(64, 4, 64).astype(np.int64)
    Vg = V.reshape(64, 4, 64).astype(np.float64)
    nz = s > 0
    assert np.all(np.abs(qg) <= 7)                                  # normal-range scales
    assert np.all(np.abs(qg).max(axis=2)[nz] == 7)                  # absmax maps to 7
    assert np.all(qg[~nz] == 0)
    err = np.abs(Vg - qg * s[:, :, None].astype(np.float64))
    assert np.all(err <= (s[:, :, None] / 2) * (1 + 2.0 ** -20))    # half-step bound
    qn, sn = O.quantize_int4(-V)                                    # odd symmetry
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


# ---------------------------------------------------------------- FP4
def check_fp4_golden():
    g = _load("e2m1_blocks.json")
    B = g["block"]
    for case in g["cases"]:
        vals = case["values"] + [0.0] * (B - len(case["values"]))
        c, sb = O.quantize_fp4(np.array([vals], np.float32))
        n = len(case["codes"])
        assert int(sb[0, 0]) == case["scale_byte"], (case["name"], sb[0, 0])
        assert c[0, :n].tolist() == case["codes"], (case["name"], c[0, :n].tolist())


def check_fp4_replay(seed=0, nblocks=60):
    rng = np.random.default_rng(seed)
    V = _random_groups(rng, nblocks, 32)
    V[5, 3] = -0.0
    c, sb = O.quantize_fp4(V.reshape(nblocks // 2, 64))
    c = c.reshape(nblocks, 32)
    sb = sb.reshape(nblocks)
    for i in range(nblocks):
        eb, ec = xf.fp4_block([float(x) for x in V[i]])
        assert int(sb[i]) == eb, (i, int(sb[i]), eb)
        assert c[i].tolist() == ec, (i, c[i].tolist(), ec)


def check_fp4_invariants(seed=0):
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-20, 20, (32, 1)))).astype(np.float32)
    c, sb = O.quantize_fp4(V)
    mag = (c & 7).reshape(32, 8, 32)
    e = sb.astype(np.int64) - 127
    unclamped = (e > -127) & (e < 127)
    assert np.all(np.isin(mag.max(axis=2)[unclamped], [6, 7]))      # top code is 4 or 6
    # dequantization is exact on grid points: re-quantizing the dequantized block
    # returns the same codes and scale
    deq = (O.decode_fp4(O.pack_nibbles(c)) * np.repeat(np.ldexp(1.0, e), 32, axis=1)).astype(np.float32)
    c2, sb2 = O.quantize_fp4(deq)
    nzb = np.repeat(mag.max(axis=2) > 0, 32, axis=1)
    assert np.array_equal((c2 & 7)[nzb], (c & 7)[nzb])


# ---------------------------------------------------------------- smoothing
def check_lambda(seed=0):
    """lambda within one fp32 ulp of the exact sqrt(ax/aw); exact special cases."""
    rng = np.random.default_rng(seed)
    X = O.f32_to_bf16((rng.standard_normal((16, 40)) * np.exp(rng.uniform(-5, 5, 40))).astype(np.float32))
    W = O.f32_to_bf16((rng.standard_normal((24, 40)) * np.exp(rng.uniform(-5, 5, 40))).astype(np.float32))
    X[:, 0] = 0                                                      # zero channel -> 1
    X[:, 1] = _f32_to_bf16_bits([8.0] * 16)                          # ax = 8, aw = 2 -> 2
    W[:, 1] = _f32_to_bf16_bits([2.0] * 24)
    W[:, 2] = 0                                                      # zero column -> 1
    lam = O.calibrate_lambda(X, W)
    assert lam.dtype == np.float32
    assert lam[0] == 1 and lam[2] == 1 and lam[1] == 2
    ax = np.abs(O.bf16_to_f32(X)).max(0)
    aw = np.abs(O.bf16_to_f32(W)).max(0)
    for j in range(3, 40):
        r = Fraction(float(ax[j])) / Fraction(float(aw[j]))
        l = Fraction(float(lam[j]))
        ulp = Fraction(2) ** (xf.floor_log2(l) - 23)
        assert (l - ulp) ** 2 <= r <= (l + ulp) ** 2, j


def check_smoothing_balance():
    """After smoothing, each channel's activation max equals its weight max
    (both sqrt(ax*aw)) up to bf16/fp32 rounding, and X_hat W_hat^T stays
    X W^T up to that rounding."""
    X, W, _ = WL.draw(WL.TINY)
    xb, wb = WL.bits(X), WL.bits(W)
    lam = O.calibrate_lambda(xb, wb)
    Xh = O.bf16_to_f32(O.smooth_act(xb, lam)).astype(np.float64)
    Wh = O.smooth_weight(wb, lam).astype(np.float64)
    ax = np.abs(O.bf16_to_f32(xb)).max(0).astype(np.float64)
    aw = np.abs(O.bf16_to_f32(wb)).max(0).astype(np.float64)
    tgt = np.sqrt(ax * aw)
    assert np.allclose(np.abs(Xh).max(0), tgt, rtol=2.0 ** -7)
    assert np.allclose(np.abs(Wh).max(0), tgt, rtol=2.0 ** -20)
    ref = O.bf16_to_f32(xb).astype(np.float64) @ O.bf16_to_f32(wb).astype(np.float64).T
    got = Xh @ Wh.T
    assert np.linalg.norm(got - ref) <= 2.0 ** -8 * np.linalg.norm(ref)


# ---------------------------------------------------------------- reductions
def _textbook_fake_quant_int4(x: torch.Tensor) -> torch.Tensor:
    """Plain symmetric per-group (64) INT4 fake quantization in torch."""
    rows, K = x.shape
    g = x.float().reshape(rows, K // 64, 64)
    s = g.abs().amax(dim=2, keepdim=True) / 7.0
    q = torch.where(s > 0, torch.round(g / torch.where(s > 0, s, torch.ones_like(s))).clamp(-8, 7),
                    torch.zeros_like(g))
    return (q.double() * s.double()).reshape(rows, K)


def _textbook_fake_quant_mxfp4(x: torch.Tensor) -> torch.Tensor:
    """Plain MXFP4 fake quantization in torch: per 32, scale 2^(floor(log2
    amax) - 2), nearest E2M1 value (ties to even code), saturate at 6."""
    rows, K = x.shape
    g = x.double().reshape(rows, K // 32, 32)
    amax = g.abs().amax(dim=2, keepdim=True)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    y = g / torch.pow(2.0, e)
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    d = (y.abs().unsqueeze(-1) - grid).abs()
    # ties: prefer the even index by penalising odd indices by a hair
    idx = torch.argmin(d + 1e-9 * (torch.arange(8) % 2), dim=-1)
    return (torch.sign(y) * grid[idx] * torch.pow(2.0, e)).reshape(rows, K)


def check_reduction_plain_w4a4(mode="int4"):
    """With r = 0 and lambda = 1 the layer is plain per-group W4A4 fake
    quantization of X and W followed by a matmul and the bias."""
    X, W, b = WL.draw(WL.TINY, M=64)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    K = xb.shape[1]
    lam = np.ones(K, np.float32)
    L1 = np.zeros((K, 0), np.uint16)
    L2 = np.zeros((0, wb.shape[0]), np.uint16)
    wc, ws = O.pack_weight(wb, lam, L1, L2, mode)
    xc, xs, T, _ = O.quantize_act(xb, lam, None, mode)
    Y = O.forward(xc, xs, T, wc, ws, L2, bb, mode)
    fq = _textbook_fake_quant_int4 if mode == "int4" else _textbook_fake_quant_mxfp4
    ref = (fq(X) @ fq(W).T + b.double()).numpy()
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _zero_residual_case(mode, seed=3, M=8, K=128, N=16, r=4):
    rng = np.random.default_rng(seed)
    L1 = rng.integers(-3, 4, (K, r)).astype(np.float32)
    L2 = rng.integers(-3, 4, (r, N)).astype(np.float32)
    lam = np.ldexp(1.0, rng.integers(-2, 3, K)).astype(np.float32)
    Wt = (L1 @ L2) / lam[:, None]                 # K x N, exact small dyadics
    W = O.f32_to_bf16(Wt.T.astype(np.float32))
    assert np.array_equal(O.bf16_to_f32(W), Wt.T.astype(np.float32))
    X = O.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    b = O.f32_to_bf16(0.01 * rng.standard_normal(N).astype(np.float32))
    return X, W, b, lam, O.f32_to_bf16(L1), O.f32_to_bf16(L2)


def check_zero_residual(mode="int4"):
    """W = (L1 L2)^T / lambda with power-of-two lambda: the residual is
    exactly zero, all weight codes and scales vanish, and the layer returns
    X W^T + b exactly."""
    X, W, b, lam, L1, L2 = _zero_residual_case(mode)
    wc, ws = O.pack_weight(W, lam, L1, L2, mode)
    assert np.all(wc == 0) and np.all(ws == 0)
    xc, xs, T, _ = O.quantize_act(X, lam, L1, mode)
    Y = O.forward(xc, xs, T, wc, ws, L2, b, mode)
    ref = (O.bf16_to_f32(X).astype(np.float64) @ O.bf16_to_f32(W).astype(np.float64).T
           + O.bf16_to_f32(b).astype(np.float64))
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)


def check_eckart_young():
    """For the rank-r factors: no rank-r matrix beats the tail energy
    sum_{i>r} s_i^2 (Eckart-Young), the bf16 factors stay within bf16
    rounding of it, the split is balanced (||L1[:, i]|| = ||L2[i, :]|| =
    sqrt(s_i)), and sum s_i^2 = ||W_hat||_F^2."""
    X, W, _ = WL.draw(WL.TINY)
    xb, wb = WL.bits(X), WL.bits(W)
    lam = O.calibrate_lambda(xb, wb)
    Wh = O.smooth_weight(wb, lam).astype(np.float64)
    for r in (1, 4, 16):
        L1, L2, S = O.lowrank_factors(Wh, r)
        assert L1.shape == (Wh.shape[1], r) and L2.shape == (r, Wh.shape[0])
        A = O.bf16_to_f32(L1).astype(np.float64) @ O.bf16_to_f32(L2).astype(np.float64)
        err = np.linalg.norm(Wh.T - A)
        tail = math.sqrt(float(np.sum(S[r:] ** 2)))
        head = math.sqrt(float(np.sum(S[:r] ** 2)))
        assert err >= tail * (1 - 1e-12)
        assert err <= tail + 2.0 ** -7 * head
        assert np.allclose(np.linalg.norm(O.bf16_to_f32(L1), axis=0), np.sqrt(S[:r]), rtol=2.0 ** -7)
        assert np.allclose(np.linalg.norm(O.bf16_to_f32(L2), axis=1), np.sqrt(S[:r]), rtol=2.0 ** -7)
    assert np.isclose(np.sum(S ** 2), np.sum(Wh ** 2), rtol=1e-12)


def check_two_formulations(mode="int4"):
    """Per-group integer sums then scales == dequantize then one fp64 matmul."""
    X, W, b = WL.draw(WL.TINY, M=48)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam = O.calibrate_lambda(xb, wb)
    L1, L2, _ = O.lowrank_factors(O.smooth_weight(wb, lam), 8)
    wc, ws = O.pack_weight(wb, lam, L1, L2, mode)
    xc, xs, T, _ = O.quantize_act(xb, lam, L1, mode)
    Y1 = O.forward(xc, xs, T, wc, ws, L2, bb, mode)
    Y2 = O.forward_dequant(xc, xs, T, wc, ws, L2, bb, mode)
    assert np.allclose(Y1, Y2, rtol=1e-12, atol=1e-12 * np.abs(Y2).max())


# ---------------------------------------------------------------- brute force
def _bf(vals_bits):
    return [Fraction(float(v)) for v in O.bf16_to_f32(np.asarray(vals_bits, np.uint16)).ravel()]


def check_pipeline_bruteforce(mode="int4", seed=0, M=3, K=128, N=4, r=2):
    """Scalar exact-rational replay of the whole layer (smoothing, residual,
    quantizers, nibble packing, main product, low-rank branch, bias) on a tiny
    shape, compared with the vectorised oracle."""
    rng = np.random.default_rng(seed)
    Xf = rng.standard_normal((M, K)).astype(np.float32)
    Xf[:, 5] *= 40
    Wf = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    Wf[:, 9] *= 10
    X = O.f32_to_bf16(Xf)
    W = O.f32_to_bf16(Wf)
    b = O.f32_to_bf16((0.01 * rng.standard_normal(N)).astype(np.float32))
    L1 = O.f32_to_bf16((0.05 * rng.standard_normal((K, r))).astype(np.float32))
    L2 = O.f32_to_bf16((0.05 * rng.standard_normal((r, N))).astype(np.float32))
    G = 64 if mode == "int4" else 32

    # --- scalar replay -------------------------------------------------
    Xq = [_bf(X[m]) for m in range(M)]
    Wq = [_bf(W[n]) for n in range(N)]
    L1q = [[Fraction(float(v)) for v in O.bf16_to_f32(L1[k])] for k in range(K)]
    L2q = [[Fraction(float(v)) for v in O.bf16_to_f32(L2[i])] for i in range(r)]
    bq = _bf(b)
    lam = []
    for k in range(K):
        ax = max(abs(Xq[m][k]) for m in range(M))
        aw = max(abs(Wq[n][k]) for n in range(N))
        if ax == 0 or aw == 0:
            lam.append(Fraction(1))
        else:
            lam.append(xf.rn_f32(Fraction(math.sqrt(float(ax) / float(aw)))))
    Xh = [[xf.rn_bf16(xf.rn_f32(Xq[m][k] / lam[k])) for k in range(K)] for m in range(M)]
    R = []
    for n in range(N):
        row = []
        for k in range(K):
            wh = xf.rn_f32(Wq[n][k] * lam[k])
            acc = Fraction(0)
            for i in range(r):
                acc = xf.rn_f32(acc + L1q[k][i] * L2q[i][n])
            row.append(xf.rn_f32(wh - acc))
        R.append(row)

    def quant_rows(rows):
        codes, scales = [], []
        for row in rows:
            c_row, s_row = [], []
            for g0 in range(0, K, G):
                grp = [float(v) for v in row[g0:g0 + G]]
                if mode == "int4":
                    s, c = xf.int4_group(grp)
                else:
                    s, c = xf.fp4_block(grp)
                c_row += c
                s_row.append(s)
            codes.append(c_row)
            scales.append(s_row)
        return codes, scales

    xc_s, xs_s = quant_rows(Xh)
    wc_s, ws_s = quant_rows(R)

    def value(code, scale):
        if mode == "int4":
            return code * scale
        mag = xf.E2M1[code & 7] * Fraction(2) ** (scale - 127)
        return -mag if code & 8 else mag

    Y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        T = [sum(Xh[m][k] * L1q[k][i] for k in range(K)) for i in range(r)]
        for n in range(N):
            y = sum(value(xc_s[m][k], xs_s[m][k // G]) * value(wc_s[n][k], ws_s[n][k // G])
                    for k in range(K))
            y += sum(T[i] * L2q[i][n] for i in range(r)) + bq[n]
            Y[m][n] = y

    def pack(codes):
        out = []
        for row in codes:
            out.append([(row[2 * j] & 0xF) | ((row[2 * j + 1] & 0xF) << 4) for j in range(K // 2)])
        return np.array(out, np.uint8)

    # --- vectorised oracle --------------------------------------------------
    lam_o = O.calibrate_lambda(X, W)
    assert [Fraction(float(v)) for v in lam_o] == lam
    wc, ws = O.pack_weight(W, lam_o, L1, L2, mode)
    xc, xs, T, Xh_o = O.quantize_act(X, lam_o, L1, mode)
    assert [[Fraction(float(v)) for v in row] for row in O.bf16_to_f32(Xh_o)] == Xh
    assert np.array_equal(wc, pack(wc_s)) and np.array_equal(xc, pack(xc_s))
    if mode == "int4":
        assert [[Fraction(float(v)) for v in row] for row in ws] == ws_s
        assert [[Fraction(float(v)) for v in row] for row in xs] == xs_s
    else:
        assert ws.tolist() == ws_s and xs.tolist() == xs_s
    Yo = O.forward(xc, xs, T, wc, ws, L2, b, mode)
    Ye = np.array([[float(v) for v in row] for row in Y])
    assert np.allclose(Yo, Ye, rtol=1e-12, atol=1e-12 * np.abs(Ye).max())


def check_rank_trend():
    """Weight reconstruction error ||W_hat - (L1 L2)^T - deq(R)||_F does not
    grow with the rank (the pages: higher rank, better fidelity)."""
    X, W, _ = WL.draw(WL.TINY)
    xb, wb = WL.bits(X), WL.bits(W)
    lam = O.calibrate_lambda(xb, wb)
    Wh = O.smooth_weight(wb, lam).astype(np.float64)
    errs = []
    for r in (0, 4, 16, 64):
        L1, L2, _ = O.lowrank_factors(Wh, r)
        wc, ws = O.pack_weight(wb, lam, L1, L2, "int4")
        deq = O.decode_int4(wc) * np.repeat(ws.astype(np.float64), 64, axis=1)
        lr = O.bf16_to_f32(L1).astype(np.float64) @ O.bf16_to_f32(L2).astype(np.float64)
        errs.append(np.linalg.norm(Wh - lr.T - deq))
    assert all(errs[i + 1] <= errs[i] for i in range(len(errs) - 1)), errs
