"""Shared helpers for the GPU parity tests: run one layer through the oracle
and through the C ABI on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import workloads as WL


def oracle_offline(xb, wb, rank, mode, lam=None, L1=None, L2=None, weight_rows=None):
    """lambda, L1, L2 and the packed weight (optionally only some rows)."""
    if lam is None:
        lam = O.calibrate_lambda(xb, wb)
    if L1 is None:
        L1, L2, _ = O.lowrank_factors(O.smooth_weight(wb, lam), rank)
    wsel = wb if weight_rows is None else wb[weight_rows]
    L2sel = L2 if weight_rows is None else L2[:, weight_rows]
    wc, ws = O.pack_weight(wsel, lam, L1, L2sel, mode)
    return lam, L1, L2, wc, ws


def to_dev_bf16(bits_arr, dev):
    return WL.from_bits(np.ascontiguousarray(bits_arr)).to(dev)


def gpu_run(dev, X, W, b, lam, L1, L2, mode, rank, out_f32=False, use_lowrank=True,
            calibrate_on_gpu=False):
    """Run calibrate (optional), pack, quantize and forward through the C ABI.
    Returns a dict of device tensors."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    M, K = X.shape
    N = W.shape[0]
    Xd, Wd = X.to(dev), W.to(dev)
    bd = None if b is None else b.to(dev)
    d = S.desc(mode, K, N, rank if use_lowrank else 0, out_f32=out_f32)
    if calibrate_on_gpu:
        lam_d = S.svdq_calibrate_lambda(Xd, Wd)
    else:
        lam_d = torch.from_numpy(np.ascontiguousarray(lam)).to(dev)
    ld = lu = None
    if use_lowrank and rank > 0:
        ld = to_dev_bf16(L1.T, dev)
        lu = to_dev_bf16(L2.T, dev)
    wc, ws = S.svdq_pack_weight(d, Wd, lam_d, ld, lu)
    T = None if ld is None else torch.empty(M, rank, dtype=torch.float32, device=dev)
    xc, xs, T, ximg = S.svdq_quantize_act(d, Xd, lam_d, ld, T=T, codes=True)
    wimg = S.svdq_prepare_weight(d, wc, ws, lu, bd)
    Y = S.svdq_linear_forward(d, M, ximg, wimg)
    torch.cuda.synchronize()
    return dict(lam=lam_d, wc=wc, ws=ws, xc=xc, xs=xs, T=T, Y=Y, ximage=ximg, wimage=wimg)


def np_(t):
    return t.cpu().numpy()


def y_error(y_gpu: np.ndarray, Y_or: np.ndarray, out_f32: bool):
    """Elementwise check of the output.

    bf16 output: |y - y_or| <= 1e-2 rms(Y_or) + 2^-8 max(|y_or|, |y|), the
    second term being the half-ulp of the bf16 rounding of the output.
    fp32 output: |y - y_or| <= 1e-2 rms(Y_or).
    Returns (ok, max|err| / rms)."""
    y = np.asarray(y_gpu, np.float64)
    rms = float(np.sqrt(np.mean(Y_or ** 2)))
    err = np.abs(y - Y_or)
    bound = 1e-2 * rms
    if not out_f32:
        bound = bound + 2.0 ** -8 * np.maximum(np.abs(Y_or), np.abs(y))
    return bool(np.all(err <= bound)), float(err.max() / rms)


def assert_y(y_gpu, Y_or, out_f32, what=""):
    ok, rel = y_error(y_gpu, Y_or, out_f32)
    assert ok, f"{what}: output outside tolerance (max|err|/rms = {rel:.4g})"
    return rel


def assert_T(T_gpu, T_or, Xh_bits, L1_bits, what=""):
    """T is accumulated in fp32 on the GPU: elementwise within 1e-5 of
    sum_k |X_hat[m, k] L1[k, i]| (the scale of the fp32 accumulation error)
    and normwise within 1e-5 of the fp64 oracle."""
    T = np.asarray(T_gpu, np.float64)
    mag = np.abs(O.bf16_to_f32(Xh_bits).astype(np.float64)) @ np.abs(
        O.bf16_to_f32(L1_bits).astype(np.float64))
    err = np.abs(T - T_or)
    assert np.all(err <= 1e-5 * mag + 1e-30), f"{what}: T elementwise error {(err / (mag + 1e-30)).max():.3g}"
    assert np.linalg.norm(T - T_or) <= 1e-5 * np.linalg.norm(T_or) + 1e-30, f"{what}: T normwise"
