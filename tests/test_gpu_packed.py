"""The layer from resident packed 4-bit weights (svdq_linear_forward_packed)
through the C ABI: Y bit for bit equal to svdq_prepare_weight followed by
svdq_linear_forward on the same inputs (whose output the other GPU tests
check against the oracle), and the scratch shared by successive layers.
Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import workloads as WL
from layer_util import gpu_run, oracle_offline

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def _layer(mode, M, K, N, r, seed, bias=True, out_f32=False):
    spec = WL.LinearSpec(f"pk_{M}x{K}x{N}", M, K, N, r, mode, x_outliers=4, x_factor=20.0,
                         w_outliers=2, w_factor=10.0)
    X, W, b = WL.draw(spec, seed=seed)
    lam, L1, L2, _, _ = oracle_offline(WL.bits(X), WL.bits(W), r, mode)
    res = gpu_run(DEV, X, W, b if bias else None, lam, L1, L2, mode, r, out_f32=out_f32)
    S = _S()
    d = S.desc(mode, K, N, r, out_f32=out_f32)
    lu = None
    if r:
        lu = WL.from_bits(np.ascontiguousarray(L2.T)).to(DEV)
    return S, d, res, lu, (b.to(DEV) if bias else None)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
@pytest.mark.parametrize("M,K,N,r,bias,out_f32", [
    (300, 1024, 640, 32, True, False), (77, 512, 256, 0, False, False),
    (513, 128, 640, 16, True, True), (1, 3072, 384, 128, True, False)])
def test_packed_forward_equals_prepared(mode, M, K, N, r, bias, out_f32):
    _say("packed forward", mode, M, K, N, r, bias, out_f32)
    S, d, res, lu, bd = _layer(mode, M, K, N, r, seed=M + N, bias=bias, out_f32=out_f32)
    scratch = torch.full((S.svdq_weight_image_size(d),), 0xA5, dtype=torch.uint8, device=DEV)
    Y = S.svdq_linear_forward_packed(d, M, res["ximage"], res["wc"], res["ws"], lu, bd,
                                     wscratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(scratch, res["wimage"]), "scratch differs from the prepared weight"
    assert torch.equal(Y.view(torch.int16 if not out_f32 else torch.int32),
                       res["Y"].view(torch.int16 if not out_f32 else torch.int32))


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_one_scratch_for_successive_layers(mode):
    """Two layers of different shapes through one scratch (sized for the
    larger), alternating A, B, A: each output equals its prepared-weight one."""
    _say("shared scratch", mode)
    SA, dA, rA, luA, bA = _layer(mode, 200, 1024, 768, 32, seed=1)
    SB, dB, rB, luB, bB = _layer(mode, 130, 512, 384, 16, seed=2)
    S = SA
    nA, nB = S.svdq_weight_image_size(dA), S.svdq_weight_image_size(dB)
    big = torch.empty(max(nA, nB), dtype=torch.uint8, device=DEV)
    for d, r, lu, b, n in ((dA, rA, luA, bA, nA), (dB, rB, luB, bB, nB), (dA, rA, luA, bA, nA)):
        Y = S.svdq_linear_forward_packed(d, r["Y"].shape[0], r["ximage"], r["wc"], r["ws"], lu, b,
                                         wscratch=big[:n])
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), r["Y"].view(torch.int16))


def test_full_size_packed_int4():
    """The C2 shape (M = 4096, K = 3072, N = 9216, rank 32): the packed path's Y
    bit for bit equal to the prepared path's."""
    _say("packed forward full size", WL.FLUX_QKV.name)
    S = _S()
    spec = WL.FLUX_QKV
    X, W, b = WL.draw(spec, seed=0)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    lam = S.svdq_calibrate_lambda(Xd, Wd)
    ld, lu, _ = S.svdq_lowrank_factors(Wd, lam, spec.rank, seed=0, want_sigma=False)
    d = S.desc(spec.mode, spec.K, spec.N, spec.rank)
    wc, ws = S.svdq_pack_weight(d, Wd, lam, ld, lu)
    xi = S.svdq_quantize_act(d, Xd, lam, ld)[3]
    Y0 = S.svdq_linear_forward(d, spec.M, xi, S.svdq_prepare_weight(d, wc, ws, lu, bd))
    Y1 = S.svdq_linear_forward_packed(d, spec.M, xi, wc, ws, lu, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
