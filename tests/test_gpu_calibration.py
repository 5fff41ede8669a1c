"""GPU parity of the calibration statistics through the C ABI: per-column
absolute maxima (one batch and a running maximum over batches), lambda from
the maxima, and the one-shot calibration at the FLUX QKV size, all bit-exact
against the oracle.  Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def test_running_absmax_over_batches():
    S = _S()
    K = 640
    _say("calibrate absmax batches", K)
    spec = WL.LinearSpec("cal", 1, K, 128, 0, "int4", x_outliers=6, x_factor=(20.0, 100.0))
    batches = [WL.draw(spec, seed=s, M=m)[0] for s, m in ((1, 300), (2, 1), (3, 77), (4, 1029))]
    amax = None
    run_o = None
    for i, X in enumerate(batches):
        amax = S.svdq_calibrate_absmax(X.to(DEV), amax, accumulate=i > 0)
        run_o = O.column_absmax(WL.bits(X), run_o)
        torch.cuda.synchronize()
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), run_o.view(np.uint32)), f"batch {i}"


def test_lambda_from_absmax_and_one_shot():
    S = _S()
    spec = WL.FLUX_QKV
    _say("calibrate lambda", spec.name)
    X, W, _ = WL.draw(spec, seed=0)
    xb, wb = WL.bits(X), WL.bits(W)
    lam_o = O.calibrate_lambda(xb, wb)
    Xd, Wd = X.to(DEV), W.to(DEV)
    lam1 = S.svdq_calibrate_lambda(Xd, Wd)
    xmax = S.svdq_calibrate_absmax(Xd[:1000])
    xmax = S.svdq_calibrate_absmax(Xd[1000:].contiguous(), xmax, accumulate=True)
    wmax = S.svdq_calibrate_absmax(Wd)
    lam2 = S.svdq_lambda_from_absmax(xmax, wmax)
    torch.cuda.synchronize()
    assert np.array_equal(lam1.cpu().numpy().view(np.uint32), lam_o.view(np.uint32))
    assert np.array_equal(lam2.cpu().numpy().view(np.uint32), lam_o.view(np.uint32))
