"""svdq_lowrank_factors_noalloc (the randomized SVD with its workspace in
the library's static device array) against svdq_lowrank_factors with a
caller workspace: bit-identical factors and singular values, on two calls in
a row, the second with a smaller shape (the static array keeps the first
call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as WL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def _inputs(N, K, seed):
    spec = WL.LinearSpec(f"noalloc_{N}x{K}", 64, K, N, 16, "int4", x_outliers=2, x_factor=20.0,
                         w_outliers=4, w_factor=10.0)
    X, W, _ = WL.draw(spec, seed=seed)
    S = _S()
    Wd = W.to(DEV)
    lam = S.svdq_calibrate_lambda(X.to(DEV), Wd)
    return Wd, lam


def _both(N, K, rank, seed, iters):
    S = _S()
    Wd, lam = _inputs(N, K, seed)
    ref_d, ref_u, ref_s = S.svdq_lowrank_factors(Wd, lam, rank, seed=seed, power_iters=iters)
    # the outputs of the no-allocation call: poisoned so stale values show
    ld = torch.full((rank, K), -7.0, dtype=torch.bfloat16, device=DEV)
    lu = torch.full((N, rank), -7.0, dtype=torch.bfloat16, device=DEV)
    sg = torch.full((rank,), -7.0, dtype=torch.float64, device=DEV)
    S.svdq_lowrank_factors_noalloc(Wd, lam, rank, seed, iters, ld, lu, sg)
    torch.cuda.synchronize()
    return (ref_d, ref_u, ref_s), (ld, lu, sg)


@pytest.mark.parametrize("first,second", [((3072, 3072, 32, 1, 2), (1024, 512, 16, 2, 1)),
                                          ((2048, 1024, 64, 3, 2), (512, 512, 16, 4, 0))])
def test_noalloc_matches_workspace_entry_point(first, second):
    for N, K, rank, seed, iters in (first, second):
        print("[case] noalloc", N, K, rank, seed, iters, flush=True)
        ref, got = _both(N, K, rank, seed, iters)
        for a, b, what in zip(ref, got, ("lora_down", "lora_up", "sigma")):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                f"{what} differs at {N}x{K} rank {rank}"
        assert np.all(np.isfinite(got[2].cpu().numpy()))


def test_noalloc_rejects_shapes_beyond_its_workspace():
    S = _S()
    lib = S.load()
    n = ctypes.c_size_t(0)
    assert lib.svdq_lowrank_factors_workspace(9216, 3072, 32, ctypes.byref(n)) == 0
    assert n.value > 64 << 20
    W = torch.zeros(9216, 3072, dtype=torch.bfloat16, device=DEV)
    lam = torch.ones(3072, dtype=torch.float32, device=DEV)
    ld = torch.empty(32, 3072, dtype=torch.bfloat16, device=DEV)
    lu = torch.empty(9216, 32, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(S.SvdqError) as e:
        S.svdq_lowrank_factors_noalloc(W, lam, 32, 0, 2, ld, lu)
    assert e.value.status == 2
