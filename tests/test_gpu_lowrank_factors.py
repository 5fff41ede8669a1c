"""GPU parity of the randomized truncated SVD that produces the low-rank
factors (svdq_lowrank_factors) through the C ABI against the CPU oracle: the
same Philox sketch, the same shifted CholeskyQR2 and power iterations, so the
singular values agree to fp64 rounding and the bf16 factors bit for bit up to
a rare rounding-boundary ulp.  Every test prints its case before touching the
GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import np_

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def _lam(K, seed):
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(-1.0, 1.0, K)).astype(np.float32)


def _run(S, W, lam, r, seed, q):
    ld, lu, sig = S.svdq_lowrank_factors(W.to(DEV), torch.from_numpy(lam).to(DEV), r, seed,
                                         power_iters=q)
    torch.cuda.synchronize()
    return WL.bits(ld.cpu()), WL.bits(lu.cpu()), sig.cpu().numpy()


def _ulps(a, b):
    """bf16 distance in units in the last place (same-sign patterns)."""
    ia = a.astype(np.int32)
    ib = b.astype(np.int32)
    ia = np.where(ia & 0x8000, 0x8000 - ia, ia)
    ib = np.where(ib & 0x8000, 0x8000 - ib, ib)
    return np.abs(ia - ib)


def _assert_factors(got, want, what):
    u = _ulps(got, want)
    assert u.max() <= 1, f"{what}: {u.max()} ulps"
    frac = np.count_nonzero(u) / u.size
    assert frac <= 1e-3, f"{what}: {frac:.2e} of the entries differ"


def _check(S, W, lam, r, seed, q, tag):
    _say("lowrank factors", tag, tuple(W.shape), "r", r, "q", q, "seed", seed)
    ld, lu, sig = _run(S, W, lam, r, seed, q)
    ld_o, lu_o, s_o = O.rsvd_factors(WL.bits(W), lam, r, seed, power_iters=q)
    assert np.allclose(sig, s_o, rtol=1e-8, atol=0), np.max(np.abs(sig / s_o - 1))
    _assert_factors(ld, ld_o, "lora_down")
    _assert_factors(lu, lu_o, "lora_up")
    return ld, lu, sig


@pytest.mark.parametrize("N,K,r,q", [(256, 128, 16, 2), (384, 512, 32, 1), (512, 256, 48, 0),
                                     (768, 640, 128, 2), (128, 1024, 112, 3), (256, 128, 128, 1)])
def test_factors_match_oracle(N, K, r, q):
    """l = r + 16 from 32 to 144, l capped by min(N, K), 0..3 power
    iterations, N above and below K."""
    S = _S()
    W = WL.spectral_weight(N, K, seed=N + K)
    _check(S, W, _lam(K, r), r, 1000 + r, q, "small")


def test_factors_near_eckart_young():
    """The GPU factors approximate W_hat close to its best rank-r error."""
    S = _S()
    N, K, r = 640, 384, 32
    W = WL.spectral_weight(N, K, seed=5, decay=0.7)
    lam = _lam(K, 6)
    _say("lowrank eckart-young", N, K, r)
    ld, lu, _ = _run(S, W, lam, r, 77, 2)
    What = O.bf16_to_f32(WL.bits(W)).astype(np.float64) * lam.astype(np.float64)[None, :]
    P = O.bf16_to_f32(lu).astype(np.float64) @ O.bf16_to_f32(ld).astype(np.float64)
    sv = np.linalg.svd(What, compute_uv=False)
    opt = np.sqrt(np.sum(sv[r:] ** 2))
    assert np.linalg.norm(What - P) <= 1.05 * opt


def test_seed_determinism_and_zero_weight():
    S = _S()
    N, K, r = 384, 256, 32
    W = WL.spectral_weight(N, K, seed=9)
    lam = _lam(K, 3)
    _say("lowrank determinism", N, K, r)
    a = _run(S, W, lam, r, 5, 2)
    b = _run(S, W, lam, r, 5, 2)
    c = _run(S, W, lam, r, 6, 2)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    assert np.allclose(a[2], c[2], rtol=2e-2)           # both near the true top values
    _say("lowrank zero weight", N, K, r)
    z = _run(S, torch.zeros(N, K, dtype=torch.bfloat16), lam, r, 5, 2)
    assert not z[0].any() and not z[1].any() and not z[2].any()


@pytest.mark.parametrize("spec,r", [(WL.FLUX_QKV, 32), (WL.FLUX_MLP_DOWN, 32),
                                    (WL.block_chain_specs(128)[0], 128)])
def test_factors_full_size(spec, r):
    """FLUX shapes with the workload's weights and lambda calibrated on its
    activations: QKV 3072 -> 9216 at rank 32, MLP down 12288 -> 3072 at rank
    32, and the image-stream QKV at rank 128 (l = 144)."""
    S = _S()
    X, W, _ = WL.draw(spec, seed=0, M=256)
    lam = O.calibrate_lambda(WL.bits(X), WL.bits(W))
    _check(S, W, lam, r, 2024, 2, spec.name)


def test_factors_feed_pack_weight():
    """W alone -> lambda (calibration), factors and residual codes on the GPU;
    the codes equal the oracle's packing of the same factors."""
    S = _S()
    spec = WL.LinearSpec("pack_from_w", 512, 1024, 768, 32, "int4", x_outliers=8, x_factor=30.0,
                         w_outliers=4, w_factor=10.0)
    X, W, _ = WL.draw(spec, seed=4)
    _say("lowrank -> pack", spec.name)
    Xd, Wd = X.to(DEV), W.to(DEV)
    lam = S.svdq_calibrate_lambda(Xd, Wd)
    ld, lu, _ = S.svdq_lowrank_factors(Wd, lam, 32, 11)
    d = S.desc("int4", spec.K, spec.N, 32)
    wc, ws = S.svdq_pack_weight(d, Wd, lam, ld, lu)
    torch.cuda.synchronize()
    lam_h = lam.cpu().numpy()
    ld_h, lu_h = WL.bits(ld.cpu()), WL.bits(lu.cpu())
    wc_o, ws_o = O.pack_weight(WL.bits(W), lam_h, ld_h.T, lu_h.T, "int4")
    assert np.array_equal(np_(wc), wc_o)
    assert np.array_equal(np_(ws), ws_o)
