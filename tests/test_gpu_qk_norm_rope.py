"""GPU parity of the Q/K RMSNorm + rotary-embedding pass (svdq_qk_norm_rope)
through the C ABI against the CPU oracle, alone on bf16 inputs and after the
W4A4 QKV layer.  Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import np_, oracle_offline

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def _bf16(a):
    return O.f32_to_bf16(np.asarray(a, np.float32))


def _inputs(M, H, seed):
    rng = np.random.default_rng(seed)
    Y = _bf16(rng.standard_normal((M, 3 * H * 128)) * rng.uniform(0.1, 10.0, (M, 1)))
    qs = _bf16(rng.uniform(0.5, 1.5, 128))
    ks = _bf16(rng.uniform(0.5, 1.5, 128))
    ang = rng.uniform(-np.pi, np.pi, (M, 64))
    return Y, qs, ks, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _run(S, Y, qs, ks, c, s, H, eps=1e-6):
    Yd = WL.from_bits(Y).to(DEV)
    S.svdq_qk_norm_rope(Yd, H, WL.from_bits(qs).to(DEV), WL.from_bits(ks).to(DEV),
                        torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV), eps)
    torch.cuda.synchronize()
    return WL.bits(Yd.cpu())


def _want(Y, qs, ks, c, s, H, eps=1e-6):
    return O.qk_norm_rope(O.bf16_to_f32(Y), H, O.bf16_to_f32(qs), O.bf16_to_f32(ks),
                          c.astype(np.float64), s.astype(np.float64), eps)


def _assert_close(got_bits, want, what):
    """fp32 arithmetic rounded once to bf16: within the bf16 half-ulp of the
    value plus fp32 noise on the head's scale (cancellation in a rotation)."""
    got = O.bf16_to_f32(got_bits).astype(np.float64)
    M, HD = want.shape
    head_rms = np.sqrt(np.mean(want.reshape(M, HD // 128, 128) ** 2, axis=2))
    floor = np.repeat(head_rms, 128, axis=1) * 2.0 ** -16
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + floor
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} entries, worst {np.max(err / bound):.3g}x the bound"


@pytest.mark.parametrize("M,H", [(1, 1), (37, 3), (256, 24), (4096, 24)])
def test_matches_oracle(M, H):
    """One token and one head up to the FLUX QKV shape (M = 4096, 24 heads)."""
    S = _S()
    _say("qk_norm_rope", M, H)
    Y, qs, ks, c, s = _inputs(M, H, seed=M + H)
    out = _run(S, Y, qs, ks, c, s, H)
    Q, K, _ = _want(Y, qs, ks, c, s, H)
    HD = H * 128
    _assert_close(out[:, :HD], Q, "Q")
    _assert_close(out[:, HD:2 * HD], K, "K")
    assert np.array_equal(out[:, 2 * HD:], Y[:, 2 * HD:]), "V must not change"


def test_zero_head_and_identity_angles():
    """A zero head stays zero; zero angles and unit scales leave the RMS
    normalisation alone, which has unit rms."""
    S = _S()
    M, H = 8, 2
    _say("qk_norm_rope zero head", M, H)
    Y, _, _, _, _ = _inputs(M, H, seed=1)
    Y[3, 128:256] = 0
    ones = _bf16(np.ones(128))
    c = np.ones((M, 64), np.float32)
    s = np.zeros((M, 64), np.float32)
    out = O.bf16_to_f32(_run(S, Y, ones, ones, c, s, H)).astype(np.float64)
    assert not out[3, 128:256].any()
    heads = out[:, :2 * H * 128].reshape(M, 2 * H, 128)
    rms = np.sqrt(np.mean(heads ** 2, axis=2))
    rms[3, 1] = 1.0
    assert np.allclose(rms, 1.0, rtol=2e-3)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_after_the_qkv_layer(mode):
    """The W4A4 QKV layer (3 heads) followed by the pass, against the oracle's
    layer output followed by the oracle's pass: the layer's tolerance
    (1e-2 rms of Y) carried through the per-head normalisation."""
    S = _S()
    H, M, K = 3, 200, 512
    N = 3 * H * 128
    _say("qkv layer + qk_norm_rope", mode, M, K, N)
    spec = WL.LinearSpec("qkv_small", M, K, N, 32, mode, x_outliers=4, x_factor=20.0)
    X, W, b = WL.draw(spec, seed=9)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, 32, mode)
    xc_o, xs_o, T_o, _ = O.quantize_act(xb, lam, L1, mode)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2, bb, mode)
    _, qs, ks, c, s = _inputs(M, H, seed=2)
    Q_o, K_o, V_o = O.qk_norm_rope(Y_o, H, O.bf16_to_f32(qs), O.bf16_to_f32(ks),
                                   c.astype(np.float64), s.astype(np.float64), 1e-6)
    d = S.desc(mode, K, N, 32)
    lamd = torch.from_numpy(lam).to(DEV)
    ld = WL.from_bits(np.ascontiguousarray(L1.T)).to(DEV)
    lu = WL.from_bits(np.ascontiguousarray(L2.T)).to(DEV)
    _, _, _, ximg = S.svdq_quantize_act(d, X.to(DEV), lamd, ld)
    wc, ws = S.svdq_pack_weight(d, W.to(DEV), lamd, ld, lu)
    Y = S.svdq_linear_forward(d, M, ximg, S.svdq_prepare_weight(d, wc, ws, lu, b.to(DEV)))
    S.svdq_qk_norm_rope(Y, H, WL.from_bits(qs).to(DEV), WL.from_bits(ks).to(DEV),
                        torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    got = O.bf16_to_f32(WL.bits(Y.cpu())).astype(np.float64)
    HD = H * 128
    for name, g, w in (("Q", got[:, :HD], Q_o), ("K", got[:, HD:2 * HD], K_o)):
        rms = np.sqrt(np.mean(w ** 2))
        assert np.max(np.abs(g - w)) <= 3e-2 * rms, f"{name}: {np.max(np.abs(g - w)) / rms:.3g} rms"


@pytest.mark.parametrize("mode,H,extra,M", [("fp4", 3, 0, 200), ("fp4", 2, 512, 333),
                                             ("int4", 3, 0, 200), ("fp4", 24, 12288, 256)])
def test_forward_qk(mode, H, extra, M):
    """svdq_linear_forward_qk: the QKV (or fused QKV + MLP, `extra` more
    columns) layer with the Q/K transform.  Q and K against the oracle layer
    followed by the oracle transform; the columns after Q and K bit-identical
    to svdq_linear_forward, and the whole output to svdq_linear_forward
    followed by svdq_qk_norm_rope.  The last case is the FLUX single-stream
    shape (24 heads, N = 21504)."""
    S = _S()
    K = 3072 if H == 24 else 512
    N = 3 * H * 128 + extra
    _say("forward_qk", mode, M, K, N, H)
    spec = WL.LinearSpec("qkv_fwd", M, K, N, 32, mode, x_outliers=4, x_factor=20.0)
    X, W, b = WL.draw(spec, seed=H + extra)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, 32, mode)
    xc_o, xs_o, T_o, _ = O.quantize_act(xb, lam, L1, mode)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2, bb, mode)
    _, qs, ks, c, s = _inputs(M, H, seed=5)
    HD = H * 128
    Q_o, K_o, _ = O.qk_norm_rope(Y_o[:, :3 * HD], H, O.bf16_to_f32(qs), O.bf16_to_f32(ks),
                                 c.astype(np.float64), s.astype(np.float64), 1e-6)
    d = S.desc(mode, K, N, 32)
    lamd = torch.from_numpy(lam).to(DEV)
    ld = WL.from_bits(np.ascontiguousarray(L1.T)).to(DEV)
    lu = WL.from_bits(np.ascontiguousarray(L2.T)).to(DEV)
    _, _, _, ximg = S.svdq_quantize_act(d, X.to(DEV), lamd, ld)
    wc, ws = S.svdq_pack_weight(d, W.to(DEV), lamd, ld, lu)
    wimg = S.svdq_prepare_weight(d, wc, ws, lu, b.to(DEV))
    args = (WL.from_bits(qs).to(DEV), WL.from_bits(ks).to(DEV), torch.from_numpy(c).to(DEV),
            torch.from_numpy(s).to(DEV))
    Yq = S.svdq_linear_forward_qk(d, M, ximg, wimg, H, *args)
    Yp = S.svdq_linear_forward(d, M, ximg, wimg)
    Yu = Yp.clone()
    S.svdq_qk_norm_rope(Yu, H, *args)
    torch.cuda.synchronize()
    got = O.bf16_to_f32(WL.bits(Yq.cpu())).astype(np.float64)
    for name, g, w in (("Q", got[:, :HD], Q_o), ("K", got[:, HD:2 * HD], K_o)):
        rms = np.sqrt(np.mean(w ** 2))
        assert np.max(np.abs(g - w)) <= 3e-2 * rms, f"{name}: {np.max(np.abs(g - w)) / rms:.3g} rms"
    assert np.array_equal(WL.bits(Yq[:, 2 * HD:].cpu()), WL.bits(Yp[:, 2 * HD:].cpu())), \
        "columns after Q and K"
    assert np.array_equal(WL.bits(Yq.cpu()), WL.bits(Yu.cpu())), "forward + pass"
