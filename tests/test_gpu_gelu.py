"""GPU parity of the GELU(tanh) input option of the activation pass (the MLP
down-projection reading the up-projection's output) through the C ABI
against the CPU oracle.  Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import assert_T, assert_y, np_, oracle_offline, to_dev_bf16

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_gelu_every_bf16_value(mode):
    """All finite bf16 inputs as a 256 x 256 X, lambda = 1 and L1 = the
    256 x 256 identity: then T = X_hat L1 is the bf16 GELU of every input,
    exactly (one nonzero product per sum), bit for bit against the oracle."""
    S = _S()
    _say("gelu exhaustive", mode)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp_all_ones = (bits & 0x7F80) == 0x7F80          # inf / NaN patterns
    bits[exp_all_ones] = 0
    xb = bits.reshape(256, 256)
    K = r = 256
    lam = np.ones(K, np.float32)
    eye = np.eye(K, dtype=np.float32)
    L1 = O.f32_to_bf16(eye)                              # [K][r]
    d = S.desc(mode, K, 256, r, gelu_in=True)
    T = torch.empty(256, r, dtype=torch.float32, device=DEV)
    S.svdq_quantize_act(d, WL.from_bits(xb).to(DEV), torch.from_numpy(lam).to(DEV),
                        to_dev_bf16(L1.T, DEV), T=T, image=False, codes=True)
    torch.cuda.synchronize()
    got = np_(T).astype(np.float32)
    want = O.bf16_to_f32(O.gelu_bf16(xb))
    bad = got.view(np.uint32) != want.view(np.uint32)
    # -0 and +0 sum to +0 in T: compare zeros by value; a subnormal GELU
    # value may read back as 0 if the matrix unit flushes subnormal inputs
    bad &= ~((got == 0) & (want == 0))
    bad &= ~((got == 0) & (np.abs(want) < np.float32(2.0 ** -126)))
    assert not bad.any(), f"{bad.sum()} mismatches, first at input {xb.reshape(-1)[np.argmax(bad.reshape(-1))]:#06x}"


@pytest.mark.parametrize("mode", ["int4", "fp4"])
@pytest.mark.parametrize("M,K,N,r", [(77, 512, 256, 16), (300, 6144, 256, 32), (130, 1024, 384, 0)])
def test_gelu_quantize_and_layer(mode, M, K, N, r):
    """Codes, scales and T of GELU(X) bit-exact / within the T tolerance, then
    the layer output through the activation image; K = 6144 splits K."""
    S = _S()
    _say("gelu layer", mode, M, K, N, r)
    spec = WL.LinearSpec(f"gelu_{M}x{K}x{N}", M, K, N, r, mode, x_outliers=4, x_factor=8.0)
    X, W, b = WL.draw(spec, seed=M + K)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    xg = O.gelu_bf16(xb)                       # the layer's input
    lam, L1, L2, wc_o, ws_o = oracle_offline(xg, wb, r, mode)
    xc_o, xs_o, T_o, Xh = O.quantize_act(xb, lam, L1 if r else None, mode, gelu_in=True)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2 if r else None, bb, mode)
    d = S.desc(mode, K, N, r, gelu_in=True)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    lamd = torch.from_numpy(lam).to(DEV)
    ld = to_dev_bf16(L1.T, DEV) if r else None
    lu = to_dev_bf16(L2.T, DEV) if r else None
    T = torch.empty(M, r, dtype=torch.float32, device=DEV) if r else None
    xc, xs, T, ximg = S.svdq_quantize_act(d, Xd, lamd, ld, T=T, codes=True)
    wc, ws = S.svdq_pack_weight(d, Wd, lamd, ld, lu)
    Y = S.svdq_linear_forward(d, M, ximg, S.svdq_prepare_weight(d, wc, ws, lu, bd))
    torch.cuda.synchronize()
    assert np.array_equal(np_(xc), xc_o), "codes"
    assert np.array_equal(np_(xs), xs_o), "scales"
    if r:
        assert_T(np_(T), T_o, Xh, L1, "T")
    assert_y(np_(Y.float()), Y_o, False, f"gelu layer {mode}")


def test_gelu_standalone_down_projection():
    """The stand-alone down-projection honours the flag as well."""
    S = _S()
    M, K, r = 150, 1024, 32
    _say("gelu lowrank_down", M, K, r)
    spec = WL.LinearSpec("gelu_down", M, K, 256, r, "int4", x_outliers=4, x_factor=8.0)
    X, W, _ = WL.draw(spec, seed=21)
    xb, wb = WL.bits(X), WL.bits(W)
    lam, L1, _, _, _ = oracle_offline(O.gelu_bf16(xb), wb, r, "int4")
    _, _, T_o, Xh = O.quantize_act(xb, lam, L1, "int4", gelu_in=True)
    d = S.desc("int4", K, 256, r, gelu_in=True)
    T = S.svdq_lowrank_down(d, X.to(DEV), torch.from_numpy(lam).to(DEV), to_dev_bf16(L1.T, DEV))
    torch.cuda.synchronize()
    assert_T(np_(T), T_o, Xh, L1, "T (stand-alone, gelu)")
