"""GPU parity of the NVFP4 variant through the C ABI against the CPU oracle:
activation and weight codes, E4M3 scales and the per-tensor scale bit for
bit, the layer output within the layer tolerance.  Every test prints its
case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import assert_T, assert_y, np_, oracle_offline

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def _g(v):
    return torch.tensor([float(v)], dtype=torch.float32, device=DEV)


def _layer(spec, seed, r, out_f32=False, rows=None, g_div=1.0):
    """Oracle and GPU through the whole NVFP4 layer; returns what the tests
    compare.  rows: the oracle's output only for these rows (large shapes).
    g_div > 1 takes the activation scale below the calibrated one, so that
    block scales saturate at 448 and codes at 6."""
    S = _S()
    X, W, b = WL.draw(spec, seed=seed)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam, L1, L2, _, _ = oracle_offline(xb, wb, r, "fp4")
    Xh = O.smooth_act(xb, lam)
    g_x = float(np.float32(O.nvfp4_global_scale(float(np.abs(O.bf16_to_f32(Xh)).max())) / g_div))
    xc_o, xs_o, _ = O.nvfp4_quantize_act(xb, lam, g_x)
    wc_o, ws_o, gw_o = O.nvfp4_pack_weight(wb, lam, L1, L2)
    sel = slice(None) if rows is None else rows
    T_o = O.bf16_to_f32(Xh[sel]).astype(np.float64) @ O.bf16_to_f32(L1).astype(np.float64) if r else None
    Y_o = O.nvfp4_forward(xc_o[sel], xs_o[sel], g_x, T_o, wc_o, ws_o, gw_o, L2 if r else None, bb)
    lamd = torch.from_numpy(lam).to(DEV)
    Xd, Wd = X.to(DEV), W.to(DEV)
    gx = _g(g_x)
    ld = WL.from_bits(np.ascontiguousarray(L1.T)).to(DEV) if r else None
    lu = WL.from_bits(np.ascontiguousarray(L2.T)).to(DEV) if r else None
    xc, xs, T = S.svdq_nvfp4_quantize_act(Xd, lamd, gx, lora_down=ld)
    wc, ws, gw = S.svdq_nvfp4_pack_weight(Wd, lamd, r, ld, lu)
    Y = S.svdq_nvfp4_linear(xc, xs, gx, wc, ws, gw, T, lu, b.to(DEV), out_f32=out_f32)
    torch.cuda.synchronize()
    return dict(xc=(np_(xc), xc_o), xs=(np_(xs), xs_o), wc=(np_(wc), wc_o), ws=(np_(ws), ws_o),
                gw=(np_(gw)[0], gw_o), Y=(np_(Y.float())[sel], Y_o),
                T=(np_(T)[sel] if r else None, T_o, Xh[sel], L1))


@pytest.mark.parametrize("M,K,N,r", [(77, 512, 256, 16), (256, 1024, 384, 32), (130, 256, 128, 0),
                                     (300, 3072, 512, 128), (1, 128, 128, 16), (513, 128, 640, 0)])
@pytest.mark.parametrize("out_f32", [False, True])
def test_layer_matches_oracle(M, K, N, r, out_f32):
    """Ragged M (one row; not a multiple of the 256-row tile), the smallest
    K (128, four K-steps), a partial last 256-column tile (N = 384, 640),
    rank 0 to 128, both output types."""
    _say("nvfp4 layer", M, K, N, r, out_f32)
    spec = WL.LinearSpec(f"nv_{M}x{K}x{N}", M, K, N, r, "fp4", x_outliers=4, x_factor=30.0,
                         w_outliers=2, w_factor=10.0)
    res = _layer(spec, seed=M + N, r=r, out_f32=out_f32)
    for k in ("xc", "xs", "wc", "ws"):
        assert np.array_equal(*res[k]), k
    assert np.float32(res["gw"][0]) == np.float32(res["gw"][1])
    if r:
        assert_T(*res["T"], "nvfp4 T (fused into the activation pass)")
    assert_y(*res["Y"], out_f32, "nvfp4 Y")


@pytest.mark.parametrize("g_div", [4.0, 64.0])
def test_activation_scale_below_calibration(g_div):
    """Activations above what the per-tensor scale was calibrated for: the
    E4M3 block scales saturate at 448 and the codes at 6, identically on both
    sides."""
    _say("nvfp4 saturating activation scale", g_div)
    spec = WL.LinearSpec("nv_sat_300x1024x256", 300, 1024, 256, 16, "fp4", x_outliers=4,
                         x_factor=30.0, w_outliers=2, w_factor=10.0)
    res = _layer(spec, seed=9, r=16, g_div=g_div)
    xs = res["xs"][1]
    assert np.count_nonzero(xs == 0x7E) > 0, "some block scale saturates at 448"
    codes = res["xc"][1]
    mags = np.concatenate([codes & 7, (codes >> 4) & 7])
    assert np.count_nonzero(mags == 7) > 0, "some code saturates at 6"
    for k in ("xc", "xs", "wc", "ws"):
        assert np.array_equal(*res[k]), k
    assert_T(*res["T"], "nvfp4 T")
    assert_y(*res["Y"], False, "nvfp4 Y")


def test_zero_blocks_and_scale_helper():
    """Zero blocks give scale 0 and +0 codes; the scale helper takes the
    maximum of a vector of maxima."""
    S = _S()
    _say("nvfp4 zero blocks")
    M, K = 64, 256
    X = torch.randn(M, K, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    X[5, 32:64] = 0
    X[9] = 0
    xb = WL.bits(X)
    lam = np.ones(K, np.float32)
    g = O.nvfp4_global_scale(float(np.abs(O.bf16_to_f32(xb)).max()))
    xc_o, xs_o, _ = O.nvfp4_quantize_act(xb, lam, g)
    amax = torch.from_numpy(np.abs(O.bf16_to_f32(xb)).max(axis=0)).to(DEV)
    gd = S.svdq_nvfp4_scale_from_absmax(amax)
    xc, xs, _ = S.svdq_nvfp4_quantize_act(X.to(DEV), torch.from_numpy(lam).to(DEV), gd)
    z = S.svdq_nvfp4_scale_from_absmax(torch.zeros(7, device=DEV))
    torch.cuda.synchronize()
    assert np.float32(np_(gd)[0]) == g
    assert np_(z)[0] == 1.0
    assert np.array_equal(np_(xc), xc_o) and np.array_equal(np_(xs), xs_o)
    assert not np_(xs)[5, 2:4].any() and not np_(xs)[9].any() and not np_(xc)[9].any()


def test_full_size_fused_projection():
    """The C4 shape (M = 4608, K = 3072, N = 21504, rank 32): every code and
    scale bit for bit, the output on 96 sampled rows (every 48th)."""
    _say("nvfp4 full size", WL.FLUX_FUSED_FP4.name)
    rows = np.arange(0, 4608, 48)
    res = _layer(WL.FLUX_FUSED_FP4, seed=0, r=32, rows=rows)
    for k in ("xc", "xs", "wc", "ws"):
        assert np.array_equal(*res[k]), k
    assert np.float32(res["gw"][0]) == np.float32(res["gw"][1])
    assert_T(*res["T"], "nvfp4 T (C4 rows)")
    assert_y(*res["Y"], False, "nvfp4 Y (C4 rows)")


def test_every_scale_byte_in_the_gemm():
    """The GEMM on hand-made codes whose block scales run through every E4M3
    byte 0x00..0x7E (zero, the 7 subnormals, all normals) on both operands,
    g_x = 0.75, g_w = 1.25, fp32 output: each output within the fp32
    summation bound (K 2^-24 sum |x w|) of the oracle's exact sum, so a wrong
    decode of any scale byte fails."""
    S = _S()
    M, N, K = 64, 128, 256
    _say("nvfp4 gemm every scale byte", M, N, K)
    rng = np.random.default_rng(11)
    nb = K // 16
    xs = ((np.arange(M)[:, None] * nb + np.arange(nb)[None, :]) % 127).astype(np.uint8)
    ws = ((np.arange(N)[:, None] * 5 + 3 * np.arange(nb)[None, :]) % 127).astype(np.uint8)
    xc = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    gx, gw = np.float32(0.75), np.float32(1.25)
    Y_o = O.nvfp4_forward(xc, xs, gx, None, wc, ws, gw, None, None)
    absum = np.abs(O.decode_nvfp4(xc, xs, gx)) @ np.abs(O.decode_nvfp4(wc, ws, gw)).T
    t = lambda a: torch.from_numpy(a).to(DEV)
    Y = S.svdq_nvfp4_linear(t(xc), t(xs), _g(gx), t(wc), t(ws), _g(gw), out_f32=True)
    torch.cuda.synchronize()
    err = np.abs(np_(Y).astype(np.float64) - Y_o)
    bound = K * 2.0 ** -24 * absum + 1e-300
    assert np.all(err <= bound), f"{np.sum(err > bound)} outputs, worst {np.max(err / bound):.3g}x"
