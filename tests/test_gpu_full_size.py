"""GPU parity at the full FLUX sizes, in the launch configuration the
benchmark times.

At the QKV (INT4, 4096 x 3072 x 9216, rank 32) and fused-projection (FP4,
4608 x 3072 x 21504, rank 32) shapes everything is compared: lambda, every
activation and weight code and scale bit for bit, T over all rows, and every
output, bf16 under the layer's tolerance and fp32 (SVDQ_FLAG_OUT_F32) under
the strict bound max|err| <= 1e-2 rms(Y_or).  The full outputs come from the
oracle's dequantize-then-matmul formulation (one fp64 product), which the
oracle's pins tie to the per-group definition to ~1e-12 relative.

The MLP pair and the eight layers of the double-stream block chain (rank
128) compare codes, scales and T over all activation rows and the weight and
output on sampled rows and columns, computed by the oracle's per-group
definition."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import assert_T, assert_y, np_, to_dev_bf16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _run_full(spec, X, W, b, mode, weight_rows=None, y_rows=None, y_cols=None, rank=None,
              gelu_in=False, check_f32=False):
    """Oracle and GPU on the same inputs; compare.  weight_rows / y_rows /
    y_cols = None means every row or column.  With gelu_in the layer's input is
    GELU(X), applied in the activation pass (lambda is then the oracle's,
    calibrated on GELU(X)).  Returns (max|err|/rms of the bf16 output, info)."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    rank = spec.rank if rank is None else rank
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    M, K = X.shape
    N = W.shape[0]
    all_w = weight_rows is None
    wrows = np.arange(N) if all_w else weight_rows
    lam = O.calibrate_lambda(O.gelu_bf16(xb) if gelu_in else xb, wb)
    L1, L2, _ = O.lowrank_factors(O.smooth_weight(wb, lam), rank)
    wc_o, ws_o = O.pack_weight(wb if all_w else wb[wrows], lam, L1,
                               L2 if all_w else L2[:, wrows], mode)
    xc_o, xs_o, T_o, Xh = O.quantize_act(xb, lam, L1, mode, gelu_in=gelu_in)

    _say(spec.name, mode, M, K, N, rank, "gelu input" if gelu_in else "",
         "all rows" if all_w else f"{len(wrows)} weight rows")
    d = S.desc(mode, K, N, rank, gelu_in=gelu_in)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    lamd = torch.from_numpy(lam).to(DEV) if gelu_in else S.svdq_calibrate_lambda(Xd, Wd)
    ld, lu = to_dev_bf16(L1.T, DEV), to_dev_bf16(L2.T, DEV)
    wc, ws = S.svdq_pack_weight(d, Wd, lamd, ld, lu)
    T = torch.empty(M, rank, dtype=torch.float32, device=DEV)
    xc, xs, T, ximg = S.svdq_quantize_act(d, Xd, lamd, ld, T=T, codes=True)
    wimg = S.svdq_prepare_weight(d, wc, ws, lu, bd)
    Y = S.svdq_linear_forward(d, M, ximg, wimg)
    Y32 = None
    if check_f32:
        Y32 = S.svdq_linear_forward(S.desc(mode, K, N, rank, out_f32=True), M, ximg, wimg)
    torch.cuda.synchronize()

    assert np.array_equal(np_(lamd), lam), "lambda"
    assert np.array_equal(np_(xc), xc_o), "activation codes"
    assert np.array_equal(np_(xs), xs_o), "activation scales"
    assert np.array_equal(np_(wc)[wrows], wc_o), "weight codes"
    assert np.array_equal(np_(ws)[wrows], ws_o), "weight scales"
    assert_T(np_(T), T_o, Xh, L1, "T")
    del wc, ws, xc, xs, T, Xd, Wd

    if y_rows is None:
        # every output: the dequantize-then-matmul formulation in fp64
        assert all_w, "full outputs need every weight row"
        Y_o = O.forward_dequant(xc_o, xs_o, T_o, wc_o, ws_o, L2, bb, mode)
        rel = assert_y(np_(Y.float()), Y_o, False, spec.name + " (bf16, all outputs)")
        if Y32 is not None:
            rel32 = assert_y(np_(Y32), Y_o, True, spec.name + " (fp32, all outputs)")
            _say(f"fp32 output: max|err|/rms = {rel32:.4g}")
        _say(f"bf16 output: max|err|/rms = {rel:.4g}")
        return rel, dict(lam=lam, L1=L1, L2=L2, Y=Y)

    # Y on sampled rows x sampled columns (weight rows = output columns)
    sel = np.searchsorted(wrows, y_cols)
    assert np.array_equal(wrows[sel], y_cols)
    Y_o = O.forward(xc_o[y_rows], xs_o[y_rows], T_o[y_rows], wc_o[sel], ws_o[sel],
                    L2[:, y_cols], bb[y_cols], mode)
    ri, ci = torch.from_numpy(y_rows).to(DEV), torch.from_numpy(y_cols).to(DEV)
    rel = assert_y(np_(Y[ri][:, ci].float()), Y_o, False, spec.name)
    if Y32 is not None:
        assert_y(np_(Y32[ri][:, ci]), Y_o, True, spec.name + " (fp32)")
    return rel, dict(lam=lam, L1=L1, L2=L2, Y=Y)


def _samples(M, N, seed, n_w=1024, n_y=96):
    rng = np.random.default_rng(seed)
    weight_rows = np.sort(rng.choice(N, size=min(n_w, N), replace=False))
    y_rows = np.sort(np.concatenate([rng.choice(M, size=n_y - 2, replace=False), [0, M - 1]]))
    y_cols = np.sort(rng.choice(weight_rows, size=min(512, weight_rows.size), replace=False))
    return weight_rows, np.unique(y_rows), y_cols


def test_flux_qkv_int4_full():
    """C2 in full: every code, scale and output, bf16 and fp32 outputs."""
    spec = WL.FLUX_QKV
    X, W, b = WL.draw(spec, seed=0)
    _run_full(spec, X, W, b, "int4", check_f32=True)


def test_fused_qkv_mlp_fp4_full():
    """C4 in full: every code, scale and output, bf16 and fp32 outputs."""
    spec = WL.FLUX_FUSED_FP4
    X, W, b = WL.draw(spec, seed=0)
    _run_full(spec, X, W, b, "fp4", check_f32=True)


def test_flux_mlp_pair_int4_full():
    """MLP up 3072 -> 12288, GELU(tanh), MLP down 12288 -> 3072, as the bench
    runs it: the down layer reads the oracle's bf16 up output (computed with
    the oracle's dequantize-then-matmul formulation, which the oracle's pins
    tie to the per-group formulation) and applies the GELU in its own
    activation pass."""
    up, down = WL.FLUX_MLP_UP, WL.FLUX_MLP_DOWN
    X, Wu, bu = WL.draw(up, seed=0)
    wr, yr, yc = _samples(up.M, up.N, 3)
    _, info = _run_full(up, X, Wu, bu, "int4", wr, yr, yc)

    # oracle up output for every token
    xb, wb, bb = WL.bits(X), WL.bits(Wu), WL.bits(bu)
    lam, L1, L2 = info["lam"], info["L1"], info["L2"]
    wc, ws = O.pack_weight(wb, lam, L1, L2, "int4")
    xc, xs, T, _ = O.quantize_act(xb, lam, L1, "int4")
    Y_up = O.forward_dequant(xc, xs, T, wc, ws, L2, bb, "int4")
    X_down = WL.from_bits(O.to_bf16_out(Y_up))
    _, Wd, bd = WL.draw(down, seed=0, M=1)
    wr, yr, yc = _samples(down.M, down.N, 4)
    _run_full(down, X_down, Wd, bd, "int4", wr, yr, yc, gelu_in=True, check_f32=True)


@pytest.mark.parametrize("layer", ["block_img_qkv", "block_img_out", "block_img_up",
                                   "block_img_down", "block_txt_qkv", "block_txt_out",
                                   "block_txt_up", "block_txt_down"])
def test_block_chain_layers_full(layer):
    """The eight linears of the double-stream block at batch 2 and rank 128,
    at their shapes: image stream M = 8192, text stream M = 1024; qkv
    3072 -> 9216, out 3072 -> 3072, MLP up 3072 -> 12288, MLP down
    12288 -> 3072 on a GELU input (its input drawn by the seeded generator,
    standing in for the up output; the GELU is applied in the activation
    pass)."""
    spec = next(s for s in WL.block_chain_specs(128) if s.name == layer)
    X, W, b = WL.draw(spec, seed=5)
    wr, yr, yc = _samples(spec.M, spec.N, 5, n_w=512)
    _run_full(spec, X, W, b, "int4", wr, yr, yc, gelu_in=layer.endswith("_down"),
              check_f32=layer.startswith("block_txt"))
