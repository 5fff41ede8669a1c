"""GPU parity of svdq_linear_forward_rowmajor, the layer from the row-major
tensors of the C ABI (activation codes, scales and T; weight codes and
scales, lora_up, bias), which writes both operand images into a workspace
and runs the GEMM.  Against the CPU oracle with the oracle's own tensors as
input, and against svdq_linear_forward on the images that the activation
pass and svdq_prepare_weight write for the same tensors."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from bit_diffusion_transformer_quantize_amd import svdq as S
from layer_util import assert_y, gpu_run, np_, oracle_offline, to_dev_bf16

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _oracle_layer(spec, mode, M, rank, seed):
    X, W, b = WL.draw(spec, seed=seed, M=M)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    if rank > 0:
        lam, L1, L2, wc, ws = oracle_offline(xb, wb, rank, mode)
    else:
        lam = O.calibrate_lambda(xb, wb)
        L1 = np.zeros((xb.shape[1], 0), np.uint16)
        L2 = np.zeros((0, wb.shape[0]), np.uint16)
        wc, ws = O.pack_weight(wb, lam, L1, L2, mode)
    xc, xs, T, _ = O.quantize_act(xb, lam, L1 if rank > 0 else None, mode)
    return X, W, b, bb, lam, L1, L2, wc, ws, xc, xs, T


@pytest.mark.parametrize("mode", ["int4", "fp4"])
@pytest.mark.parametrize("M,rank,out_f32", [(256, 16, False), (1, 16, False), (300, 32, False),
                                            (130, 0, False), (96, 128, True), (77, 32, True)])
def test_oracle_tensors_in(mode, M, rank, out_f32):
    """The oracle's codes, scales and T (fp64, handed over as fp32) in; the
    output within the layer's tolerance of the oracle's forward."""
    spec = WL.TINY
    X, W, b, bb, lam, L1, L2, wc, ws, xc, xs, T, = _oracle_layer(spec, mode, M, rank, M + rank)
    Y_o = O.forward(xc, xs, T if rank > 0 else None, wc, ws, L2 if rank > 0 else None, bb, mode)
    _say("rowmajor vs oracle", mode, "M", M, "rank", rank, "f32" if out_f32 else "bf16")
    d = S.desc(mode, spec.K, spec.N, rank, out_f32=out_f32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    Td = t(T.astype(np.float32)) if rank > 0 else None
    lu = to_dev_bf16(L2.T, DEV) if rank > 0 else None
    Y = S.svdq_linear_forward_rowmajor(d, t(xc), t(xs), Td, t(wc), t(ws), lu, b.to(DEV))
    torch.cuda.synchronize()
    assert_y(np_(Y.float()), Y_o, out_f32, f"rowmajor {mode} M={M} r={rank}")


def _image_path_equal(mode, spec, M, rank, seed, workspace=None):
    X, W, b = WL.draw(spec, seed=seed, M=M)
    xb, wb = WL.bits(X), WL.bits(W)
    lam, L1, L2, _, _ = oracle_offline(xb, wb, rank, mode)
    g = gpu_run(DEV, X, W, b, lam, L1, L2, mode, rank)
    d = S.desc(mode, spec.K, spec.N, rank)
    lu = to_dev_bf16(L2.T, DEV)
    Y = S.svdq_linear_forward_rowmajor(d, g["xc"], g["xs"], g["T"], g["wc"], g["ws"], lu,
                                       b.to(DEV), workspace=workspace)
    torch.cuda.synchronize()
    # equal as values (an exact zero may differ in sign: the image path's
    # activation codes keep the sign of a value that rounds to zero)
    assert torch.equal(Y.float() == g["Y"].float(), torch.ones_like(Y, dtype=torch.bool)), \
        f"rowmajor {mode} M={M}: differs from the image path"


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_equals_image_path_multi_tile(mode):
    """Several output tiles per workgroup, ragged rows and columns: identical
    to svdq_linear_forward on the pass's images."""
    spec = WL.LinearSpec("rowmajor_1100x512x13440", 1100, 512, 13440, 32, mode, x_outliers=4,
                         x_factor=20.0)
    _say("rowmajor vs image path", mode, spec.name)
    _image_path_equal(mode, spec, spec.M, 32, 7)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_workspace_reused_with_fewer_rows(mode):
    """One workspace for two calls, the second with fewer rows (its padded
    image is shorter, so stale bytes of the first lie past it): both equal
    the image path."""
    spec = WL.LinearSpec("rowmajor_600x1024x1024", 600, 1024, 1024, 16, mode, x_outliers=4,
                         x_factor=20.0)
    d = S.desc(mode, spec.K, spec.N, 16)
    ws = torch.empty(S.svdq_linear_rowmajor_workspace_size(d, 600), dtype=torch.uint8, device=DEV)
    for M, seed in ((600, 3), (200, 4)):
        _say("rowmajor workspace reuse", mode, "M", M)
        _image_path_equal(mode, spec, M, 16, seed, workspace=ws)
