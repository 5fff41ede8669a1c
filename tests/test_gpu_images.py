"""The operand images the GEMM reads, decoded on the host and compared with
what they stand for: every activation and weight code and scale bit for bit
with the oracle, T's bf16 halves bit for bit with the split of the fp32 T
the same call returns (itself checked against the oracle), L2 and the bias bit
for bit with the inputs, and the padding zero.  The layouts are those
include/svdq.h documents; the decoder is tests/image_decode.py."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from image_decode import decode_act_image, decode_weight_image
from layer_util import assert_T, gpu_run, np_, oracle_offline

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _split_bf16(v32: np.ndarray):
    """(hi, lo) bf16 bit patterns: hi = bf16_RNE(v), lo = bf16_RNE(v - hi)
    (the fp32 difference is exact)."""
    v32 = np.asarray(v32, np.float32)
    hi = O.f32_to_bf16(v32)
    lo = O.f32_to_bf16((v32 - O.bf16_to_f32(hi)).astype(np.float32))
    return hi, lo


def _scale_dwords(s: np.ndarray, pattern: str) -> np.ndarray:
    """The 4 dwords of the INT4 scale operand (slot r dwords 0, 1; slot
    32 + r dwords 0, 1) for fp32 scales s [rows][G]."""
    hi, lo = _split_bf16(s)
    hi, lo = hi.astype(np.uint32), lo.astype(np.uint32)
    z = np.zeros_like(hi)
    if pattern == "act":
        return np.stack([hi | (lo << 16), hi, lo, z], axis=-1)
    return np.stack([hi | (hi << 16), lo, lo, z], axis=-1)


CASES = [
    ("int4", 300, 512, 384, 16),     # ragged M, INT4 columns padded to 384
    ("int4", 256, 512, 256, 0),      # no low-rank branch
    ("int4", 300, 6144, 256, 32),    # K split into two ranges (partial sums + second pass)
    ("fp4", 300, 512, 384, 16),      # FP4 columns padded to 512
    ("fp4", 77, 1024, 128, 32),
    ("fp4", 300, 6144, 256, 16),
]


@pytest.mark.parametrize("mode,M,K,N,rank", CASES)
def test_images_decode_to_the_oracle(mode, M, K, N, rank):
    print("[case]", mode, M, K, N, rank, flush=True)
    spec = WL.LinearSpec(f"img_{mode}_{M}x{K}x{N}_r{rank}", M, K, N, rank, mode,
                         x_outliers=4, x_factor=50.0)
    X, W, b = WL.draw(spec, seed=11)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, rank, mode)
    xc_o, xs_o, T_o, Xh = O.quantize_act(xb, lam, L1, mode)
    g = gpu_run(DEV, X, W, b, lam, L1, L2, mode, rank, use_lowrank=rank > 0)

    a = decode_act_image(np_(g["ximage"]), mode, M, K, rank)
    Mp = a["codes"].shape[0]
    assert np.array_equal(a["codes"][:M], xc_o), "activation codes in the image"
    assert not a["codes"][M:].any(), "padding rows of the activation image"
    if mode == "int4":
        assert np.array_equal(a["scales"][:M], _scale_dwords(xs_o, "act")), "activation scales"
        assert not a["scales"][M:].any()
    else:
        assert np.array_equal(a["scales"][:M], xs_o), "activation scale bytes"
        assert not a["scales"][M:].any()
    if rank > 0:
        T = np_(g["T"])
        assert_T(T, T_o, Xh, L1, "T")
        hi, lo = _split_bf16(T)
        assert np.array_equal(a["t_hi"][:M], hi), "T high halves"
        assert np.array_equal(a["t_lo"][:M], lo), "T low halves"
        assert not a["t_hi"][M:].any() and not a["t_lo"][M:].any(), "T of padding rows"
        assert Mp == a["layout"]["RT"] * 32

    w = decode_weight_image(np_(g["wimage"]), mode, N, K, rank)
    assert np.array_equal(w["codes"][:N], wc_o), "weight codes in the image"
    assert not w["codes"][N:].any(), "padding columns of the weight image"
    if mode == "int4":
        assert np.array_equal(w["scales"][:N], _scale_dwords(ws_o, "weight")), "weight scales"
    else:
        assert np.array_equal(w["scales"][:N], ws_o), "weight scale bytes"
    assert not w["scales"][N:].any()
    if rank > 0:
        assert np.array_equal(w["lora_up"][:N], np.ascontiguousarray(L2.T)), "L2 in the image"
        assert not w["lora_up"][N:].any()
    assert np.array_equal(w["bias"][:N], bb), "bias in the image"
    assert not w["bias"][N:].any() and not w["tail"].any(), "bias padding and tail"


@pytest.mark.parametrize("mode,M,K,N,rank", [CASES[0], CASES[1], CASES[3], CASES[4]])
def test_rowmajor_workspace_images_decode_to_the_oracle(mode, M, K, N, rank):
    """svdq_linear_forward_rowmajor writes both images into its workspace
    (the activation image, then the prepared weight at the next 256-byte
    boundary) from the oracle's own row-major tensors: decoded, they hold
    those tensors bit for bit (T's halves: the split of the fp32 T handed
    over), zero padding included."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    from image_decode import act_layout, weight_layout
    from layer_util import to_dev_bf16
    print("[case] rowmajor workspace images", mode, M, K, N, rank, flush=True)
    spec = WL.LinearSpec(f"rmimg_{mode}_{M}x{K}x{N}_r{rank}", M, K, N, rank, mode,
                         x_outliers=4, x_factor=50.0)
    X, W, b = WL.draw(spec, seed=13)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    if rank > 0:
        lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, rank, mode)
    else:
        lam = O.calibrate_lambda(xb, wb)
        L1 = np.zeros((K, 0), np.uint16)
        L2 = np.zeros((0, N), np.uint16)
        wc_o, ws_o = O.pack_weight(wb, lam, L1, L2, mode)
    xc_o, xs_o, T_o, _ = O.quantize_act(xb, lam, L1 if rank > 0 else None, mode)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    T32 = T_o.astype(np.float32) if rank > 0 else None
    d = S.desc(mode, K, N, rank)
    ws = torch.full((S.svdq_linear_rowmajor_workspace_size(d, M),), 0xA5, dtype=torch.uint8,
                    device=DEV)
    S.svdq_linear_forward_rowmajor(d, t(xc_o), t(xs_o), None if T32 is None else t(T32), t(wc_o),
                                   t(ws_o), to_dev_bf16(L2.T, DEV) if rank > 0 else None,
                                   b.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    buf = np_(ws)
    al, wl = act_layout(mode, M, K, rank), weight_layout(mode, N, K, rank)
    xoff = (al["bytes"] + 255) // 256 * 256
    # the partial-sum region of the activation image is not the GEMM's input
    # and is not written; compare up to it
    a = decode_act_image(np.concatenate([buf[:al["tpart"]],
                                         np.zeros(al["bytes"] - al["tpart"], np.uint8)]),
                         mode, M, K, rank)
    assert np.array_equal(a["codes"][:M], xc_o), "activation codes"
    assert not a["codes"][M:].any(), "padding rows of the activation image"
    if mode == "int4":
        assert np.array_equal(a["scales"][:M], _scale_dwords(xs_o, "act")), "activation scales"
    else:
        assert np.array_equal(a["scales"][:M], xs_o), "activation scale bytes"
    assert not a["scales"][M:].any()
    if rank > 0:
        hi, lo = _split_bf16(T32)
        assert np.array_equal(a["t_hi"][:M], hi), "T high halves"
        assert np.array_equal(a["t_lo"][:M], lo), "T low halves"
        assert not a["t_hi"][M:].any() and not a["t_lo"][M:].any(), "T of padding rows"
    w = decode_weight_image(buf[xoff:xoff + wl["bytes"]], mode, N, K, rank)
    assert np.array_equal(w["codes"][:N], wc_o), "weight codes"
    if mode == "int4":
        assert np.array_equal(w["scales"][:N], _scale_dwords(ws_o, "weight")), "weight scales"
    else:
        assert np.array_equal(w["scales"][:N], ws_o), "weight scale bytes"
    assert np.array_equal(w["bias"][:N], bb), "bias"
