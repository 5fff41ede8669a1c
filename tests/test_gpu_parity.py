"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Codes, scales and lambda bit-exact; T and Y within the
stated tolerances.  Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import assert_T, assert_y, gpu_run, np_, oracle_offline, to_dev_bf16

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _full_check(spec, mode, M=None, seed=0, rank=None, out_f32=False, use_lowrank=True,
                with_bias=True, calibrate_on_gpu=True):
    rank = spec.rank if rank is None else rank
    X, W, b = WL.draw(spec, seed=seed, M=M)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    if not with_bias:
        b, bb = None, None
    lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, rank, mode)
    if not use_lowrank:
        L1 = np.zeros((xb.shape[1], 0), np.uint16)
        L2 = np.zeros((0, wb.shape[0]), np.uint16)
        wc_o, ws_o = O.pack_weight(wb, lam, L1, L2, mode)
    xc_o, xs_o, T_o, Xh = O.quantize_act(xb, lam, L1 if use_lowrank else None, mode)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2 if use_lowrank else None, bb, mode)
    _say(spec.name, mode, "M", X.shape[0], "rank", rank, "f32" if out_f32 else "bf16",
         "lowrank" if use_lowrank else "no-lowrank")
    g = gpu_run(DEV, X, W, b, lam, L1, L2, mode, rank, out_f32=out_f32,
                use_lowrank=use_lowrank, calibrate_on_gpu=calibrate_on_gpu)
    if calibrate_on_gpu:
        assert np.array_equal(np_(g["lam"]), lam), "lambda"
    assert np.array_equal(np_(g["wc"]), wc_o), "weight codes"
    assert np.array_equal(np_(g["ws"]), ws_o), "weight scales"
    assert np.array_equal(np_(g["xc"]), xc_o), "activation codes"
    assert np.array_equal(np_(g["xs"]), xs_o), "activation scales"
    if use_lowrank and rank > 0:
        assert_T(np_(g["T"]), T_o, Xh, L1, "T")
    y = np_(g["Y"].float())
    return assert_y(y, Y_o, out_f32, f"{spec.name} {mode}")


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_tiny_layer(mode):
    _full_check(WL.TINY, mode)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_tiny_layer_fp32_output(mode):
    _full_check(WL.TINY, mode, out_f32=True)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
@pytest.mark.parametrize("M", [1, 17, 130, 300])
def test_ragged_rows(mode, M):
    _full_check(WL.TINY, mode, M=M, seed=M)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
@pytest.mark.parametrize("rank", [32, 48, 128, 256])
def test_ranks(mode, rank):
    _full_check(WL.TINY, mode, M=96, rank=rank, seed=rank)


# Ranks 48..128 run the activation pass on 32-row workgroups: rows past M
# inside the second 16-row block, and 96 groups of K, which the pass splits
# into two K ranges whose partial T sums a second pass adds.
@pytest.mark.parametrize("mode", ["int4", "fp4"])
@pytest.mark.parametrize("M,rank", [(17, 64), (40, 96), (300, 128)])
def test_large_rank_ragged_split(mode, M, rank):
    spec = WL.LinearSpec(f"lr_{M}x6144x256_r{rank}", M, 6144, 256, rank, mode, x_outliers=4,
                         x_factor=20.0)
    _full_check(spec, mode, seed=M + rank)


# short K (few code stages per tile) with more output tiles than workgroups,
# so that workgroups walk several tiles and the DMA stream crosses tile
# boundaries from the pre-stages and the first code groups; 300 tiles take
# the round-robin tile order, 320 the per-XCD one
SHORT_K = [("int4", 128, 16, 11520), ("int4", 256, 128, 12288), ("int4", 384, 0, 11520),
           ("fp4", 128, 16, 16384), ("fp4", 256, 128, 13312), ("fp4", 384, 0, 16384)]


@pytest.mark.parametrize("mode,K,rank,N", SHORT_K)
def test_short_k_many_tiles(mode, K, rank, N):
    spec = WL.LinearSpec(f"shortk_1100x{K}x{N}", 1100, K, N, rank, mode, x_outliers=4,
                         x_factor=20.0)
    _full_check(spec, mode, seed=K + rank, use_lowrank=rank > 0)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_no_lowrank_no_bias(mode):
    _full_check(WL.TINY, mode, M=64, use_lowrank=False, with_bias=False)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_zero_residual(mode):
    """W = (L1 L2)^T / lambda with power-of-two lambda: the packed weight is
    all zero and the layer returns X W^T + b up to the output rounding."""
    rng = np.random.default_rng(7)
    M, K, N, r = 40, 256, 256, 16
    L1 = rng.integers(-3, 4, (K, r)).astype(np.float32)
    L2 = rng.integers(-3, 4, (r, N)).astype(np.float32)
    lam = np.ldexp(1.0, rng.integers(-2, 3, K)).astype(np.float32)
    W = O.f32_to_bf16(((L1 @ L2) / lam[:, None]).T.astype(np.float32))
    X = O.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    b = O.f32_to_bf16(0.01 * rng.standard_normal(N).astype(np.float32))
    L1b, L2b = O.f32_to_bf16(L1), O.f32_to_bf16(L2)
    wc_o, ws_o = O.pack_weight(W, lam, L1b, L2b, mode)
    assert np.all(wc_o == 0) and np.all(ws_o == 0)
    xc_o, xs_o, T_o, Xh = O.quantize_act(X, lam, L1b, mode)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2b, b, mode)
    _say("zero-residual", mode)
    g = gpu_run(DEV, WL.from_bits(X), WL.from_bits(W), WL.from_bits(b), lam, L1b, L2b, mode, r,
                out_f32=True)
    assert np.all(np_(g["wc"]) == 0) and np.all(np_(g["ws"]) == 0)
    assert np.array_equal(np_(g["xc"]), xc_o) and np.array_equal(np_(g["xs"]), xs_o)
    assert_T(np_(g["T"]), T_o, Xh, L1b, "T")
    assert_y(np_(g["Y"]), Y_o, True, "zero residual")


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_edge_values(mode):
    """Zero channels, all-zero rows, subnormal and huge activations, a
    negative-zero input, and lambda = 1 columns."""
    spec = WL.TINY
    X, W, b = WL.draw(spec, seed=11, M=70)
    xf = X.float()
    xf[:, 3] = 0.0                       # zero channel -> lambda 1
    xf[5, :] = 0.0                       # all-zero row -> zero scales
    xf[6, :] = -0.0
    xf[7, :64] = 1e-39                   # subnormal bf16 values
    xf[8, 100] = 3e4                     # huge outlier
    xf[9, :] *= 1e-30
    X = xf.to(torch.bfloat16)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, spec.rank, mode)
    xc_o, xs_o, T_o, Xh = O.quantize_act(xb, lam, L1, mode)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2, bb, mode)
    _say("edge values", mode)
    g = gpu_run(DEV, X, W, b, lam, L1, L2, mode, spec.rank, out_f32=True, calibrate_on_gpu=True)
    assert np.array_equal(np_(g["lam"]), lam)
    assert np.array_equal(np_(g["wc"]), wc_o) and np.array_equal(np_(g["ws"]), ws_o)
    assert np.array_equal(np_(g["xc"]), xc_o) and np.array_equal(np_(g["xs"]), xs_o)
    assert_T(np_(g["T"]), T_o, Xh, L1, "T")
    assert_y(np_(g["Y"]), Y_o, True, "edge values")


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_determinism_and_guard_bands(mode):
    """Two runs give bitwise-identical outputs, every byte of both operand
    images is written (the two runs pre-fill the buffers with different
    bytes), and nothing is written past the end of any output (canary bytes
    after each buffer stay intact)."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    spec = WL.TINY
    M = 131
    X, W, b = WL.draw(spec, seed=5, M=M)
    xb, wb = WL.bits(X), WL.bits(W)
    lam, L1, L2, _, _ = oracle_offline(xb, wb, spec.rank, mode)
    K, N, r = spec.K, spec.N, spec.rank
    d = S.desc(mode, K, N, r)
    _say("determinism/guard bands", mode)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    lamd = torch.from_numpy(lam).to(DEV)
    ld, lu = to_dev_bf16(L1.T, DEV), to_dev_bf16(L2.T, DEV)
    sdt = S.scale_dtype(mode)
    sc = S.scale_cols(mode, K)
    PAD = 4096

    def guarded(n, dtype, fill):
        buf = torch.empty((n * torch.tensor([], dtype=dtype).element_size() + PAD * 4,),
                          dtype=torch.uint8, device=DEV)
        buf.fill_(fill)
        return buf

    outs = []
    for fill in (0x5A, 0xA5):
        nimx, nimw = S.svdq_act_image_size(d, M), S.svdq_weight_image_size(d)
        sizes = dict(wc=N * K // 2, ws=N * sc * (4 if mode == "int4" else 1), xc=M * K // 2,
                     xs=M * sc * (4 if mode == "int4" else 1), T=M * r * 4, Y=M * N * 2,
                     xi=nimx, wi=nimw)
        bufs = {k: guarded(n, torch.uint8, fill) for k, n in sizes.items()}
        v = {k: bufs[k][:n] for k, n in sizes.items()}
        wc, ws = S.svdq_pack_weight(d, Wd, lamd, ld, lu, v["wc"].view(N, K // 2),
                                    v["ws"].view(sdt).view(N, sc))
        xc, xs, T, ximg = S.svdq_quantize_act(d, Xd, lamd, ld, v["xc"].view(M, K // 2),
                                              v["xs"].view(sdt).view(M, sc),
                                              v["T"].view(torch.float32).view(M, r), v["xi"])
        wimg = S.svdq_prepare_weight(d, wc, ws, lu, bd, v["wi"])
        Y = S.svdq_linear_forward(d, M, ximg, wimg, v["Y"].view(torch.bfloat16).view(M, N))
        torch.cuda.synchronize()
        for k, n in sizes.items():
            tail = bufs[k][n:].cpu().numpy()
            assert np.all(tail == fill), f"write past the end of {k}"
        outs.append([np_(t.view(torch.uint8)) for t in (wc, ws, xc, xs, T, Y, ximg, wimg)])
    for name, a, bb in zip(("wc", "ws", "xc", "xs", "T", "Y", "ximage", "wimage"), *outs):
        assert np.array_equal(a, bb), f"{name}: non-deterministic or partly unwritten"


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_unfused_schedule(mode):
    """quantize (no T) + stand-alone down-projection + GEMM (rank 0: no
    low-rank term) + stand-alone up-projection gives the same layer output."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    spec = WL.TINY
    X, W, b = WL.draw(spec, seed=9, M=200)
    xb, wb, bb = WL.bits(X), WL.bits(W), WL.bits(b)
    lam, L1, L2, wc_o, ws_o = oracle_offline(xb, wb, spec.rank, mode)
    xc_o, xs_o, T_o, Xh = O.quantize_act(xb, lam, L1, mode)
    Y_o = O.forward(xc_o, xs_o, T_o, wc_o, ws_o, L2, bb, mode)
    K, N, r = spec.K, spec.N, spec.rank
    _say("unfused schedule", mode)
    d = S.desc(mode, K, N, r, out_f32=True)
    d0 = S.desc(mode, K, N, 0, out_f32=True)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    lamd = torch.from_numpy(lam).to(DEV)
    ld, lu = to_dev_bf16(L1.T, DEV), to_dev_bf16(L2.T, DEV)
    wc, ws = S.svdq_pack_weight(d, Wd, lamd, ld, lu)
    xc, xs, _, ximg = S.svdq_quantize_act(d0, Xd, lamd, None, codes=True)
    T = S.svdq_lowrank_down(d, Xd, lamd, ld)
    Y = S.svdq_linear_forward(d0, 200, ximg, S.svdq_prepare_weight(d0, wc, ws, None, bd))
    S.svdq_lowrank_up(d, T, lu, Y)
    torch.cuda.synchronize()
    assert np.array_equal(np_(xc), xc_o) and np.array_equal(np_(xs), xs_o)
    assert_T(np_(T), T_o, Xh, L1, "T (stand-alone)")
    assert_y(np_(Y), Y_o, True, "unfused")


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_image_only_quantize(mode):
    """The activation image written without the row-major codes and T (the
    production call) gives the same layer output as the one written with
    them."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    spec = WL.TINY
    M = 77
    X, W, b = WL.draw(spec, seed=13, M=M)
    xb, wb = WL.bits(X), WL.bits(W)
    lam, L1, L2, _, _ = oracle_offline(xb, wb, spec.rank, mode)
    _say("image-only quantize", mode)
    g = gpu_run(DEV, X, W, b, lam, L1, L2, mode, spec.rank)
    d = S.desc(mode, spec.K, spec.N, spec.rank)
    lamd = torch.from_numpy(lam).to(DEV)
    _, _, _, ximg = S.svdq_quantize_act(d, X.to(DEV), lamd, to_dev_bf16(L1.T, DEV))
    Y = S.svdq_linear_forward(d, M, ximg, g["wimage"])
    torch.cuda.synchronize()
    assert np.array_equal(np_(ximg), np_(g["ximage"]))
    assert np.array_equal(np_(Y.view(torch.int16)), np_(g["Y"].view(torch.int16)))


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_split_k_quantize(mode):
    """K = 6144 with 300 rows: the activation pass splits K into two ranges
    and a second kernel adds the partial sums of T.  Codes, scales and T
    against the oracle, and the layer output."""
    spec = WL.LinearSpec("split_300x6144x256_r32", 300, 6144, 256, 32, mode,
                         x_outliers=6, x_factor=50.0)
    _full_check(spec, mode, seed=3)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_rows_past_2_31_elements(mode):
    """X of 2^22 + 77 rows x 512 (more than 2^31 elements, so row offsets
    need 64 bits): rows at the start, past the 2^31-element mark and at the
    ragged end equal, bit for bit, the same rows run as a separate 300-row
    layer (every output depends on its own row of X only, and both calls add
    in the same order).  Inputs drawn on the GPU; no oracle at this size."""
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    M, K, N, r = (1 << 22) + 77, 512, 256, 16
    _say("rows past 2^31 elements", mode, M, K, N, r)
    g = torch.Generator(device=DEV).manual_seed(5)
    X = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16)
    W = (0.02 * torch.randn(N, K, generator=g, device=DEV)).to(torch.bfloat16)
    b = (0.01 * torch.randn(N, generator=g, device=DEV)).to(torch.bfloat16)
    lam = S.svdq_calibrate_lambda(X[:4096], W)
    ld, lu, _ = S.svdq_lowrank_factors(W, lam, r, seed=0, want_sigma=False)
    d = S.desc(mode, K, N, r)
    wc, ws = S.svdq_pack_weight(d, W, lam, ld, lu)
    wi = S.svdq_prepare_weight(d, wc, ws, lu, b)
    xi = S.svdq_quantize_act(d, X, lam, ld)[3]
    Y = S.svdq_linear_forward(d, M, xi, wi)
    for m0 in (0, (1 << 22) - 250, M - 300):
        xs = S.svdq_quantize_act(d, X[m0:m0 + 300].contiguous(), lam, ld)[3]
        ys = S.svdq_linear_forward(d, 300, xs, wi)
        torch.cuda.synchronize()
        assert torch.equal(Y[m0:m0 + 300], ys), f"rows {m0}..{m0 + 299}"
    del X, Y, xi
    torch.cuda.empty_cache()
