"""GPU parity of the AWQ W4A16 linear layer (4-bit weights, 16-bit
activations) through the C ABI against the CPU oracle: packed codes, scales
and zero points bit-exact; Y within a bound derived from the kernel's fp32
arithmetic and within 1e-2 rms (plus the bf16 half-ulp of a bf16 output).  Every test prints its case before touching
the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from layer_util import assert_y

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _S():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    return S


def _spec(M, K, N, seed_outliers=True):
    return WL.LinearSpec(f"awq_{M}x{K}x{N}", M, K, N, 0, "awq", x_outliers=0, x_factor=1.0,
                         w_outliers=max(1, K // 200) if seed_outliers else 0, w_factor=10.0)


def _bf16_dev(bits):
    return WL.from_bits(bits).to(DEV)


def _pack_check(wb):
    """GPU packing of bf16 bits wb [N][K] against the oracle, bit for bit."""
    S = _S()
    c_o, s_o, z_o = O.awq_quantize(wb)
    c, s, z = S.svdq_awq_pack_weight(_bf16_dev(wb))
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), c_o), "codes"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), "scales"
    assert np.array_equal(z.cpu().numpy(), z_o), "zeros"
    return c_o, s_o, z_o


def _y_check(xb, c_o, s_o, z_o, bb, out_f32):
    """Run the GEMV on the oracle's codes and compare with the fp64 oracle."""
    S = _S()
    M, K = xb.shape
    N = c_o.shape[0]
    Y = torch.full((M, N), float("nan"), dtype=torch.float32 if out_f32 else torch.bfloat16,
                   device=DEV)
    S.svdq_awq_linear(_bf16_dev(xb), torch.from_numpy(c_o).to(DEV), torch.from_numpy(s_o).to(DEV),
                      torch.from_numpy(z_o).to(DEV), None if bb is None else _bf16_dev(bb), Y=Y,
                      out_f32=out_f32)
    y = Y.float().cpu().numpy().astype(np.float64)
    Y_o = O.awq_forward(xb, c_o, s_o, z_o, bb)
    assert np.all(np.isfinite(y)), "unwritten or non-finite outputs"
    # error bound of the kernel's arithmetic: per 16 weights, fp32 sums of
    # (128 + q) x and of x (magnitude <= 143 sum|x|, 8 roundings each) scaled
    # by s, then fp32 accumulation over K; plus the bf16 rounding of Y
    x = O.bf16_to_f32(xb).astype(np.float64)
    sg = np.repeat(s_o.astype(np.float64), 64, axis=1)              # [N][K]
    E = np.abs(x) @ sg.T                                              # sum_k s|x|
    A = np.abs(x) @ np.abs(O.awq_dequant(c_o, s_o, z_o)).T            # sum_k |w x|
    tol = 2.0 ** -12 * E + 2.0 ** -16 * A
    if not out_f32:
        tol = tol + 2.0 ** -8 * np.abs(Y_o)
    err = np.abs(y - Y_o)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"max excess at {worst}: err {err[worst]} tol {tol[worst]}"
    # and the layer-level bar: 1e-2 rms(Y), plus the bf16 half-ulp for bf16 Y
    assert_y(y, Y_o, out_f32, "awq")


@pytest.mark.parametrize("N,K", [(200, 3072), (37, 4224), (1, 128), (16, 256)])
def test_awq_pack_bit_exact(N, K):
    _say("awq pack", N, K)
    X, W, b = WL.draw(_spec(1, K, N), seed=3)
    wb = WL.bits(W)
    if N >= 16:
        # special groups: constant zero, constant positive, all positive, all
        # negative, below the step floor, large magnitude, an exact 4-bit grid
        w = O.bf16_to_f32(wb).copy()
        w[0, :64] = 0.0
        w[1, :64] = 0.75
        w[2, :64] = np.abs(w[2, :64]) + 0.5
        w[3, :64] = -np.abs(w[3, :64]) - 0.25
        w[4, :64] = 1e-7 * np.arange(64, dtype=np.float32)
        w[5, :64] = 3e4 * w[5, :64]
        q = np.arange(64) % 16
        w[6, :64] = (2.0 ** -7) * (q - 5).astype(np.float32)
        wb = (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    _pack_check(wb)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9])
def test_awq_linear_small_batch(M):
    N, K = 200, 3072
    _say("awq linear", M, K, N)
    X, W, b = WL.draw(_spec(M, K, N), seed=M)
    c, s, z = O.awq_quantize(WL.bits(W))
    _y_check(WL.bits(X), c, s, z, WL.bits(b), out_f32=False)


@pytest.mark.parametrize("M,K,N,bias,f32", [(4, 3072, 200, True, True), (1, 3072, 64, False, False),
                                            (2, 4224, 37, True, False), (6, 4224, 37, False, True),
                                            (1, 128, 1, True, False), (3, 256, 16, True, True)])
def test_awq_linear_shapes(M, K, N, bias, f32):
    _say("awq linear", M, K, N, "bias" if bias else "no-bias", "f32" if f32 else "bf16")
    X, W, b = WL.draw(_spec(M, K, N), seed=7)
    c, s, z = O.awq_quantize(WL.bits(W))
    _y_check(WL.bits(X), c, s, z, WL.bits(b) if bias else None, out_f32=f32)


@pytest.mark.parametrize("M", [1, 2])
def test_awq_full_size_modulation(M):
    """The FLUX double-stream modulation shape, 3072 -> 18432, end to end
    through the C ABI: GPU packing bit-exact, then the GEMV on its codes."""
    spec = WL.modulation_specs(M)[0][0]
    _say("awq full size", spec.name)
    X, W, b = WL.draw(spec, seed=0)
    c, s, z = _pack_check(WL.bits(W))
    _y_check(WL.bits(X), c, s, z, WL.bits(b), out_f32=False)


def _graph_replays_match(run, Y, reps=3):
    """Capture run() (which writes Y) in a HIP graph; replay it reps times
    with eager work and synchronisation between replays, each replay
    bit-identical to the eager result."""
    run()
    torch.cuda.synchronize()
    ref = Y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(reps):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"


def test_awq_graph_replay_matches_eager():
    S = _S()
    M, K, N = 2, 3072, 4096
    _say("awq graph replay", M, K, N)
    X, W, b = WL.draw(_spec(M, K, N), seed=11)
    c, s, z = S.svdq_awq_pack_weight(W.to(DEV))
    Xd, bd = X.to(DEV), b.to(DEV)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    _graph_replays_match(lambda: S.svdq_awq_linear(Xd, c, s, z, bd, Y=Y), Y)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_w4a4_graph_replay_matches_eager(mode):
    """The W4A4 step (quantize_act into the image, then the GEMM) replayed
    from a HIP graph; K = 6144 makes the quantize pass split K."""
    S = _S()
    M, K, N, r = 300, 6144, 256, 32
    _say("w4a4 graph replay", mode, M, K, N, r)
    spec = WL.LinearSpec("graph", M, K, N, r, mode, x_outliers=8, x_factor=30.0)
    X, W, b = WL.draw(spec, seed=5)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    g = torch.Generator(device=DEV).manual_seed(5)
    ld = (0.02 * torch.randn(r, K, device=DEV, generator=g)).to(torch.bfloat16)
    lu = (0.02 * torch.randn(N, r, device=DEV, generator=g)).to(torch.bfloat16)
    d = S.desc(mode, K, N, r)
    lam = S.svdq_calibrate_lambda(Xd, Wd)
    wc, ws = S.svdq_pack_weight(d, Wd, lam, ld, lu)
    wi = S.svdq_prepare_weight(d, wc, ws, lu, bd)
    xi = torch.empty(S.svdq_act_image_size(d, M), dtype=torch.uint8, device=DEV)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)

    def run():
        S.svdq_quantize_act(d, Xd, lam, ld, ximage=xi)
        S.svdq_linear_forward(d, M, xi, wi, Y)
    _graph_replays_match(run, Y)


@pytest.mark.parametrize("K", [128, 256])
def test_awq_linear_streaming_single_row(K):
    """M = 1 with N large enough for the streaming kernel (several blocks
    per resident wave); K = 128 leaves most lanes without a unit."""
    M, N = 1, 140000
    _say("awq linear streaming", M, K, N)
    X, W, b = WL.draw(_spec(M, K, N), seed=13)
    c, s, z = O.awq_quantize(WL.bits(W))
    _y_check(WL.bits(X), c, s, z, WL.bits(b), out_f32=False)


def test_awq_fused_modulation_sampled():
    """All 77 modulation maps of a FLUX.1 forward as one call: the packed
    weights of the three layer shapes concatenated along N (38 + 38 + 1
    copies, 1,056,768 rows), M = 1; 1024 sampled outputs against the oracle
    of their source layer."""
    S = _S()
    plan = WL.modulation_specs(1)
    _say("awq fused modulation", sum(sp.N * n for sp, n in plan), "rows")
    X = None
    parts, oracle_parts = [], []
    for spec, count in plan:
        Xs, W, b = WL.draw(spec, seed=0)
        X = Xs if X is None else X        # the shared conditioning vector
        c, s, z = _pack_check(WL.bits(W))
        cd, sd, zd = (torch.from_numpy(a).to(DEV) for a in (c, s, z))
        bd = b.to(DEV)
        parts.append((cd, sd, zd, bd, count))
        oracle_parts.append((spec.N, count, c, s, z, WL.bits(b)))
    C = torch.cat([p[0] for p in parts for _ in range(p[4])])
    Sc = torch.cat([p[1] for p in parts for _ in range(p[4])])
    Z = torch.cat([p[2] for p in parts for _ in range(p[4])])
    B = torch.cat([p[3] for p in parts for _ in range(p[4])])
    N = C.shape[0]
    xb = WL.bits(X)
    Y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    S.svdq_awq_linear(X.to(DEV), C, Sc, Z, B, Y=Y)
    y = Y.float().cpu().numpy()[0].astype(np.float64)
    del C, Sc, Z, B
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(N, 1024, replace=False))
    # map each sampled row to (layer shape, row within the layer)
    starts, off = [], 0
    for n, count, *_ in oracle_parts:
        starts.append(off)
        off += n * count
    got, want, ref_rows = [], [], []
    for r in rows:
        k = max(i for i, st in enumerate(starts) if st <= r)
        n, count, c, s, z, bb = oracle_parts[k]
        ref_rows.append((k, (r - starts[k]) % n))
    for k in range(len(oracle_parts)):
        sel = [i for i, (kk, _) in enumerate(ref_rows) if kk == k]
        if not sel:
            continue
        lr = np.array([ref_rows[i][1] for i in sel])
        n, count, c, s, z, bb = oracle_parts[k]
        Yo = O.awq_forward(xb, c[lr], s[lr], z[lr], bb[lr])[0]
        x = O.bf16_to_f32(xb).astype(np.float64)
        sg = np.repeat(s[lr].astype(np.float64), 64, axis=1)
        E = (np.abs(x) @ sg.T)[0]
        A = (np.abs(x) @ np.abs(O.awq_dequant(c[lr], s[lr], z[lr])).T)[0]
        tol = 2.0 ** -12 * E + 2.0 ** -16 * A + 2.0 ** -8 * np.abs(Yo)
        err = np.abs(y[rows[sel]] - Yo)
        assert np.all(err <= tol), f"layer shape {k}: max excess {(err - tol).max()}"
