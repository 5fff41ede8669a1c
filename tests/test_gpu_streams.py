"""Concurrent use of the library: two layers (INT4 and FP4, different
shapes) run on two HIP streams at once, and from two host threads each with
its own stream; every output is bit-identical to the same layer run alone.
The library keeps no per-call state between launches, so nothing but the
caller's buffers may differ."""
import threading

import pytest
import torch

import workloads as WL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)


def _layer(S, mode, M, K, N, r, seed):
    spec = WL.LinearSpec(f"streams_{mode}", M, K, N, r, mode, x_outliers=4, x_factor=20.0)
    X, W, b = WL.draw(spec, seed=seed)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    ld = (0.02 * torch.randn(r, K, device=DEV, generator=g)).to(torch.bfloat16)
    lu = (0.02 * torch.randn(N, r, device=DEV, generator=g)).to(torch.bfloat16)
    d = S.desc(mode, K, N, r)
    lam = S.svdq_calibrate_lambda(Xd, Wd)
    wc, ws = S.svdq_pack_weight(d, Wd, lam, ld, lu)
    wi = S.svdq_prepare_weight(d, wc, ws, lu, bd)
    xi = torch.empty(S.svdq_act_image_size(d, M), dtype=torch.uint8, device=DEV)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)

    def step():
        S.svdq_quantize_act(d, Xd, lam, ld, ximage=xi)
        S.svdq_linear_forward(d, M, xi, wi, Y)

    return step, Y


def _setup():
    from bit_diffusion_transformer_quantize_amd import svdq as S
    S.load()
    a = _layer(S, "int4", 300, 1024, 640, 32, 1)
    b = _layer(S, "fp4", 200, 512, 768, 16, 2)
    refs = []
    for step, Y in (a, b):
        step()
        torch.cuda.synchronize()
        refs.append(Y.clone())
    return (a, b), refs


def _same(Y, ref):
    return torch.equal(Y.view(torch.int16), ref.view(torch.int16))


def test_two_streams_match_alone():
    _say("two layers on two streams")
    layers, refs = _setup()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for (_, Y) in layers:
            Y.fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(4):
            for (step, _), s in zip(layers, streams):
                with torch.cuda.stream(s):
                    step()
        torch.cuda.synchronize()
        for (_, Y), ref in zip(layers, refs):
            assert _same(Y, ref), f"rep {rep}"


def test_two_host_threads_match_alone():
    _say("two layers from two host threads")
    layers, refs = _setup()
    errors = []

    def worker(step, Y, ref):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    step()
            s.synchronize()
            if not _same(Y, ref):
                errors.append("output differs")
        except Exception as e:  # reported in the main thread
            errors.append(repr(e))

    for (_, Y) in layers:
        Y.fill_(float("nan"))
    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(step, Y, ref))
               for (step, Y), ref in zip(layers, refs)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
