"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any HIP call (no GPU
is needed for any of this; nothing here launches a kernel)."""
import ctypes

import pytest

from bit_diffusion_transformer_quantize_amd import svdq as S

ARG, SHAPE, HIP = 1, 2, 4
A = 0x10000          # a 16-byte-aligned address that is never dereferenced
MIS = 0x10008        # a misaligned one


def _lib():
    return S.load()


def _d(mode=0, K=512, N=512, rank=16, flags=0):
    return ctypes.byref(S.SvdqDesc(mode, K, N, rank, flags))


def _xb(M=256, **kw):
    """The activation image size the library gives for _d(**kw) and M (0 if
    the descriptor or M is invalid)."""
    n = ctypes.c_size_t(0)
    st = _lib().svdq_act_image_size(_d(**kw), M, ctypes.byref(n))
    return n.value if st == 0 else 0


def _wb(**kw):
    n = ctypes.c_size_t(0)
    st = _lib().svdq_weight_image_size(_d(**kw), ctypes.byref(n))
    return n.value if st == 0 else 0


def test_exports_every_header_symbol():
    lib = _lib()
    names = S.header_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for code in range(5):
        assert S.svdq_status_string(code).startswith(S.STATUS[code])
    assert S.svdq_version() == "0.1.0"


@pytest.mark.parametrize("name,ok", [("gfx950", True), ("gfx950:sramecc+:xnack-", True),
                                     ("gfx9500", False), ("gfx942", False), ("gfx90a", False),
                                     ("", False), ("gfx95", False)])
def test_arch_predicate(name, ok):
    assert S.svdq_arch_supported(name) is ok


def test_arch_predicate_null():
    assert _lib().svdq_arch_supported(None) == 0


def _act_bytes(mode, M, K, rank):
    """Activation image size from the documented blocks: rows padded to 256;
    per (64-group, 32 rows) 2048 bytes (INT4) or 1024 + 64 bytes (FP4); per
    (16 ranks, 32 rows) 2048 bytes of T; with rank > 0 and S > 1 K ranges
    (S = ceil(1024 / 16-row blocks), at most 16 and at most (K/64)/48) S
    fp32 partial sums of T per padded row."""
    rt = -(-M // 256) * 8
    per = 2048 if mode == 0 else 1024 + 64
    S = max(1, min(16, -(-1024 // (rt * 2)), (K // 64) // 48))
    part = S * rt * 32 * rank * 4 if rank > 0 and S > 1 else 0
    return (K // 64) * rt * per + (rank // 16) * rt * 2048 + part


def _weight_bytes(mode, N, K, rank):
    """Weight image size: columns padded to 192 (INT4) or 256 (FP4); code
    blocks as above, 1024 bytes of L2 per (16 ranks, 32 columns), 64 bytes of
    bias per 32 columns and a 1024-byte zero tail."""
    ct = -(-N // (192 if mode == 0 else 256)) * (6 if mode == 0 else 8)
    per = 2048 if mode == 0 else 1024 + 64
    return (K // 64) * ct * per + (rank // 16) * ct * 1024 + ct * 64 + 1024


@pytest.mark.parametrize("mode,M,K,rank", [(0, 300, 512, 16), (0, 256, 512, 0), (1, 256, 512, 16),
                                           (1, 1, 128, 32), (0, 4096, 3072, 32),
                                           (1, 4096, 3072, 32), (0, 300, 6144, 32),
                                           (0, 4608, 12288, 32), (1, 1024, 12288, 128),
                                           (0, 8192, 12288, 0)])
def test_act_image_size_is_host_only(mode, M, K, rank):
    n = ctypes.c_size_t(123)
    assert _lib().svdq_act_image_size(_d(mode=mode, K=K, rank=rank), M, ctypes.byref(n)) == 0
    assert n.value == _act_bytes(mode, M, K, rank)


def test_act_image_size_validation():
    n = ctypes.c_size_t(0)
    assert _lib().svdq_act_image_size(_d(), 256, None) == ARG
    assert _lib().svdq_act_image_size(_d(K=96), 256, ctypes.byref(n)) == SHAPE
    assert _lib().svdq_act_image_size(_d(), 0, ctypes.byref(n)) == SHAPE
    assert _lib().svdq_act_image_size(None, 256, ctypes.byref(n)) == ARG


@pytest.mark.parametrize("mode,N,K,rank", [(0, 256, 512, 16), (0, 9216, 3072, 32),
                                           (1, 256, 512, 16), (1, 21504, 3072, 32),
                                           (1, 128, 128, 0), (0, 128, 128, 256)])
def test_weight_image_size_is_host_only(mode, N, K, rank):
    n = ctypes.c_size_t(0)
    assert _lib().svdq_weight_image_size(_d(mode=mode, K=K, N=N, rank=rank), ctypes.byref(n)) == 0
    assert n.value == _weight_bytes(mode, N, K, rank)


def test_weight_image_size_validation():
    n = ctypes.c_size_t(0)
    assert _lib().svdq_weight_image_size(_d(), None) == ARG
    assert _lib().svdq_weight_image_size(_d(N=200), ctypes.byref(n)) == SHAPE


def test_prepare_weight_validation():
    p = _lib().svdq_prepare_weight
    wb = _wb()
    assert p(None, A, A, A, A, A, wb, None) == ARG
    assert p(_d(mode=3), A, A, A, A, A, wb, None) == ARG
    assert p(_d(K=96), A, A, A, A, A, wb, None) == SHAPE
    assert p(_d(), None, A, A, A, A, wb, None) == ARG               # codes null
    assert p(_d(), A, MIS, A, A, A, wb, None) == ARG                # scales misaligned
    assert p(_d(), A, A, None, A, A, wb, None) == ARG               # rank > 0 needs lora_up
    assert p(_d(rank=0), A, A, A, A, A, _wb(rank=0), None) == ARG   # rank 0 forbids it
    assert p(_d(), A, A, A, MIS, A, wb, None) == ARG                # bias misaligned
    assert p(_d(), A, A, A, A, None, wb, None) == ARG               # image null
    # the image must be exactly svdq_weight_image_size bytes
    assert p(_d(), A, A, A, A, A, wb - 16, None) == ARG
    assert p(_d(), A, A, A, A, A, wb + 16, None) == ARG
    assert p(_d(), A, A, A, A, A, 0, None) == ARG
    assert p(_d(), A, A, A, A, A, _wb(rank=32), None) == ARG        # built for another rank
    assert p(_d(), A, A, A, A, A, _wb(mode=1), None) == ARG         # built for another mode


@pytest.mark.parametrize("kw,status", [
    (dict(mode=2), ARG), (dict(mode=-1), ARG), (dict(flags=4), ARG),
    (dict(K=0), SHAPE), (dict(K=64), SHAPE), (dict(K=100), SHAPE), (dict(K=1 << 21), SHAPE),
    (dict(N=0), SHAPE), (dict(N=64), SHAPE), (dict(N=200), SHAPE),
    (dict(rank=8), SHAPE), (dict(rank=-16), SHAPE), (dict(rank=272), SHAPE),
])
def test_desc_validation(kw, status):
    lib = _lib()
    d = _d(**kw)
    assert lib.svdq_quantize_act(d, 256, A, A, A, A, A, A, A, 1 << 20, None) == status
    assert lib.svdq_pack_weight(d, A, A, A, A, A, A, None) == status
    assert lib.svdq_prepare_weight(d, A, A, A, A, A, 1 << 20, None) == status
    assert lib.svdq_linear_forward(d, 256, A, 1 << 20, A, 1 << 20, A, None) == status
    assert lib.svdq_lowrank_down(d, 256, A, A, A, A, None) == status
    assert lib.svdq_lowrank_up(d, 256, A, A, A, None) == status


def test_null_desc():
    lib = _lib()
    assert lib.svdq_quantize_act(None, 256, A, A, A, A, A, A, A, _xb(), None) == ARG
    assert lib.svdq_linear_forward(None, 256, A, _xb(), A, _wb(), A, None) == ARG


@pytest.mark.parametrize("M", [0, -1, 1 << 40])
def test_rows_validation(M):
    lib = _lib()
    assert lib.svdq_quantize_act(_d(), M, A, A, A, A, A, A, A, _xb(), None) == SHAPE
    assert lib.svdq_linear_forward(_d(), M, A, _xb(), A, _wb(), A, None) == SHAPE
    assert lib.svdq_calibrate_lambda(M, 512, 512, A, A, A, None) == SHAPE


def test_quantize_act_pointer_validation():
    lib = _lib()
    xb = _xb()

    def q(d, M, X, lam, ld, xc, xs, T, xi, nb=None):
        if nb is None:
            nb = 0 if xi is None else xb
        return lib.svdq_quantize_act(d, M, X, lam, ld, xc, xs, T, xi, nb, None)

    assert q(_d(), 256, None, A, A, A, A, A, A) == ARG        # X null
    assert q(_d(), 256, MIS, A, A, A, A, A, A) == ARG         # X misaligned
    assert q(_d(), 256, A, None, A, A, A, A, A) == ARG        # lambda null
    assert q(_d(), 256, A, A, A, None, A, A, A) == ARG        # codes without scales
    assert q(_d(), 256, A, A, A, A, None, A, A) == ARG        # scales without codes
    assert q(_d(), 256, A, A, None, A, A, A, None) == ARG     # T needs lora_down
    assert q(_d(), 256, A, A, None, A, A, None, A) == ARG     # image needs lora_down
    assert q(_d(), 256, A, A, A, A, A, None, None) == ARG     # lora_down unused
    assert q(_d(), 256, A, A, MIS, A, A, A, A) == ARG         # lora_down misaligned
    assert q(_d(rank=0), 256, A, A, A, A, A, None, A, _xb(rank=0)) == ARG  # lora_down, rank 0
    assert q(_d(rank=0), 256, A, A, None, A, A, A, A, _xb(rank=0)) == ARG  # T with rank 0
    assert q(_d(), 256, A, A, A, A, A, MIS, A) == ARG         # T misaligned
    assert q(_d(), 256, A, A, A, A, A, A, MIS) == ARG         # image misaligned
    assert q(_d(), 256, A, A, A, None, None, None, None) == ARG   # no output
    # the image must be exactly svdq_act_image_size bytes, and 0 without one
    assert q(_d(), 256, A, A, A, A, A, A, A, xb - 16) == ARG
    assert q(_d(), 256, A, A, A, A, A, A, A, xb + 1) == ARG
    assert q(_d(), 256, A, A, A, A, A, A, None, xb) == ARG
    assert q(_d(), 256, A, A, A, A, A, A, A, _xb(M=512)) == ARG          # another M
    assert q(_d(), 256, A, A, A, A, A, A, A, _xb(rank=32)) == ARG        # another rank
    assert q(_d(), 256, A, A, A, A, A, A, A, _xb(mode=1)) == ARG         # another mode


def test_pack_weight_pointer_validation():
    lib = _lib()
    p = lib.svdq_pack_weight
    assert p(_d(), None, A, A, A, A, A, None) == ARG
    assert p(_d(), A, A, None, A, A, A, None) == ARG             # rank>0 needs lora_down
    assert p(_d(), A, A, A, None, A, A, None) == ARG             # and lora_up
    assert p(_d(rank=0), A, A, A, None, A, A, None) == ARG       # rank 0 forbids them
    assert p(_d(), A, A, A, A, None, A, None) == ARG
    assert p(_d(), A, A, A, A, A, MIS, None) == ARG


def test_linear_forward_pointer_validation():
    lib = _lib()
    xb, wb = _xb(), _wb()

    def f(d, M, xi, wi, Y, nx=xb, nw=wb):
        return lib.svdq_linear_forward(d, M, xi, nx, wi, nw, Y, None)

    assert f(_d(), 256, None, A, A) == ARG    # activation image null
    assert f(_d(), 256, MIS, A, A) == ARG     # misaligned
    assert f(_d(), 256, A, None, A) == ARG    # weight image null
    assert f(_d(), 256, A, MIS, A) == ARG
    assert f(_d(), 256, A, A, None) == ARG    # Y null
    assert f(_d(), 256, A, A, MIS) == ARG
    # output larger than 2^46 elements
    assert f(_d(N=1 << 20), 1 << 27, A, A, A) == SHAPE


def test_linear_forward_packed_validation():
    """The packed-weight forward checks its arguments as svdq_prepare_weight and
    svdq_linear_forward do, the scratch against svdq_weight_image_size, before
    anything is enqueued."""
    lib = _lib()
    xb, wb = _xb(), _wb()

    def f(d, M=256, xi=A, nx=xb, wc=A, ws=A, lu=A, b=A, sc=A, ns=wb, Y=A):
        return lib.svdq_linear_forward_packed(d, M, xi, nx, wc, ws, lu, b, sc, ns, Y, None)

    assert f(None) == ARG
    assert f(_d(mode=3)) == ARG
    assert f(_d(K=96)) == SHAPE
    assert f(_d(), M=0) == SHAPE
    assert f(_d(N=1 << 20), M=1 << 27) == SHAPE                   # output past 2^46 elements
    assert f(_d(), xi=None) == ARG
    assert f(_d(), xi=MIS) == ARG
    assert f(_d(), wc=None) == ARG                                # codes null
    assert f(_d(), ws=MIS) == ARG                                 # scales misaligned
    assert f(_d(), lu=None) == ARG                                # rank > 0 needs lora_up
    assert f(_d(rank=0), nx=_xb(rank=0), ns=_wb(rank=0)) == ARG   # rank 0 forbids it
    assert f(_d(), b=MIS) == ARG                                  # bias misaligned
    assert f(_d(), sc=None) == ARG                                # scratch null
    assert f(_d(), Y=None) == ARG
    assert f(_d(), ns=wb - 16) == ARG                             # scratch of another size
    assert f(_d(), ns=_wb(mode=1)) == ARG
    assert f(_d(), nx=_xb(M=1024)) == ARG                         # activation image for another M


def _rb(M=256, **kw):
    n = ctypes.c_size_t(0)
    st = _lib().svdq_linear_rowmajor_workspace_size(_d(**kw), M, ctypes.byref(n))
    return n.value if st == 0 else 0


def test_linear_forward_rowmajor_validation():
    """The row-major forward checks every tensor pointer, the rank rule for T
    and lora_up, and the workspace against svdq_linear_rowmajor_workspace_size
    (the activation image rounded up to 256 bytes, then the prepared weight),
    before anything is enqueued."""
    lib = _lib()
    for kw in (dict(), dict(mode=1), dict(rank=0), dict(K=3072, N=9216, rank=32)):
        for M in (1, 256, 300):
            xb = (_xb(M=M, **kw) + 255) // 256 * 256
            assert _rb(M=M, **kw) == xb + _wb(**kw)
    n = ctypes.c_size_t(0)
    assert lib.svdq_linear_rowmajor_workspace_size(_d(), 256, None) == ARG
    assert lib.svdq_linear_rowmajor_workspace_size(_d(K=96), 256, ctypes.byref(n)) == SHAPE
    assert lib.svdq_linear_rowmajor_workspace_size(_d(), 0, ctypes.byref(n)) == SHAPE
    rb = _rb()

    def f(d, M=256, xc=A, xs=A, T=A, wc=A, ws=A, lu=A, b=A, Y=A, w=A, nw=rb):
        return lib.svdq_linear_forward_rowmajor(d, M, xc, xs, T, wc, ws, lu, b, Y, w, nw, None)

    assert f(None) == ARG
    assert f(_d(mode=3)) == ARG
    assert f(_d(K=96)) == SHAPE
    assert f(_d(), M=0) == SHAPE
    assert f(_d(N=1 << 20), M=1 << 27) == SHAPE                   # output past 2^46 elements
    for name in ("xc", "xs", "wc", "ws", "Y", "w"):
        assert f(_d(), **{name: None}) == ARG, name
        assert f(_d(), **{name: MIS}) == ARG, name
    assert f(_d(), b=MIS) == ARG                                  # bias misaligned
    assert f(_d(), T=None) == ARG                                 # rank > 0 needs T
    assert f(_d(), lu=None) == ARG                                # and lora_up
    assert f(_d(), T=MIS) == ARG
    assert f(_d(rank=0), nw=_rb(rank=0)) == ARG                   # rank 0 takes neither
    assert f(_d(rank=0), lu=None, nw=_rb(rank=0)) == ARG
    assert f(_d(), nw=rb - 1) == ARG                              # workspace too small
    assert f(_d(), M=300, nw=_rb(M=256)) == ARG                   # one sized for fewer rows


@pytest.mark.parametrize("what,kw", [
    ("activation image for another M", dict(nx=_xb(M=1024))),
    ("activation image for another rank", dict(nx=_xb(rank=32))),
    ("activation image for rank 0", dict(nx=_xb(rank=0))),
    ("activation image for another mode", dict(nx=_xb(mode=1))),
    ("activation image for another K", dict(nx=_xb(K=1024))),
    ("weight image for another rank", dict(nw=_wb(rank=32))),
    ("weight image for another mode", dict(nw=_wb(mode=1))),
    ("weight image for another N", dict(nw=_wb(N=1024))),
    ("weight image for another K", dict(nw=_wb(K=1024))),
    ("truncated activation image", dict(nx=_xb() - 16)),
    ("truncated weight image", dict(nw=_wb() - 16)),
    ("zero sizes", dict(nx=0, nw=0)),
])
def test_linear_forward_rejects_mismatched_images(what, kw):
    """An image whose size is not the one desc and M give is refused on the
    host (SVDQ_ERR_ARG) before anything is enqueued: a GEMM launched on it
    would address past the buffer."""
    lib = _lib()
    nx, nw = kw.get("nx", _xb()), kw.get("nw", _wb())
    assert lib.svdq_linear_forward(_d(), 256, A, nx, A, nw, A, None) == ARG, what
    d = _d(N=9216, rank=16)
    g = lib.svdq_linear_forward_qk
    nxq = kw.get("nx", _xb())
    nwq = kw.get("nw", _wb(N=9216))
    assert g(d, 256, A, nxq, A, nwq, 24, A, A, A, A, 1e-6, A, None) == ARG, what


def test_same_padded_rows_share_an_image_size():
    """Activation rows are padded to a multiple of 256, so M = 200 and 256
    give the same image: an image written for one is in bounds for the other
    (rows past the smaller M are zero)."""
    assert _xb(M=200) == _xb(M=256) != _xb(M=257)


def test_lowrank_pieces_validation():
    lib = _lib()
    assert lib.svdq_lowrank_down(_d(rank=0), 256, A, A, A, A, None) == SHAPE
    assert lib.svdq_lowrank_up(_d(rank=0), 256, A, A, A, None) == SHAPE
    assert lib.svdq_lowrank_down(_d(), 256, A, A, None, A, None) == ARG
    assert lib.svdq_lowrank_up(_d(), 256, A, MIS, A, None) == ARG


def test_calibrate_validation():
    lib = _lib()
    assert lib.svdq_calibrate_absmax(16, 512, None, A, 0, None) == ARG
    assert lib.svdq_calibrate_absmax(16, 512, A, MIS, 0, None) == ARG
    assert lib.svdq_calibrate_absmax(16, 512, A, A, 2, None) == ARG
    assert lib.svdq_calibrate_absmax(0, 512, A, A, 0, None) == SHAPE
    assert lib.svdq_calibrate_absmax(16, 500, A, A, 1, None) == SHAPE
    assert lib.svdq_lambda_from_absmax(512, A, None, A, None) == ARG
    assert lib.svdq_lambda_from_absmax(500, A, A, A, None) == SHAPE
    assert lib.svdq_calibrate_lambda(16, 512, 16, None, A, A, None) == ARG
    assert lib.svdq_calibrate_lambda(16, 500, 16, A, A, A, None) == SHAPE
    assert lib.svdq_calibrate_lambda(16, 512, 0, A, A, A, None) == SHAPE


def test_awq_validation():
    lib = _lib()
    p = lib.svdq_awq_pack_weight
    assert p(64, 3072, None, A, A, A, None) == ARG
    assert p(64, 3072, A, MIS, A, A, None) == ARG
    assert p(64, 3072, A, A, None, A, None) == ARG
    assert p(64, 3072, A, A, A, MIS, None) == ARG
    assert p(0, 3072, A, A, A, A, None) == SHAPE
    assert p(64, 3000, A, A, A, A, None) == SHAPE      # K % 128
    assert p(64, 64, A, A, A, A, None) == SHAPE
    assert p((1 << 24) + 1, 128, A, A, A, A, None) == SHAPE
    assert p(1 << 24, 8192, A, A, A, A, None) == SHAPE          # N*K > 2^36
    f = lib.svdq_awq_linear
    assert f(1, 64, 3072, A, A, A, A, None, 2, A, None) == ARG    # unknown flag
    assert f(1, 64, 3072, None, A, A, A, None, 0, A, None) == ARG
    assert f(1, 64, 3072, A, A, A, A, MIS, 0, A, None) == ARG     # bias misaligned
    assert f(1, 64, 3072, A, A, A, A, None, 0, None, None) == ARG
    assert f(0, 64, 3072, A, A, A, A, None, 0, A, None) == SHAPE
    assert f(65, 64, 3072, A, A, A, A, None, 0, A, None) == SHAPE
    assert f(1, 0, 3072, A, A, A, A, None, 0, A, None) == SHAPE
    assert f(1, 64, 3008, A, A, A, A, None, 0, A, None) == SHAPE


def test_lowrank_factors_validation():
    lib = _lib()
    n = ctypes.c_size_t(0)
    ws = lib.svdq_lowrank_factors_workspace
    assert ws(3072, 1024, 32, ctypes.byref(n)) == 0
    need = n.value
    # transposed weight + sketch buffers dominate: at least N*K*2 + (N + K)*l*8
    assert need >= 3072 * 1024 * 2 + (3072 + 1024) * 48 * 8
    assert ws(3072, 1024, 32, None) == ARG
    for N, K, r in [(3000, 1024, 32), (3072, 64, 32), (3072, 1024, 0), (3072, 1024, 144),
                    (3072, 1024, 40), (1 << 21, 128, 16), (1 << 17, 1 << 16, 16)]:
        assert ws(N, K, r, ctypes.byref(n)) == SHAPE, (N, K, r)
    # workspace grows with the rank
    assert ws(3072, 1024, 128, ctypes.byref(n)) == 0 and n.value > need
    f = lib.svdq_lowrank_factors
    ok = (3072, 1024, 32, A, A, 7, 2, A, A, None, A, need, None)

    def call(**kw):
        names = ["N", "K", "r", "W", "lam", "seed", "q", "ld", "lu", "sig", "ws", "wsb", "st"]
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[k] for k in names])

    assert call(W=None) == ARG
    assert call(lam=MIS) == ARG
    assert call(ld=None) == ARG
    assert call(lu=MIS) == ARG
    assert call(sig=MIS) == ARG
    assert call(ws=None) == ARG
    assert call(ws=A + 16) == ARG                 # workspace must be 256-byte aligned
    assert call(wsb=need - 1) == ARG
    assert call(q=-1) == SHAPE
    assert call(q=9) == SHAPE
    assert call(r=48) == ARG                      # rank 48 needs a larger workspace
    assert call(N=3000) == SHAPE


def test_lowrank_factors_noalloc_validation():
    """The no-allocation SVD refuses, on the host, shapes whose workspace
    exceeds its 64 MiB static array, and bad pointers, like the workspace
    entry point."""
    f = _lib().svdq_lowrank_factors_noalloc
    assert f(9216, 3072, 32, A, A, 1, 2, A, A, None, None) == SHAPE     # 118 MiB of workspace
    assert f(3072, 12288, 32, A, A, 1, 2, A, A, None, None) == SHAPE
    assert f(500, 512, 16, A, A, 1, 2, A, A, None, None) == SHAPE       # N not a multiple of 128
    assert f(512, 512, 8, A, A, 1, 2, A, A, None, None) == SHAPE        # rank below 16
    assert f(512, 512, 16, A, A, 1, 9, A, A, None, None) == SHAPE       # power iterations
    assert f(512, 512, 16, None, A, 1, 2, A, A, None, None) == ARG
    assert f(512, 512, 16, A, A, 1, 2, MIS, A, None, None) == ARG
    assert f(512, 512, 16, A, A, 1, 2, A, None, None, None) == ARG
    assert f(512, 512, 16, A, A, 1, 2, A, A, MIS, None) == ARG


def test_gelu_quantize_validation():
    """The fused MLP-up entry point refuses, on the host, descriptors that do
    not form an INT4 up layer feeding an INT4 GELU-input down layer, and
    images, workspaces and pointers of the wrong size or alignment."""
    lib = _lib()
    f = lib.svdq_linear_forward_gelu_quantize
    up = dict(mode=0, K=512, N=384, rank=16)
    dn = dict(mode=0, K=384, N=256, rank=32, flags=2)
    nx, nw, nd = _xb(M=300, **up), _wb(**up), _xb(M=300, **dn)
    n = ctypes.c_size_t(0)
    assert lib.svdq_gelu_quantize_workspace_size(_d(**up), 300, _d(**dn), ctypes.byref(n)) == 0
    ws = n.value
    assert ws == 384 // 128 * 512 * 32 * 4

    def call(u=up, d=dn, M=300, xi=A, nx_=nx, wi=A, nw_=nw, lam=A, ld=A, di=A, nd_=nd, Y=None,
             T=None, w=A, nws=ws):
        return f(_d(**u), M, xi, nx_, wi, nw_, _d(**d), lam, ld, di, nd_, Y, T, w, nws, None)

    assert call(d=dict(dn, flags=0)) == ARG                 # down layer without the GELU flag
    assert call(u=dict(up, mode=1)) == ARG                  # FP4 up layer
    assert call(d=dict(dn, mode=1)) == ARG                  # FP4 down layer
    assert call(u=dict(up, flags=1)) == ARG                 # fp32 up output
    assert call(d=dict(dn, K=512)) == SHAPE                 # down K != up N
    assert call(d=dict(dn, rank=144)) == SHAPE              # down rank above 128
    assert call(nx_=nx - 16) == ARG                         # up images
    assert call(nw_=nw + 16) == ARG
    assert call(nd_=nd - 16) == ARG                         # down image
    assert call(nd_=_xb(M=300, **dict(dn, rank=16))) == ARG
    assert call(nws=ws - 4) == ARG                          # workspace too small
    assert call(w=None) == ARG
    assert call(ld=None) == ARG                             # down rank > 0 needs lora_down
    assert call(lam=None) == ARG
    assert call(di=MIS) == ARG
    assert call(Y=MIS) == ARG
    assert call(M=0) == SHAPE
    d0 = dict(dn, rank=0)
    assert f(_d(**up), 300, A, nx, A, nw, _d(**d0), A, A, A, _xb(M=300, **d0), None, None, None, 0,
             None) == ARG                                   # lora_down with rank 0


def test_qk_norm_rope_validation():
    f = _lib().svdq_qk_norm_rope
    ok = dict(M=64, H=24, ld=9216, Y=A, qs=A, ks=A, c=A, s=A, eps=1e-6)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["M"], a["H"], a["ld"], a["Y"], a["qs"], a["ks"], a["c"], a["s"], a["eps"], None)

    assert call(Y=None) == ARG
    assert call(Y=MIS) == ARG
    assert call(qs=None) == ARG
    assert call(ks=MIS) == ARG
    assert call(c=None) == ARG
    assert call(s=MIS) == ARG
    assert call(eps=0.0) == ARG
    assert call(eps=-1.0) == ARG
    assert call(eps=float("nan")) == ARG
    assert call(eps=float("inf")) == ARG
    assert call(M=0) == SHAPE
    assert call(H=0) == SHAPE
    assert call(H=2049) == SHAPE
    assert call(ld=6143) == SHAPE            # shorter than Q and K
    assert call(ld=9220) == SHAPE            # rows not 16-byte aligned
    g = _lib().svdq_linear_forward_qk
    d = _d(mode=1, K=512, N=9216, rank=32)
    nx, nw = _xb(M=64, mode=1, rank=32), _wb(mode=1, N=9216, rank=32)
    assert g(d, 64, A, nx, A, nw, 24, A, A, A, A, 1e-6, None, None) == ARG    # Y null
    assert g(d, 64, None, nx, A, nw, 24, A, A, A, A, 1e-6, A, None) == ARG
    assert g(_d(mode=1, K=512, N=9216, rank=32, flags=1), 64, A, nx, A, nw, 24, A, A, A, A, 1e-6,
             A, None) == ARG                                                   # fp32 output
    assert g(d, 64, A, nx, A, nw, 37, A, A, A, A, 1e-6, A, None) == SHAPE     # 2 H 128 > N
    assert g(d, 64, A, nx, A, nw, 24, A, A, A, A, 0.0, A, None) == ARG
    assert g(_d(mode=1, K=500, N=9216), 64, A, nx, A, nw, 24, A, A, A, A, 1e-6, A,
             None) == SHAPE


def _has_gpu():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_has_gpu(), reason="only meaningful without a GPU: with one these "
                    "valid-looking fake pointers would be launched on")
def test_no_device_is_a_hip_error():
    lib = _lib()
    assert lib.svdq_quantize_act(_d(), 256, A, A, A, A, A, A, A, _xb(), None) == HIP
    assert lib.svdq_linear_forward(_d(), 256, A, _xb(), A, _wb(), A, None) == HIP
    assert lib.svdq_linear_forward(_d(mode=1), 256, A, _xb(mode=1), A, _wb(mode=1), A,
                                   None) == HIP
    assert lib.svdq_prepare_weight(_d(), A, A, A, None, A, _wb(), None) == HIP
    assert lib.svdq_linear_forward_packed(_d(), 256, A, _xb(), A, A, A, None, A, _wb(), A,
                                          None) == HIP
    assert lib.svdq_linear_forward_rowmajor(_d(), 256, A, A, A, A, A, A, None, A, A, _rb(),
                                            None) == HIP
    assert lib.svdq_awq_pack_weight(64, 3072, A, A, A, A, None) == HIP
    assert lib.svdq_awq_linear(1, 64, 3072, A, A, A, A, None, 0, A, None) == HIP
    n = ctypes.c_size_t(0)
    assert lib.svdq_lowrank_factors_workspace(512, 512, 16, ctypes.byref(n)) == 0
    assert lib.svdq_lowrank_factors(512, 512, 16, A, A, 1, 2, A, A, None, A, n.value, None) == HIP
    assert lib.svdq_lowrank_factors_noalloc(512, 512, 16, A, A, 1, 2, A, A, None, None) == HIP
    assert lib.svdq_qk_norm_rope(64, 24, 9216, A, A, A, A, A, 1e-6, None) == HIP
    assert lib.svdq_linear_forward_qk(_d(mode=1, N=9216), 256, A, _xb(mode=1), A,
                                      _wb(mode=1, N=9216), 24, A, A, A, A, 1e-6, A, None) == HIP


def test_nvfp4_validation():
    lib = _lib()
    sfa = lib.svdq_nvfp4_scale_from_absmax
    assert sfa(4, None, A, None) == ARG
    assert sfa(4, A, MIS, None) == ARG
    assert sfa(0, A, A, None) == SHAPE
    qa = lib.svdq_nvfp4_quantize_act
    assert qa(64, 512, 0, None, A, A, None, A, A, None, None) == ARG
    assert qa(64, 512, 0, A, A, A, None, A, MIS, None, None) == ARG
    assert qa(64, 512, 16, A, A, A, None, A, A, A, None) == ARG     # rank > 0 needs lora_down and T
    assert qa(64, 512, 16, A, A, A, A, A, A, MIS, None) == ARG
    assert qa(64, 512, 0, A, A, A, A, A, A, None, None) == ARG      # rank 0 takes neither
    for M, K, r in [(0, 512, 0), (64, 96, 0), (64, 0, 0), (64, 1 << 21, 0), (64, 512, 24),
                    (64, 512, 272)]:
        ld, T = (A, A) if r else (None, None)
        assert qa(M, K, r, A, A, A, ld, A, A, T, None) == SHAPE, (M, K, r)
    pw = lib.svdq_nvfp4_pack_weight
    assert pw(256, 512, 16, A, A, None, A, A, A, A, None) == ARG       # rank > 0 needs both factors
    assert pw(256, 512, 0, A, A, A, None, A, A, A, None) == ARG        # rank 0 takes none
    assert pw(256, 512, 16, A, A, A, A, A, A, None, None) == ARG       # g null
    for N, K, r in [(200, 512, 16), (256, 200, 16), (256, 512, 24), (256, 512, 272)]:
        assert pw(N, K, r, A, A, A, A, A, A, A, None) == SHAPE, (N, K, r)
    assert pw(256, 512, -16, A, A, None, None, A, A, A, None) == SHAPE
    lin = lib.svdq_nvfp4_linear
    ok = dict(M=64, N=256, K=512, r=16, xc=A, xs=A, gx=A, wc=A, ws=A, gw=A, T=A, lu=A, b=None,
              fl=0, Y=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lin(a["M"], a["N"], a["K"], a["r"], a["xc"], a["xs"], a["gx"], a["wc"], a["ws"],
                   a["gw"], a["T"], a["lu"], a["b"], a["fl"], a["Y"], None)

    assert call(fl=2) == ARG                 # only the fp32-output flag is defined
    assert call(xc=None) == ARG
    assert call(ws=MIS) == ARG
    assert call(gw=None) == ARG
    assert call(Y=None) == ARG
    assert call(b=MIS) == ARG
    assert call(T=None) == ARG               # rank 16 needs T and lora_up
    assert call(r=0) == ARG                  # rank 0 takes neither
    assert call(r=0, T=None, lu=None, M=0) == SHAPE
    assert call(N=200) == SHAPE
    assert call(K=96) == SHAPE
    assert call(r=24) == SHAPE
