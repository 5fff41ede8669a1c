"""Python binding of libsvdq (ctypes).  Argument marshalling only.

Each function takes torch tensors on the current HIP device, checks dtype,
shape, device and contiguity, allocates missing outputs with ``torch.empty``
(PyTorch is used for device memory and the current stream, nothing else) and
calls the C function of the same name on
``torch.cuda.current_stream()``.  Every step of the layer runs in the
library's kernels; if ``libsvdq.so`` is missing the import-time loader raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "svdq.h")

SVDQ_MODE_INT4 = 0
SVDQ_MODE_FP4 = 1
SVDQ_FLAG_OUT_F32 = 0x1
SVDQ_FLAG_GELU_IN = 0x2
MODES = {"int4": SVDQ_MODE_INT4, "fp4": SVDQ_MODE_FP4}
STATUS = {0: "SVDQ_OK", 1: "SVDQ_ERR_ARG", 2: "SVDQ_ERR_SHAPE", 3: "SVDQ_ERR_ARCH",
          4: "SVDQ_ERR_HIP"}


class SvdqDesc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class SvdqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}")
        self.status = status


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_DESC = ctypes.POINTER(SvdqDesc)

_SIGNATURES = {
    "svdq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "svdq_arch_supported": (ctypes.c_int, [ctypes.c_char_p]),
    "svdq_version": (ctypes.c_char_p, []),
    "svdq_calibrate_lambda": (ctypes.c_int, [_i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "svdq_calibrate_absmax": (ctypes.c_int, [_i64, _i32, _vp, _vp, _i32, _vp]),
    "svdq_lambda_from_absmax": (ctypes.c_int, [_i32, _vp, _vp, _vp, _vp]),
    "svdq_pack_weight": (ctypes.c_int, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "svdq_act_image_size": (ctypes.c_int, [_DESC, _i64, ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_weight_image_size": (ctypes.c_int, [_DESC, ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_quantize_act": (ctypes.c_int, [_DESC, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                         _vp]),
    "svdq_prepare_weight": (ctypes.c_int, [_DESC, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "svdq_linear_forward": (ctypes.c_int, [_DESC, _i64, _vp, _sz, _vp, _sz, _vp, _vp]),
    "svdq_linear_forward_packed": (ctypes.c_int, [_DESC, _i64, _vp, _sz, _vp, _vp, _vp, _vp, _vp,
                                                  _sz, _vp, _vp]),
    "svdq_linear_rowmajor_workspace_size": (ctypes.c_int, [_DESC, _i64,
                                                           ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_linear_forward_rowmajor": (ctypes.c_int, [_DESC, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _vp, _vp, _vp, _sz, _vp]),
    "svdq_gelu_quantize_workspace_size": (ctypes.c_int, [_DESC, _i64, _DESC,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_linear_forward_gelu_quantize": (ctypes.c_int, [_DESC, _i64, _vp, _sz, _vp, _sz, _DESC, _vp,
                                                         _vp, _vp, _sz, _vp, _vp, _vp, _sz, _vp]),
    "svdq_lowrank_down": (ctypes.c_int, [_DESC, _i64, _vp, _vp, _vp, _vp, _vp]),
    "svdq_lowrank_up": (ctypes.c_int, [_DESC, _i64, _vp, _vp, _vp, _vp]),
    "svdq_awq_pack_weight": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "svdq_awq_linear": (ctypes.c_int, [_i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, ctypes.c_uint32,
                                       _vp, _vp]),
    "svdq_qk_norm_rope": (ctypes.c_int, [_i64, _i32, _i64, _vp, _vp, _vp, _vp, _vp,
                                         ctypes.c_float, _vp]),
    "svdq_linear_forward_qk": (ctypes.c_int, [_DESC, _i64, _vp, _sz, _vp, _sz, _i32, _vp, _vp,
                                              _vp, _vp, ctypes.c_float, _vp, _vp]),
    "svdq_nvfp4_scale_from_absmax": (ctypes.c_int, [_i32, _vp, _vp, _vp]),
    "svdq_nvfp4_quantize_act": (ctypes.c_int, [_i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp]),
    "svdq_nvfp4_pack_weight": (ctypes.c_int, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp]),
    "svdq_nvfp4_linear": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, ctypes.c_uint32, _vp, _vp]),
    "svdq_lowrank_factors_workspace": (ctypes.c_int, [_i32, _i32, _i32,
                                                      ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_lowrank_factors": (ctypes.c_int, [_i32, _i32, _i32, _vp, _vp, ctypes.c_uint64, _i32, _vp,
                                            _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "svdq_lowrank_factors_noalloc": (ctypes.c_int, [_i32, _i32, _i32, _vp, _vp, ctypes.c_uint64, _i32,
                                                    _vp, _vp, _vp, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libsvdq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def header_symbols() -> list:
    """Names of the functions include/svdq.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", text)))


def desc(mode, K: int, N: int, rank: int, out_f32: bool = False, gelu_in: bool = False) -> SvdqDesc:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    flags = (SVDQ_FLAG_OUT_F32 if out_f32 else 0) | (SVDQ_FLAG_GELU_IN if gelu_in else 0)
    return SvdqDesc(m, K, N, rank, flags)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t: Optional[torch.Tensor]) -> int:
    """Byte count of a buffer passed to the library (0 for none)."""
    return 0 if t is None else t.numel() * t.element_size()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, dtype, shape=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check(fn: str, st: int):
    if st != 0:
        raise SvdqError(fn, st)


def scale_dtype(mode) -> torch.dtype:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return torch.float32 if m == SVDQ_MODE_INT4 else torch.uint8


def scale_cols(mode, K: int) -> int:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return K // 64 if m == SVDQ_MODE_INT4 else K // 32


def svdq_status_string(status: int) -> str:
    return load().svdq_status_string(status).decode()


def svdq_arch_supported(name: str) -> bool:
    return bool(load().svdq_arch_supported(name.encode()))


def svdq_version() -> str:
    return load().svdq_version().decode()


def svdq_calibrate_lambda(X: torch.Tensor, W: torch.Tensor, lam: Optional[torch.Tensor] = None):
    M, K = X.shape
    N = W.shape[0]
    _need(X, "X", torch.bfloat16, (M, K))
    _need(W, "W", torch.bfloat16, (N, K))
    if lam is None:
        lam = torch.empty(K, dtype=torch.float32, device=X.device)
    _need(lam, "lambda", torch.float32, (K,))
    _check("svdq_calibrate_lambda",
           load().svdq_calibrate_lambda(M, K, N, _p(X), _p(W), _p(lam), _stream()))
    return lam


def svdq_calibrate_absmax(A, amax=None, accumulate: bool = False):
    """Per-column absolute maximum of a bf16 matrix, combined with amax when
    accumulate (the running statistic over calibration batches)."""
    R, K = A.shape
    _need(A, "A", torch.bfloat16, (R, K))
    if amax is None:
        if accumulate:
            raise ValueError("accumulate needs amax")
        amax = torch.empty(K, dtype=torch.float32, device=A.device)
    _need(amax, "amax", torch.float32, (K,))
    _check("svdq_calibrate_absmax",
           load().svdq_calibrate_absmax(R, K, _p(A), _p(amax), 1 if accumulate else 0, _stream()))
    return amax


def svdq_lambda_from_absmax(xmax, wmax, lam=None):
    K = xmax.shape[0]
    _need(xmax, "xmax", torch.float32, (K,))
    _need(wmax, "wmax", torch.float32, (K,))
    if lam is None:
        lam = torch.empty(K, dtype=torch.float32, device=xmax.device)
    _need(lam, "lambda", torch.float32, (K,))
    _check("svdq_lambda_from_absmax",
           load().svdq_lambda_from_absmax(K, _p(xmax), _p(wmax), _p(lam), _stream()))
    return lam


def svdq_pack_weight(d: SvdqDesc, W, lam, lora_down=None, lora_up=None, wcodes=None, wscales=None):
    N, K, r = d.N, d.K, d.rank
    _need(W, "W", torch.bfloat16, (N, K))
    _need(lam, "lambda", torch.float32, (K,))
    _need(lora_down, "lora_down", torch.bfloat16, (r, K), optional=True)
    _need(lora_up, "lora_up", torch.bfloat16, (N, r), optional=True)
    if wcodes is None:
        wcodes = torch.empty(N, K // 2, dtype=torch.uint8, device=W.device)
    if wscales is None:
        wscales = torch.empty(N, scale_cols(d.mode, K), dtype=scale_dtype(d.mode), device=W.device)
    _need(wcodes, "wcodes", torch.uint8, (N, K // 2))
    _need(wscales, "wscales", scale_dtype(d.mode), (N, scale_cols(d.mode, K)))
    _check("svdq_pack_weight",
           load().svdq_pack_weight(ctypes.byref(d), _p(W), _p(lam), _p(lora_down), _p(lora_up),
                                   _p(wcodes), _p(wscales), _stream()))
    return wcodes, wscales


def svdq_act_image_size(d: SvdqDesc, M: int) -> int:
    n = ctypes.c_size_t(0)
    _check("svdq_act_image_size",
           load().svdq_act_image_size(ctypes.byref(d), M, ctypes.byref(n)))
    return n.value


def svdq_weight_image_size(d: SvdqDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("svdq_weight_image_size", load().svdq_weight_image_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def svdq_quantize_act(d: SvdqDesc, X, lam, lora_down=None, xcodes=None, xscales=None, T=None,
                      ximage=None, image=True, codes=False):
    """Quantize X; returns (xcodes, xscales, T, ximage), each None when not written.

    ``image`` asks for the activation image (allocated when ``ximage`` is
    None), ``codes`` for the row-major codes and scales (allocated when
    missing); buffers passed in are always written.  T is written when it is
    passed in (it needs lora_down)."""
    M = X.shape[0]
    K, r = d.K, d.rank
    _need(X, "X", torch.bfloat16, (M, K))
    _need(lam, "lambda", torch.float32, (K,))
    _need(lora_down, "lora_down", torch.bfloat16, (r, K), optional=True)
    if codes and xcodes is None:
        xcodes = torch.empty(M, K // 2, dtype=torch.uint8, device=X.device)
    if codes and xscales is None:
        xscales = torch.empty(M, scale_cols(d.mode, K), dtype=scale_dtype(d.mode), device=X.device)
    if image and ximage is None:
        ximage = torch.empty(svdq_act_image_size(d, M), dtype=torch.uint8, device=X.device)
    _need(xcodes, "xcodes", torch.uint8, (M, K // 2), optional=True)
    _need(xscales, "xscales", scale_dtype(d.mode), (M, scale_cols(d.mode, K)), optional=True)
    _need(T, "T", torch.float32, (M, r), optional=True)
    _need(ximage, "ximage", torch.uint8, optional=True)
    _check("svdq_quantize_act",
           load().svdq_quantize_act(ctypes.byref(d), M, _p(X), _p(lam), _p(lora_down),
                                    _p(xcodes), _p(xscales), _p(T), _p(ximage), _nbytes(ximage),
                                    _stream()))
    return xcodes, xscales, T, ximage


def svdq_prepare_weight(d: SvdqDesc, wcodes, wscales, lora_up=None, bias=None, wimage=None):
    """Prepared weight (opaque uint8 image) of packed codes and scales, L2 and the bias."""
    N, K, r = d.N, d.K, d.rank
    _need(wcodes, "wcodes", torch.uint8, (N, K // 2))
    _need(wscales, "wscales", scale_dtype(d.mode), (N, scale_cols(d.mode, K)))
    _need(lora_up, "lora_up", torch.bfloat16, (N, r), optional=True)
    _need(bias, "bias", torch.bfloat16, (N,), optional=True)
    if wimage is None:
        wimage = torch.empty(svdq_weight_image_size(d), dtype=torch.uint8, device=wcodes.device)
    _need(wimage, "wimage", torch.uint8)
    _check("svdq_prepare_weight",
           load().svdq_prepare_weight(ctypes.byref(d), _p(wcodes), _p(wscales), _p(lora_up),
                                      _p(bias), _p(wimage), _nbytes(wimage), _stream()))
    return wimage


def svdq_linear_forward(d: SvdqDesc, M: int, ximage, wimage, Y=None):
    out_dtype = torch.float32 if (d.flags & SVDQ_FLAG_OUT_F32) else torch.bfloat16
    _need(ximage, "ximage", torch.uint8)
    _need(wimage, "wimage", torch.uint8)
    if Y is None:
        Y = torch.empty(M, d.N, dtype=out_dtype, device=ximage.device)
    _need(Y, "Y", out_dtype, (M, d.N))
    _check("svdq_linear_forward",
           load().svdq_linear_forward(ctypes.byref(d), M, _p(ximage), _nbytes(ximage), _p(wimage),
                                      _nbytes(wimage), _p(Y), _stream()))
    return Y


def svdq_linear_forward_packed(d: SvdqDesc, M: int, ximage, wcodes, wscales, lora_up=None,
                               bias=None, wscratch=None, Y=None):
    """The layer from the packed 4-bit weight (codes, scales), L2 and the bias:
    the prepared weight is written into wscratch (allocated when None) and the
    GEMM runs on it; returns Y."""
    N, K, r = d.N, d.K, d.rank
    out_dtype = torch.float32 if (d.flags & SVDQ_FLAG_OUT_F32) else torch.bfloat16
    _need(ximage, "ximage", torch.uint8)
    _need(wcodes, "wcodes", torch.uint8, (N, K // 2))
    _need(wscales, "wscales", scale_dtype(d.mode), (N, scale_cols(d.mode, K)))
    _need(lora_up, "lora_up", torch.bfloat16, (N, r), optional=True)
    _need(bias, "bias", torch.bfloat16, (N,), optional=True)
    if wscratch is None:
        wscratch = torch.empty(svdq_weight_image_size(d), dtype=torch.uint8, device=wcodes.device)
    _need(wscratch, "wscratch", torch.uint8)
    if Y is None:
        Y = torch.empty(M, N, dtype=out_dtype, device=ximage.device)
    _need(Y, "Y", out_dtype, (M, N))
    _check("svdq_linear_forward_packed",
           load().svdq_linear_forward_packed(ctypes.byref(d), M, _p(ximage), _nbytes(ximage), _p(wcodes),
                                             _p(wscales), _p(lora_up), _p(bias), _p(wscratch),
                                             _nbytes(wscratch), _p(Y), _stream()))
    return Y


def svdq_gelu_quantize_workspace_size(up: SvdqDesc, M: int, down: SvdqDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("svdq_gelu_quantize_workspace_size",
           load().svdq_gelu_quantize_workspace_size(ctypes.byref(up), M, ctypes.byref(down),
                                                    ctypes.byref(n)))
    return n.value


def svdq_linear_rowmajor_workspace_size(d: SvdqDesc, M: int) -> int:
    n = ctypes.c_size_t(0)
    _check("svdq_linear_rowmajor_workspace_size",
           load().svdq_linear_rowmajor_workspace_size(ctypes.byref(d), M, ctypes.byref(n)))
    return n.value


def svdq_linear_forward_rowmajor(d: SvdqDesc, xcodes, xscales, T, wcodes, wscales, lora_up=None,
                                 bias=None, workspace=None, Y=None):
    """The layer from the row-major codes, scales and T of both sides (the
    images are written into workspace, allocated when None); returns Y."""
    M = xcodes.shape[0]
    N, K, r = d.N, d.K, d.rank
    out_dtype = torch.float32 if (d.flags & SVDQ_FLAG_OUT_F32) else torch.bfloat16
    _need(xcodes, "xcodes", torch.uint8, (M, K // 2))
    _need(xscales, "xscales", scale_dtype(d.mode), (M, scale_cols(d.mode, K)))
    _need(T, "T", torch.float32, (M, r), optional=r == 0)
    _need(wcodes, "wcodes", torch.uint8, (N, K // 2))
    _need(wscales, "wscales", scale_dtype(d.mode), (N, scale_cols(d.mode, K)))
    _need(lora_up, "lora_up", torch.bfloat16, (N, r), optional=r == 0)
    _need(bias, "bias", torch.bfloat16, (N,), optional=True)
    if workspace is None:
        workspace = torch.empty(svdq_linear_rowmajor_workspace_size(d, M), dtype=torch.uint8,
                                device=xcodes.device)
    _need(workspace, "workspace", torch.uint8)
    if Y is None:
        Y = torch.empty(M, N, dtype=out_dtype, device=xcodes.device)
    _need(Y, "Y", out_dtype, (M, N))
    _check("svdq_linear_forward_rowmajor",
           load().svdq_linear_forward_rowmajor(ctypes.byref(d), M, _p(xcodes), _p(xscales), _p(T),
                                               _p(wcodes), _p(wscales), _p(lora_up), _p(bias), _p(Y),
                                               _p(workspace), _nbytes(workspace), _stream()))
    return Y


def svdq_linear_forward_gelu_quantize(up: SvdqDesc, M: int, ximage, wimage, down: SvdqDesc,
                                      lam_down, lora_down=None, ximage_down=None, Y=None, T=None,
                                      workspace=None):
    """The up layer's GEMM whose epilogue applies GELU and writes the down
    layer's activation image (returns it; Y and T are written when given)."""
    _need(ximage, "ximage", torch.uint8)
    _need(wimage, "wimage", torch.uint8)
    _need(lam_down, "lambda_down", torch.float32, (up.N,))
    _need(lora_down, "lora_down", torch.bfloat16, (down.rank, up.N), optional=True)
    if ximage_down is None:
        ximage_down = torch.empty(svdq_act_image_size(down, M), dtype=torch.uint8,
                                  device=ximage.device)
    _need(ximage_down, "ximage_down", torch.uint8)
    _need(Y, "Y", torch.bfloat16, (M, up.N), optional=True)
    _need(T, "T", torch.float32, (M, down.rank), optional=True)
    nws = svdq_gelu_quantize_workspace_size(up, M, down)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=ximage.device)
    _need(workspace, "workspace", torch.uint8, optional=True)
    _check("svdq_linear_forward_gelu_quantize",
           load().svdq_linear_forward_gelu_quantize(
               ctypes.byref(up), M, _p(ximage), _nbytes(ximage), _p(wimage), _nbytes(wimage),
               ctypes.byref(down), _p(lam_down), _p(lora_down), _p(ximage_down),
               _nbytes(ximage_down), _p(Y), _p(T), _p(workspace), _nbytes(workspace), _stream()))
    return ximage_down


def svdq_lowrank_down(d: SvdqDesc, X, lam, lora_down, T=None):
    M = X.shape[0]
    _need(X, "X", torch.bfloat16, (M, d.K))
    _need(lam, "lambda", torch.float32, (d.K,))
    _need(lora_down, "lora_down", torch.bfloat16, (d.rank, d.K))
    if T is None:
        T = torch.empty(M, d.rank, dtype=torch.float32, device=X.device)
    _need(T, "T", torch.float32, (M, d.rank))
    _check("svdq_lowrank_down",
           load().svdq_lowrank_down(ctypes.byref(d), M, _p(X), _p(lam), _p(lora_down), _p(T),
                                    _stream()))
    return T


def svdq_lowrank_up(d: SvdqDesc, T, lora_up, Y):
    M = T.shape[0]
    out_dtype = torch.float32 if (d.flags & SVDQ_FLAG_OUT_F32) else torch.bfloat16
    _need(T, "T", torch.float32, (M, d.rank))
    _need(lora_up, "lora_up", torch.bfloat16, (d.N, d.rank))
    _need(Y, "Y", out_dtype, (M, d.N))
    _check("svdq_lowrank_up",
           load().svdq_lowrank_up(ctypes.byref(d), M, _p(T), _p(lora_up), _p(Y), _stream()))
    return Y


AWQ_GROUP = 64


def svdq_awq_pack_weight(W, codes=None, scales=None, zeros=None):
    """AWQ W4A16 packing of a bf16 weight [N][K]; returns (codes, scales, zeros)."""
    N, K = W.shape
    G = K // AWQ_GROUP
    _need(W, "W", torch.bfloat16, (N, K))
    if codes is None:
        codes = torch.empty(N, K // 2, dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty(N, G, dtype=torch.float32, device=W.device)
    if zeros is None:
        zeros = torch.empty(N, G, dtype=torch.uint8, device=W.device)
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", torch.float32, (N, G))
    _need(zeros, "zeros", torch.uint8, (N, G))
    _check("svdq_awq_pack_weight",
           load().svdq_awq_pack_weight(N, K, _p(W), _p(codes), _p(scales), _p(zeros), _stream()))
    return codes, scales, zeros


def svdq_awq_linear(X, codes, scales, zeros, bias=None, Y=None, out_f32: bool = False):
    """Y = X deq(W)^T + bias for the AWQ W4A16 layer (small M)."""
    M, K = X.shape
    N = codes.shape[0]
    G = K // AWQ_GROUP
    out_dtype = torch.float32 if out_f32 else torch.bfloat16
    _need(X, "X", torch.bfloat16, (M, K))
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", torch.float32, (N, G))
    _need(zeros, "zeros", torch.uint8, (N, G))
    _need(bias, "bias", torch.bfloat16, (N,), optional=True)
    if Y is None:
        Y = torch.empty(M, N, dtype=out_dtype, device=X.device)
    _need(Y, "Y", out_dtype, (M, N))
    _check("svdq_awq_linear",
           load().svdq_awq_linear(M, N, K, _p(X), _p(codes), _p(scales), _p(zeros), _p(bias),
                                  SVDQ_FLAG_OUT_F32 if out_f32 else 0, _p(Y), _stream()))
    return Y


def svdq_lowrank_factors_workspace(N: int, K: int, rank: int) -> int:
    """Bytes of device workspace svdq_lowrank_factors needs for this shape."""
    n = ctypes.c_size_t(0)
    _check("svdq_lowrank_factors_workspace",
           load().svdq_lowrank_factors_workspace(N, K, rank, ctypes.byref(n)))
    return n.value


def svdq_lowrank_factors(W, lam, rank: int, seed: int, power_iters: int = 2, lora_down=None,
                         lora_up=None, sigma=None, workspace=None, want_sigma: bool = True):
    """Rank-r factors of W diag(lambda) by the library's randomized SVD; returns
    (lora_down bf16 [r][K], lora_up bf16 [N][r], sigma fp64 [r] or None)."""
    N, K = W.shape
    _need(W, "W", torch.bfloat16, (N, K))
    _need(lam, "lambda", torch.float32, (K,))
    if lora_down is None:
        lora_down = torch.empty(rank, K, dtype=torch.bfloat16, device=W.device)
    if lora_up is None:
        lora_up = torch.empty(N, rank, dtype=torch.bfloat16, device=W.device)
    if sigma is None and want_sigma:
        sigma = torch.empty(rank, dtype=torch.float64, device=W.device)
    _need(lora_down, "lora_down", torch.bfloat16, (rank, K))
    _need(lora_up, "lora_up", torch.bfloat16, (N, rank))
    _need(sigma, "sigma", torch.float64, (rank,), optional=True)
    need = svdq_lowrank_factors_workspace(N, K, rank)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=W.device)
    _need(workspace, "workspace", torch.uint8)
    _check("svdq_lowrank_factors",
           load().svdq_lowrank_factors(N, K, rank, _p(W), _p(lam), ctypes.c_uint64(seed),
                                       power_iters, _p(lora_down), _p(lora_up), _p(sigma),
                                       _p(workspace), workspace.numel(), _stream()))
    return lora_down, lora_up, sigma


def svdq_lowrank_factors_noalloc(W, lam, rank: int, seed: int, power_iters: int, lora_down,
                                 lora_up, sigma=None):
    """svdq_lowrank_factors with the library's static workspace: the outputs
    are the caller's (lora_down bf16 [r][K], lora_up bf16 [N][r], sigma fp64
    [r] or None); the library allocates nothing."""
    N, K = W.shape
    _need(W, "W", torch.bfloat16, (N, K))
    _need(lam, "lambda", torch.float32, (K,))
    _need(lora_down, "lora_down", torch.bfloat16, (rank, K))
    _need(lora_up, "lora_up", torch.bfloat16, (N, rank))
    _need(sigma, "sigma", torch.float64, (rank,), optional=True)
    _check("svdq_lowrank_factors_noalloc",
           load().svdq_lowrank_factors_noalloc(N, K, rank, _p(W), _p(lam), ctypes.c_uint64(seed),
                                               power_iters, _p(lora_down), _p(lora_up), _p(sigma),
                                               _stream()))
    return lora_down, lora_up, sigma


HEAD_DIM = 128


def svdq_qk_norm_rope(Y, heads: int, q_scale, k_scale, cos, sin, eps: float = 1e-6):
    """Per-head RMSNorm + rotary embedding of the Q and K columns (the first
    2 heads 128) of Y (bf16 [M][ld]), in place; returns Y."""
    M, ld = Y.shape
    _need(Y, "Y", torch.bfloat16, (M, ld))
    _need(q_scale, "q_scale", torch.bfloat16, (HEAD_DIM,))
    _need(k_scale, "k_scale", torch.bfloat16, (HEAD_DIM,))
    _need(cos, "cos", torch.float32, (M, HEAD_DIM // 2))
    _need(sin, "sin", torch.float32, (M, HEAD_DIM // 2))
    _check("svdq_qk_norm_rope",
           load().svdq_qk_norm_rope(M, heads, ld, _p(Y), _p(q_scale), _p(k_scale), _p(cos),
                                    _p(sin), float(eps), _stream()))
    return Y


def svdq_linear_forward_qk(d: SvdqDesc, M: int, ximage, wimage, heads: int, q_scale, k_scale,
                           cos, sin, eps: float = 1e-6, Y=None):
    """The layer's forward followed by the Q/K RMSNorm + rotary embedding of
    its first 2 heads 128 output columns (the GEMM, then the in-place pass)."""
    if Y is None:
        Y = torch.empty(M, d.N, dtype=torch.bfloat16, device=ximage.device)
    _need(Y, "Y", torch.bfloat16, (M, d.N))
    _need(ximage, "ximage", torch.uint8)
    _need(wimage, "wimage", torch.uint8)
    _need(q_scale, "q_scale", torch.bfloat16, (HEAD_DIM,))
    _need(k_scale, "k_scale", torch.bfloat16, (HEAD_DIM,))
    _need(cos, "cos", torch.float32, (M, HEAD_DIM // 2))
    _need(sin, "sin", torch.float32, (M, HEAD_DIM // 2))
    _check("svdq_linear_forward_qk",
           load().svdq_linear_forward_qk(ctypes.byref(d), M, _p(ximage), _nbytes(ximage),
                                         _p(wimage), _nbytes(wimage), heads,
                                         _p(q_scale), _p(k_scale), _p(cos), _p(sin), float(eps),
                                         _p(Y), _stream()))
    return Y


NVFP4_BLOCK = 16


def svdq_nvfp4_scale_from_absmax(amax, g=None):
    """g = fp32(max(amax) / 2688) (1 if the maximum is 0), as a 1-element
    device tensor."""
    _need(amax, "amax", torch.float32, (amax.numel(),))
    if g is None:
        g = torch.empty(1, dtype=torch.float32, device=amax.device)
    _need(g, "g", torch.float32, (1,))
    _check("svdq_nvfp4_scale_from_absmax",
           load().svdq_nvfp4_scale_from_absmax(amax.numel(), _p(amax), _p(g), _stream()))
    return g


def svdq_nvfp4_quantize_act(X, lam, g, xcodes=None, xscales=None, lora_down=None, T=None):
    """NVFP4 codes [M][K/2] and E4M3 scales [M][K/16] of X_hat = X / lambda,
    and T = X_hat L1 [M][r] fp32 from the same pass when lora_down ([r][K])
    is given.  Returns (xcodes, xscales, T or None)."""
    M, K = X.shape
    rank = 0 if lora_down is None else lora_down.shape[0]
    _need(X, "X", torch.bfloat16, (M, K))
    _need(lam, "lambda", torch.float32, (K,))
    _need(g, "g", torch.float32, (1,))
    if xcodes is None:
        xcodes = torch.empty(M, K // 2, dtype=torch.uint8, device=X.device)
    if xscales is None:
        xscales = torch.empty(M, K // NVFP4_BLOCK, dtype=torch.uint8, device=X.device)
    _need(xcodes, "xcodes", torch.uint8, (M, K // 2))
    _need(xscales, "xscales", torch.uint8, (M, K // NVFP4_BLOCK))
    if rank:
        _need(lora_down, "lora_down", torch.bfloat16, (rank, K))
        if T is None:
            T = torch.empty(M, rank, dtype=torch.float32, device=X.device)
        _need(T, "T", torch.float32, (M, rank))
    _check("svdq_nvfp4_quantize_act",
           load().svdq_nvfp4_quantize_act(M, K, rank, _p(X), _p(lam), _p(g), _p(lora_down),
                                          _p(xcodes), _p(xscales), _p(T if rank else None),
                                          _stream()))
    return xcodes, xscales, (T if rank else None)


def svdq_nvfp4_pack_weight(W, lam, rank: int, lora_down=None, lora_up=None):
    """(codes [N][K/2], E4M3 scales [N][K/16], g [1]) of the weight residual."""
    N, K = W.shape
    _need(W, "W", torch.bfloat16, (N, K))
    _need(lam, "lambda", torch.float32, (K,))
    _need(lora_down, "lora_down", torch.bfloat16, (rank, K), optional=rank == 0)
    _need(lora_up, "lora_up", torch.bfloat16, (N, rank), optional=rank == 0)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=W.device)
    scales = torch.empty(N, K // NVFP4_BLOCK, dtype=torch.uint8, device=W.device)
    g = torch.empty(1, dtype=torch.float32, device=W.device)
    _check("svdq_nvfp4_pack_weight",
           load().svdq_nvfp4_pack_weight(N, K, rank, _p(W), _p(lam), _p(lora_down), _p(lora_up),
                                         _p(codes), _p(scales), _p(g), _stream()))
    return codes, scales, g


def svdq_nvfp4_linear(xcodes, xscales, g_x, wcodes, wscales, g_w, T=None, lora_up=None,
                      bias=None, Y=None, out_f32: bool = False):
    """Y = deq(X) deq(W)^T + T L2 + bias for NVFP4 operands."""
    M, K2 = xcodes.shape
    N = wcodes.shape[0]
    K = 2 * K2
    rank = 0 if lora_up is None else lora_up.shape[1]
    out_dtype = torch.float32 if out_f32 else torch.bfloat16
    _need(xcodes, "xcodes", torch.uint8, (M, K // 2))
    _need(xscales, "xscales", torch.uint8, (M, K // NVFP4_BLOCK))
    _need(wcodes, "wcodes", torch.uint8, (N, K // 2))
    _need(wscales, "wscales", torch.uint8, (N, K // NVFP4_BLOCK))
    _need(g_x, "g_x", torch.float32, (1,))
    _need(g_w, "g_w", torch.float32, (1,))
    _need(T, "T", torch.float32, (M, rank), optional=rank == 0)
    _need(bias, "bias", torch.bfloat16, (N,), optional=True)
    if Y is None:
        Y = torch.empty(M, N, dtype=out_dtype, device=xcodes.device)
    _need(Y, "Y", out_dtype, (M, N))
    _check("svdq_nvfp4_linear",
           load().svdq_nvfp4_linear(M, N, K, rank, _p(xcodes), _p(xscales), _p(g_x), _p(wcodes),
                                    _p(wscales), _p(g_w), _p(T), _p(lora_up), _p(bias),
                                    SVDQ_FLAG_OUT_F32 if out_f32 else 0, _p(Y), _stream()))
    return Y
