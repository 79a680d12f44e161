"""Python binding of libfp8lin: FP8 block-scaled quantized linear layer on MI355X.

Thin ctypes marshalling over the C ABI in ``include/fp8lin.h``; every step of
the computation runs in the library's HIP kernels.  PyTorch only provides the
device memory (output tensors) and the current HIP stream.  The functions keep
the C names.  The library is loaded from this package directory and must have
been built first (``python -m fp8_block_scaled_act_amd._build`` or
``__graft_entry__.build()``); if it is missing, importing the functions raises.

Tensor conventions: BF16 tensors are ``torch.bfloat16``; FP8 E4M3 codes are
``torch.uint8``; scales are ``torch.float32``; everything is contiguous and on
the current CUDA/HIP device.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "Fp8LinError", "GROUP",
    "fp8_quant_act", "fp8_quant_weight", "fp8_weight_transpose", "fp8_weight_pack", "fp8_quant_transpose",
    "fp8_gemm_fwd", "fp8_gemm_fwd_unified", "fp8_gemm_fwd_packed",
    "fp8_gemm_fwd_packed_splitk", "fp8_gemm_fwd_packed_splitk_workspace", "fp8_gemm_fwd_packed_splitk_noalloc",
    "SPLITK_SCRATCH_BYTES", "fp8_linear_fwd", "fp8_gemm_dgrad", "fp8_gemm_dgrad_t", "fp8_gemm_wgrad",
    "fp8_rmsnorm_quant", "fp8_rmsnorm_bwd", "fp8_rmsnorm_bwd_workspace", "fp8_swiglu_quant", "fp8_swiglu_bwd", "fp8_swiglu_bwd_quant", "fp8_mlp_fwd", "fp8_mlp_bwd",
    "fp8_mxfp4_quant_weight", "fp8_gemm_fwd_w4",
    "fp8lin_encode_e4m3", "fp8lin_decode_e4m3", "fp8lin_gemm_fwd_mfma_probe", "MFMA_PROBE_FORMS",
    "fp8lin_math_probe",
    "fp8lin_flag_probe",
    "SRC_BF16", "SRC_FP8_ROWQ",
]

GROUP = 128
SPLITK_SCRATCH_BYTES = 4 << 20     # FP8LIN_SPLITK_SCRATCH_BYTES
SRC_BF16 = 0
SRC_FP8_ROWQ = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8lin.so")

_SYMBOLS = {
    # name: (argtypes, restype)
    "fp8lin_version": ([], ctypes.c_int),
    "fp8lin_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "fp8lin_last_hip_error": ([], ctypes.c_int),
    "fp8_quant_act": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p], ctypes.c_int),
    "fp8_quant_weight": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_void_p], ctypes.c_int),
    "fp8_weight_transpose": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "fp8_weight_pack": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p],
                        ctypes.c_int),
    "fp8_gemm_fwd_packed": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8_quant_transpose": ([ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p], ctypes.c_int),
    "fp8_gemm_fwd": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8_gemm_fwd_packed_splitk": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2 +
                                   [ctypes.c_int64, ctypes.c_void_p], ctypes.c_int),
    "fp8_gemm_fwd_packed_splitk_workspace": ([ctypes.c_int64] * 3, ctypes.c_int64),
    "fp8_gemm_fwd_packed_splitk_noalloc": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2,
                                           ctypes.c_int),
    "fp8_gemm_fwd_unified": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8_linear_fwd": ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 4, ctypes.c_int),
    "fp8_gemm_dgrad": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8_gemm_dgrad_t": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8_gemm_wgrad": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8_rmsnorm_quant": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "fp8_rmsnorm_bwd_workspace": ([ctypes.c_int64] * 2, ctypes.c_int64),
    "fp8_rmsnorm_bwd": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 3 +
                        [ctypes.c_int64, ctypes.c_void_p], ctypes.c_int),
    "fp8_swiglu_quant": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "fp8_swiglu_bwd": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "fp8_swiglu_bwd_quant": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                              ctypes.c_int64] + [ctypes.c_void_p] * 5, ctypes.c_int),
    "fp8_mlp_fwd": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float] + [ctypes.c_void_p] * 4 +
                    [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 8, ctypes.c_int),
    "fp8_mxfp4_quant_weight": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "fp8_gemm_fwd_w4": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2, ctypes.c_int),
    "fp8lin_encode_e4m3": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p],
                           ctypes.c_int),
    "fp8lin_decode_e4m3": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p],
                           ctypes.c_int),
    "fp8lin_gemm_fwd_mfma_probe": ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 +
                                   [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p], ctypes.c_int),
    "fp8lin_math_probe": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p],
                          ctypes.c_int),
    "fp8lin_flag_probe": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p],
                          ctypes.c_int),
}

_lib = None


class Fp8LinError(RuntimeError):
    def __init__(self, status: int, where: str):
        text = lib().fp8lin_status_string(status).decode()
        extra = ""
        if status == 6:
            extra = " (hipError_t %d)" % lib().fp8lin_last_hip_error()
        super().__init__("%s: %s%s" % (where, text, extra))
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libfp8lin (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libfp8lin.so is not built at %s; run __graft_entry__.build() or "
                              "python -m fp8_block_scaled_act_amd._build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SYMBOLS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Fp8LinError(status, where)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() and not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)


def _expect_workspace(ws: torch.Tensor, name: str, dtype: torch.dtype, like: torch.Tensor) -> int:
    """Checks a caller workspace like any other operand (a tensor of `dtype`,
    contiguous, on the device of `like`) and returns its size in bytes."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if ws.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, ws.dtype))
    if not ws.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if not ws.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if like.is_cuda and ws.device != like.device:
        raise ValueError("%s must be on %s, got %s" % (name, like.device, ws.device))
    return ws.numel() * ws.element_size()


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


# --------------------------------------------------------------- quantization

def fp8_quant_act(x: torch.Tensor, out=None, stream=None):
    """1x128 row-group quantization: x bf16 [M,K] -> (codes u8 [M,K], scales f32 [M,K/128])."""
    M, K = x.shape
    _expect(x, "x", torch.bfloat16, (M, K))
    q, s = out if out is not None else (_empty((M, K), torch.uint8, x), _empty((M, K // GROUP), torch.float32, x))
    _expect(q, "xq", torch.uint8, (M, K))
    _expect(s, "sx", torch.float32, (M, K // GROUP))
    _check(lib().fp8_quant_act(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(stream)), "fp8_quant_act")
    return q, s


def fp8_quant_weight(w: torch.Tensor, out=None, stream=None):
    """128x128 block quantization: w bf16 [N,K] -> (codes u8 [N,K], scales f32 [N/128,K/128])."""
    N, K = w.shape
    _expect(w, "w", torch.bfloat16, (N, K))
    q, s = out if out is not None else (_empty((N, K), torch.uint8, w),
                                        _empty((N // GROUP, K // GROUP), torch.float32, w))
    _expect(q, "wq", torch.uint8, (N, K))
    _expect(s, "sw", torch.float32, (N // GROUP, K // GROUP))
    _check(lib().fp8_quant_weight(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(stream)), "fp8_quant_weight")
    return q, s


def fp8_weight_transpose(wq: torch.Tensor, sw: torch.Tensor, out=None, stream=None):
    """Exact transposed copy of a quantized weight: (wq u8 [N,K], sw f32 [N/128,K/128]) ->
    (wqT u8 [K,N], swT f32 [K/128,N/128]), for fp8_gemm_dgrad_t."""
    N, K = wq.shape
    _expect(wq, "wq", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    qT, sT = out if out is not None else (_empty((K, N), torch.uint8, wq),
                                          _empty((K // GROUP, N // GROUP), torch.float32, wq))
    _expect(qT, "wqT", torch.uint8, (K, N))
    _expect(sT, "swT", torch.float32, (K // GROUP, N // GROUP))
    _check(lib().fp8_weight_transpose(_ptr(wq), _ptr(sw), N, K, _ptr(qT), _ptr(sT), _stream(stream)),
           "fp8_weight_transpose")
    return qT, sT


def fp8_weight_pack(wq: torch.Tensor, out=None, stream=None):
    """Decode layout of quantized weight codes u8 [N,K] (same bytes, reordered;
    a u8 tensor of shape [N,K]) for fp8_gemm_fwd_packed."""
    N, K = wq.shape
    _expect(wq, "wq", torch.uint8, (N, K))
    wqp = out if out is not None else _empty((N, K), torch.uint8, wq)
    _expect(wqp, "wqp", torch.uint8, (N, K))
    _check(lib().fp8_weight_pack(_ptr(wq), N, K, _ptr(wqp), _stream(stream)), "fp8_weight_pack")
    return wqp


def fp8_quant_transpose(src: torch.Tensor, src_scales: torch.Tensor | None = None, dual: bool = False,
                        out=None, stream=None):
    """128-along-T quantization written transposed (WGrad operands).

    src bf16 [T,C] (src_scales None), or saved FP8 codes u8 [T,C] with 1x128
    scales f32 [T,C/128].  Returns (codesT u8 [C,T], scalesT f32 [C,T/128]) and,
    with dual=True (BF16 only), also (codes u8 [T,C], scales f32 [T,C/128]) of
    the 1x128 row quantization from the same read."""
    T, C = src.shape
    if src_scales is None:
        kind = SRC_BF16
        _expect(src, "src", torch.bfloat16, (T, C))
    else:
        kind = SRC_FP8_ROWQ
        _expect(src, "src", torch.uint8, (T, C))
        _expect(src_scales, "src_scales", torch.float32, (T, C // GROUP))
    if out is None:
        qT, sT = _empty((C, T), torch.uint8, src), _empty((C, T // GROUP), torch.float32, src)
        qr = sr = None
        if dual:
            qr, sr = _empty((T, C), torch.uint8, src), _empty((T, C // GROUP), torch.float32, src)
    else:
        qT, sT, qr, sr = out
    _expect(qT, "dstT", torch.uint8, (C, T))
    _expect(sT, "sT", torch.float32, (C, T // GROUP))
    if qr is not None:
        _expect(qr, "dst_rowq", torch.uint8, (T, C))
        _expect(sr, "s_rowq", torch.float32, (T, C // GROUP))
    _check(lib().fp8_quant_transpose(kind, _ptr(src), _ptr(src_scales), T, C, _ptr(qT), _ptr(sT), _ptr(qr),
                                     _ptr(sr), _stream(stream)), "fp8_quant_transpose")
    return (qT, sT, qr, sr) if dual else (qT, sT)


# ---------------------------------------------------------------------- GEMMs

def fp8_gemm_fwd(xq, sx, wq, sw, out=None, stream=None):
    """Y[M,N] bf16 = X W^T from 1x128-quantized X [M,K] and 128x128-quantized W [N,K]."""
    M, K = xq.shape
    N = wq.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(wq, "wq", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    y = out if out is not None else _empty((M, N), torch.bfloat16, xq)
    _expect(y, "y", torch.bfloat16, (M, N))
    _check(lib().fp8_gemm_fwd(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _stream(stream)),
           "fp8_gemm_fwd")
    return y


MX_BLOCK = 32


def fp8_mxfp4_quant_weight(w: torch.Tensor, out=None, stream=None):
    """MXFP4 quantization of 4-bit rollout weights: w bf16 [N,K] -> (codes u8
    [N,K/2], two E2M1 codes per byte with the even k in the low nibble; scales
    u8 [N,K/32], E8M0 per 32-block)."""
    N, K = w.shape
    _expect(w, "w", torch.bfloat16, (N, K))
    c, s = out if out is not None else (_empty((N, K // 2), torch.uint8, w),
                                        _empty((N, K // MX_BLOCK), torch.uint8, w))
    _expect(c, "codes", torch.uint8, (N, K // 2))
    _expect(s, "scales", torch.uint8, (N, K // MX_BLOCK))
    _check(lib().fp8_mxfp4_quant_weight(_ptr(w), N, K, _ptr(c), _ptr(s), _stream(stream)),
           "fp8_mxfp4_quant_weight")
    return c, s


def fp8_gemm_fwd_w4(xq, sx, codes, scales, out=None, stream=None):
    """Y[M,N] bf16 = X W^T from 1x128-quantized X [M,K] and MXFP4 W (codes
    [N,K/2], scales [N,K/32])."""
    M, K = xq.shape
    N = codes.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(codes, "codes", torch.uint8, (N, K // 2))
    _expect(scales, "scales", torch.uint8, (N, K // MX_BLOCK))
    y = out if out is not None else _empty((M, N), torch.bfloat16, xq)
    _expect(y, "y", torch.bfloat16, (M, N))
    _check(lib().fp8_gemm_fwd_w4(_ptr(xq), _ptr(sx), _ptr(codes), _ptr(scales), M, N, K, _ptr(y),
                                 _stream(stream)), "fp8_gemm_fwd_w4")
    return y


def fp8_gemm_fwd_packed_splitk_workspace(M: int, N: int, K: int) -> int:
    """Workspace bytes fp8_gemm_fwd_packed_splitk needs for this shape (0: none)."""
    n = lib().fp8_gemm_fwd_packed_splitk_workspace(M, N, K)
    if n < 0:
        raise Fp8LinError(2, "fp8_gemm_fwd_packed_splitk_workspace")
    return n


def fp8_gemm_fwd_packed_splitk(xq, sx, wqp, sw, workspace=None, out=None, stream=None):
    """fp8_gemm_fwd_packed split over K for few output columns.  workspace: a
    float32 CUDA tensor of at least fp8_gemm_fwd_packed_splitk_workspace bytes
    (allocated here when None)."""
    M, K = xq.shape
    N = wqp.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(wqp, "wqp", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    need = fp8_gemm_fwd_packed_splitk_workspace(M, N, K)
    if workspace is None:
        workspace = _empty((max(need // 4, 1),), torch.float32, xq)
    nbytes = _expect_workspace(workspace, "workspace", torch.float32, xq)
    y = out if out is not None else _empty((M, N), torch.bfloat16, xq)
    _expect(y, "y", torch.bfloat16, (M, N))
    _check(lib().fp8_gemm_fwd_packed_splitk(_ptr(xq), _ptr(sx), _ptr(wqp), _ptr(sw), M, N, K, _ptr(y),
                                            _ptr(workspace), nbytes, _stream(stream)),
           "fp8_gemm_fwd_packed_splitk")
    return y


def fp8_gemm_fwd_packed_splitk_noalloc(xq, sx, wqp, sw, out=None, stream=None):
    """fp8_gemm_fwd_packed_splitk with its fp32 partial sums in the library's
    static per-GPU scratch (FP8LIN_SPLITK_SCRATCH_BYTES): the C call allocates
    nothing.  Pass `out` to keep this wrapper allocation-free as well.  Calls
    that overlap on one GPU race on the shared scratch."""
    M, K = xq.shape
    N = wqp.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(wqp, "wqp", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    y = out if out is not None else _empty((M, N), torch.bfloat16, xq)
    _expect(y, "y", torch.bfloat16, (M, N))
    _check(lib().fp8_gemm_fwd_packed_splitk_noalloc(_ptr(xq), _ptr(sx), _ptr(wqp), _ptr(sw), M, N, K, _ptr(y),
                                                    _stream(stream)), "fp8_gemm_fwd_packed_splitk_noalloc")
    return y


def fp8_gemm_fwd_unified(xq, sx, wq, sw, out=None, stream=None):
    """fp8_gemm_fwd computed by one kernel for every M: a row's output bits do
    not depend on the rows it is computed with (decode and prefill agree)."""
    M, K = xq.shape
    N = wq.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(wq, "wq", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    y = out if out is not None else _empty((M, N), torch.bfloat16, xq)
    _expect(y, "y", torch.bfloat16, (M, N))
    _check(lib().fp8_gemm_fwd_unified(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _stream(stream)),
           "fp8_gemm_fwd_unified")
    return y


def fp8_gemm_fwd_packed(xq, sx, wqp, sw, out=None, stream=None):
    """Y[M,N] bf16 = X W^T for M <= 64 from the decode layout wqp = fp8_weight_pack(wq)."""
    M, K = xq.shape
    N = wqp.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(wqp, "wqp", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    y = out if out is not None else _empty((M, N), torch.bfloat16, xq)
    _expect(y, "y", torch.bfloat16, (M, N))
    _check(lib().fp8_gemm_fwd_packed(_ptr(xq), _ptr(sx), _ptr(wqp), _ptr(sw), M, N, K, _ptr(y), _stream(stream)),
           "fp8_gemm_fwd_packed")
    return y


def fp8_linear_fwd(x, wq, sw, out=None, stream=None):
    """Quantize x bf16 [M,K] (1x128) and multiply by the quantized W [N,K]:
    returns (y bf16 [M,N], xq u8 [M,K], sx f32 [M,K/128])."""
    M, K = x.shape
    N = wq.shape[0]
    _expect(x, "x", torch.bfloat16, (M, K))
    _expect(wq, "wq", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    if out is None:
        y, q, s = (_empty((M, N), torch.bfloat16, x), _empty((M, K), torch.uint8, x),
                   _empty((M, K // GROUP), torch.float32, x))
    else:
        y, q, s = out
    _expect(y, "y", torch.bfloat16, (M, N))
    _expect(q, "xq", torch.uint8, (M, K))
    _expect(s, "sx", torch.float32, (M, K // GROUP))
    _check(lib().fp8_linear_fwd(_ptr(x), _ptr(wq), _ptr(sw), M, N, K, _ptr(q), _ptr(s), _ptr(y), _stream(stream)),
           "fp8_linear_fwd")
    return y, q, s


# ------------------------------------------------- producers fused with quant

def fp8_rmsnorm_quant(x, gamma, eps: float = 1e-6, out=None, rstd: bool = True, stream=None):
    """RMSNorm of x bf16 [M,K] with gamma bf16 [K], quantized 1x128 without
    storing the BF16 output: returns (xq u8 [M,K], sx f32 [M,K/128], rstd f32 [M]
    or None)."""
    M, K = x.shape
    _expect(x, "x", torch.bfloat16, (M, K))
    _expect(gamma, "gamma", torch.bfloat16, (K,))
    if out is None:
        q, s = _empty((M, K), torch.uint8, x), _empty((M, K // GROUP), torch.float32, x)
        r = _empty((M,), torch.float32, x) if rstd else None
    else:
        q, s, r = out
    _expect(q, "xq", torch.uint8, (M, K))
    _expect(s, "sx", torch.float32, (M, K // GROUP))
    if r is not None:
        _expect(r, "rstd", torch.float32, (M,))
    _check(lib().fp8_rmsnorm_quant(_ptr(x), _ptr(gamma), M, K, float(eps), _ptr(q), _ptr(s), _ptr(r),
                                   _stream(stream)), "fp8_rmsnorm_quant")
    return q, s, r


def fp8_rmsnorm_bwd_workspace(M: int, K: int) -> int:
    n = lib().fp8_rmsnorm_bwd_workspace(M, K)
    if n < 0:
        raise Fp8LinError(2, "fp8_rmsnorm_bwd_workspace")
    return n


def fp8_rmsnorm_bwd(x, gamma, rstd, dy, dgamma: bool = True, workspace=None, out=None, stream=None):
    """Backward of fp8_rmsnorm_quant's RMSNorm: x, dy bf16 [M,K], gamma bf16 [K],
    rstd f32 [M] -> (dx bf16 [M,K], dgamma f32 [K] or None).  workspace: a
    float64 CUDA tensor of fp8_rmsnorm_bwd_workspace bytes (allocated here when
    None)."""
    M, K = x.shape
    _expect(x, "x", torch.bfloat16, (M, K))
    _expect(dy, "dy", torch.bfloat16, (M, K))
    _expect(gamma, "gamma", torch.bfloat16, (K,))
    _expect(rstd, "rstd", torch.float32, (M,))
    if out is None:
        dx = _empty((M, K), torch.bfloat16, x)
        dg = _empty((K,), torch.float32, x) if dgamma else None
    else:
        dx, dg = out
    _expect(dx, "dx", torch.bfloat16, (M, K))
    if dg is not None:
        _expect(dg, "dgamma", torch.float32, (K,))
    need = fp8_rmsnorm_bwd_workspace(M, K) if dg is not None else 0
    if workspace is None and need:
        workspace = _empty((need // 8,), torch.float64, x)
    nbytes = _expect_workspace(workspace, "workspace", torch.float64, x) if workspace is not None else 0
    _check(lib().fp8_rmsnorm_bwd(_ptr(x), _ptr(gamma), _ptr(rstd), _ptr(dy), M, K, _ptr(dx), _ptr(dg),
                                 _ptr(workspace), nbytes, _stream(stream)), "fp8_rmsnorm_bwd")
    return dx, dg


def fp8_swiglu_quant(gate, up, out=None, stream=None):
    """silu(gate) * up of bf16 [M,F] operands, quantized 1x128 without storing
    the BF16 product: returns (hq u8 [M,F], sh f32 [M,F/128]).  gate and up may
    be row-strided views (e.g. the two halves of one [M,2F] tensor) with equal
    row strides and unit column stride."""
    if gate.shape != up.shape or gate.dim() != 2:
        raise ValueError("gate and up must be 2-D tensors of one shape")
    M, F = gate.shape
    for t, name in ((gate, "gate"), (up, "up")):
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be torch.bfloat16" % name)
        if t.numel() and not t.is_cuda:
            raise ValueError("%s must be on the GPU" % name)
        if M and F and t.stride(1) != 1:
            raise ValueError("%s must have unit column stride" % name)
    ld = gate.stride(0) if M > 1 else F
    if M > 1 and up.stride(0) != ld:
        raise ValueError("gate and up must have the same row stride")
    q, s = out if out is not None else (_empty((M, F), torch.uint8, gate),
                                        _empty((M, F // GROUP), torch.float32, gate))
    _expect(q, "hq", torch.uint8, (M, F))
    _expect(s, "sh", torch.float32, (M, F // GROUP))
    _check(lib().fp8_swiglu_quant(_ptr(gate), _ptr(up), ld, M, F, _ptr(q), _ptr(s), _stream(stream)),
           "fp8_swiglu_quant")
    return q, s


def fp8_swiglu_bwd(gate, up, dh, out=None, stream=None):
    """BF16 gradients of silu(gate) * up given dh bf16 [M,F]: returns dgu bf16
    [M,2F] = [d_gate | d_up].  gate and up may be row-strided views (e.g. the
    two halves of the saved [M,2F] gate/up output) with equal row strides."""
    if gate.shape != up.shape or gate.dim() != 2:
        raise ValueError("gate and up must be 2-D tensors of one shape")
    M, F = gate.shape
    _expect(dh, "dh", torch.bfloat16, (M, F))
    for t, name in ((gate, "gate"), (up, "up")):
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be torch.bfloat16" % name)
        if t.numel() and not t.is_cuda:
            raise ValueError("%s must be on the GPU" % name)
        if M and F and t.stride(1) != 1:
            raise ValueError("%s must have unit column stride" % name)
    ld = gate.stride(0) if M > 1 else F
    if M > 1 and up.stride(0) != ld:
        raise ValueError("gate and up must have the same row stride")
    dgu = out if out is not None else _empty((M, 2 * F), torch.bfloat16, dh)
    _expect(dgu, "dgu", torch.bfloat16, (M, 2 * F))
    _check(lib().fp8_swiglu_bwd(_ptr(gate), _ptr(up), ld, _ptr(dh), M, F, _ptr(dgu), _stream(stream)),
           "fp8_swiglu_bwd")
    return dgu


def fp8_swiglu_bwd_quant(gate, up, dh, out=None, stream=None):
    """SwiGLU backward fused with the dual FP8 quantization of its result:
    returns (dguTq u8 [2F,T], sdguT f32 [2F,T/128], dguq u8 [T,2F], sdgu f32
    [T,2F/128]) -- the order of fp8_quant_transpose(..., dual=True)."""
    if gate.shape != up.shape or gate.dim() != 2:
        raise ValueError("gate and up must be 2-D tensors of one shape")
    T, F = gate.shape
    _expect(dh, "dh", torch.bfloat16, (T, F))
    for t, name in ((gate, "gate"), (up, "up")):
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be torch.bfloat16" % name)
        if T and F and t.stride(1) != 1:
            raise ValueError("%s must have unit column stride" % name)
    ld = gate.stride(0) if T > 1 else F
    if T > 1 and up.stride(0) != ld:
        raise ValueError("gate and up must have the same row stride")
    if out is None:
        qT, sT = _empty((2 * F, T), torch.uint8, dh), _empty((2 * F, T // GROUP), torch.float32, dh)
        q, s = _empty((T, 2 * F), torch.uint8, dh), _empty((T, 2 * F // GROUP), torch.float32, dh)
    else:
        qT, sT, q, s = out
    _expect(qT, "dguTq", torch.uint8, (2 * F, T))
    _expect(sT, "sdguT", torch.float32, (2 * F, T // GROUP))
    _expect(q, "dguq", torch.uint8, (T, 2 * F))
    _expect(s, "sdgu", torch.float32, (T, 2 * F // GROUP))
    _check(lib().fp8_swiglu_bwd_quant(_ptr(gate), _ptr(up), ld, _ptr(dh), T, F, _ptr(q), _ptr(s), _ptr(qT), _ptr(sT),
                                      _stream(stream)), "fp8_swiglu_bwd_quant")
    return qT, sT, q, s


def fp8_mlp_fwd(x, gamma, wgu, sgu, wdown, sdown, eps: float = 1e-6, out=None, rstd: bool = True, stream=None):
    """Forward pass of an FP8 MLP block: RMSNorm -> gate/up GEMM -> SwiGLU -> down GEMM.

    x bf16 [T,K], gamma bf16 [K], wgu/sgu the 128x128 quantization of the fused
    [gate; up] weight [2F,K], wdown/sdown that of the down weight [K,F].
    Returns dict(y, xq, sx, rstd, gu, hq, sh): the output and what the backward
    pass keeps (FP8 inputs of both linear layers, rstd, and the BF16 gate/up
    output)."""
    T, K = x.shape
    F2 = wgu.shape[0]
    F = F2 // 2
    _expect(x, "x", torch.bfloat16, (T, K))
    _expect(gamma, "gamma", torch.bfloat16, (K,))
    _expect(wgu, "wgu", torch.uint8, (F2, K))
    _expect(sgu, "sgu", torch.float32, (F2 // GROUP, K // GROUP))
    _expect(wdown, "wdown", torch.uint8, (K, F))
    _expect(sdown, "sdown", torch.float32, (K // GROUP, F // GROUP))
    if out is None:
        out = {"y": _empty((T, K), torch.bfloat16, x), "xq": _empty((T, K), torch.uint8, x),
               "sx": _empty((T, K // GROUP), torch.float32, x),
               "rstd": _empty((T,), torch.float32, x) if rstd else None,
               "gu": _empty((T, F2), torch.bfloat16, x), "hq": _empty((T, F), torch.uint8, x),
               "sh": _empty((T, F // GROUP), torch.float32, x)}
    _expect(out["y"], "y", torch.bfloat16, (T, K))
    _expect(out["xq"], "xq", torch.uint8, (T, K))
    _expect(out["sx"], "sx", torch.float32, (T, K // GROUP))
    if out["rstd"] is not None:
        _expect(out["rstd"], "rstd", torch.float32, (T,))
    _expect(out["gu"], "gu", torch.bfloat16, (T, F2))
    _expect(out["hq"], "hq", torch.uint8, (T, F))
    _expect(out["sh"], "sh", torch.float32, (T, F // GROUP))
    _check(lib().fp8_mlp_fwd(_ptr(x), _ptr(gamma), float(eps), _ptr(wgu), _ptr(sgu), _ptr(wdown), _ptr(sdown),
                             T, K, F, _ptr(out["xq"]), _ptr(out["sx"]), _ptr(out["rstd"]), _ptr(out["gu"]),
                             _ptr(out["hq"]), _ptr(out["sh"]), _ptr(out["y"]), _stream(stream)), "fp8_mlp_fwd")
    return out


def fp8_mlp_bwd(dy, saved, wguT, sguT, wdT, sdT, x=None, gamma=None, stream=None):
    """Backward pass of the FP8 MLP block through its three linear layers, as a
    fixed sequence of C-ABI calls on one stream (every step runs in the
    library's kernels; this function only allocates the intermediates):

      fp8_quant_transpose(dy, dual)           -> dYq (1x128), dY^T q (128 along T)
      fp8_quant_transpose(hq, sh)             -> H^T q        (saved FP8 SwiGLU output)
      fp8_gemm_wgrad(dY^T q, H^T q)           -> dw_down [K,F]
      fp8_gemm_dgrad_t(dYq, W_down^T)         -> dh [T,F]
      fp8_swiglu_bwd_quant(gate, up, dh)      -> dGUq, dGU^T q (SwiGLU backward fused with the
                                                 dual quantization of its BF16 result)
      fp8_quant_transpose(xq, sx)             -> X^T q        (saved FP8 block input)
      fp8_gemm_wgrad(dGU^T q, X^T q)          -> dw_gu [2F,K]
      fp8_gemm_dgrad_t(dGUq, W_gu^T)          -> dxn [T,K]    (gradient of the RMSNorm output)
      fp8_rmsnorm_bwd(x, gamma, rstd, dxn)    -> dx [T,K], dgamma [K]   (when x and gamma are given)

    dy bf16 [T,K]; saved is the dict returned by fp8_mlp_fwd; wguT/sguT and
    wdT/sdT are the transposed weight copies (fp8_weight_transpose of the
    fused gate/up and down weights).  T % 128 == 0 (WGrad groups run along T).
    x, gamma: the block's input and RMSNorm gain (the forward's arguments);
    with them the RMSNorm backward runs too.
    Returns dict(dxn, dw_gu, dw_down, dh[, dx, dgamma])."""
    T, K = dy.shape
    F = saved["hq"].shape[1]
    st = stream
    dyTq, sdyT, dyq, sdy = fp8_quant_transpose(dy, dual=True, stream=st)
    hTq, shT = fp8_quant_transpose(saved["hq"], saved["sh"], stream=st)
    dw_down = fp8_gemm_wgrad(dyTq, sdyT, hTq, shT, stream=st)
    dh = fp8_gemm_dgrad_t(dyq, sdy, wdT, sdT, stream=st)
    gu = saved["gu"]
    dguTq, sguT_, dguq, sdgu = fp8_swiglu_bwd_quant(gu[:, :F], gu[:, F:], dh, stream=st)
    xTq, sxT = fp8_quant_transpose(saved["xq"], saved["sx"], stream=st)
    dw_gu = fp8_gemm_wgrad(dguTq, sguT_, xTq, sxT, stream=st)
    dxn = fp8_gemm_dgrad_t(dguq, sdgu, wguT, sguT, stream=st)
    grads = {"dxn": dxn, "dw_gu": dw_gu, "dw_down": dw_down, "dh": dh}
    if x is not None and gamma is not None:
        grads["dx"], grads["dgamma"] = fp8_rmsnorm_bwd(x, gamma, saved["rstd"], dxn, stream=st)
    return grads


def fp8_gemm_dgrad(dyq, sdy, wq, sw, out=None, stream=None):
    """dX[T,K] bf16 = dY W from 1x128-quantized dY [T,N] and 128x128-quantized W [N,K]."""
    T, N = dyq.shape
    K = wq.shape[1]
    _expect(dyq, "dyq", torch.uint8, (T, N))
    _expect(sdy, "sdy", torch.float32, (T, N // GROUP))
    _expect(wq, "wq", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    dx = out if out is not None else _empty((T, K), torch.bfloat16, dyq)
    _expect(dx, "dx", torch.bfloat16, (T, K))
    _check(lib().fp8_gemm_dgrad(_ptr(dyq), _ptr(sdy), _ptr(wq), _ptr(sw), T, N, K, _ptr(dx), _stream(stream)),
           "fp8_gemm_dgrad")
    return dx


def fp8_gemm_dgrad_t(dyq, sdy, wqT, swT, out=None, stream=None):
    """dX[T,K] bf16 = dY W from 1x128-quantized dY [T,N] and the transposed
    weight copy (fp8_weight_transpose): wqT [K,N], swT [K/128,N/128]."""
    T, N = dyq.shape
    K = wqT.shape[0]
    _expect(dyq, "dyq", torch.uint8, (T, N))
    _expect(sdy, "sdy", torch.float32, (T, N // GROUP))
    _expect(wqT, "wqT", torch.uint8, (K, N))
    _expect(swT, "swT", torch.float32, (K // GROUP, N // GROUP))
    dx = out if out is not None else _empty((T, K), torch.bfloat16, dyq)
    _expect(dx, "dx", torch.bfloat16, (T, K))
    _check(lib().fp8_gemm_dgrad_t(_ptr(dyq), _ptr(sdy), _ptr(wqT), _ptr(swT), T, N, K, _ptr(dx), _stream(stream)),
           "fp8_gemm_dgrad_t")
    return dx


def fp8_gemm_wgrad(dyTq, sdyT, xTq, sxT, out=None, stream=None):
    """dW[N,K] bf16 = dY^T X from operands grouped 128-along-T: dY^T [N,T], X^T [K,T]."""
    N, T = dyTq.shape
    K = xTq.shape[0]
    _expect(dyTq, "dyTq", torch.uint8, (N, T))
    _expect(sdyT, "sdyT", torch.float32, (N, T // GROUP))
    _expect(xTq, "xTq", torch.uint8, (K, T))
    _expect(sxT, "sxT", torch.float32, (K, T // GROUP))
    dw = out if out is not None else _empty((N, K), torch.bfloat16, dyTq)
    _expect(dw, "dw", torch.bfloat16, (N, K))
    _check(lib().fp8_gemm_wgrad(_ptr(dyTq), _ptr(sdyT), _ptr(xTq), _ptr(sxT), N, K, T, _ptr(dw),
                                _stream(stream)), "fp8_gemm_wgrad")
    return dw


# ---------------------------------------------------------------- diagnostics

def fp8lin_encode_e4m3(x: torch.Tensor, method: int = 0, out=None, stream=None):
    """Device fp32 -> E4M3 encoder on a flat float32 tensor (method 0 = kernels')."""
    _expect(x, "in", torch.float32, tuple(x.shape))
    q = out if out is not None else torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().fp8lin_encode_e4m3(_ptr(x), x.numel(), _ptr(q), method, _stream(stream)), "fp8lin_encode_e4m3")
    return q


def fp8lin_decode_e4m3(q: torch.Tensor, method: int = 0, out=None, stream=None):
    """Device E4M3 -> fp32 decoder on a flat uint8 tensor (method 0 = kernels')."""
    _expect(q, "in", torch.uint8, tuple(q.shape))
    x = out if out is not None else torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib().fp8lin_decode_e4m3(_ptr(q), q.numel(), _ptr(x), method, _stream(stream)), "fp8lin_decode_e4m3")
    return x


def fp8lin_math_probe(x: torch.Tensor, fn: int, out=None, stream=None):
    """Device fp32 function on a flat float32 tensor: fn 0 = 2^x (v_exp_f32),
    fn 1 = 1/x (v_rcp_f32), fn 2 = x/448 and fn 3 = 1/x as the quantizers form
    their group scale and reciprocal without a division."""
    _expect(x, "in", torch.float32, tuple(x.shape))
    y = out if out is not None else torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _expect(y, "out", torch.float32, tuple(x.shape))
    _check(lib().fp8lin_math_probe(_ptr(x), x.numel(), _ptr(y), int(fn), _stream(stream)), "fp8lin_math_probe")
    return y


def fp8lin_flag_probe(v: torch.Tensor, lim: float, out=None, stream=None):
    """The SwiGLU kernels' fp64 re-evaluation test on a flat float32 tensor
    with bound lim (fp32 ulps): 1.0 where it flags the value, else 0.0."""
    _expect(v, "v", torch.float32, tuple(v.shape))
    y = out if out is not None else torch.empty(v.shape, dtype=torch.float32, device=v.device)
    _expect(y, "out", torch.float32, tuple(v.shape))
    _check(lib().fp8lin_flag_probe(_ptr(v), v.numel(), float(lim), _ptr(y), _stream(stream)), "fp8lin_flag_probe")
    return y


MFMA_PROBE_FORMS = {
    0: "v_mfma_scale_f32_16x16x128_f8f6f4",
    1: "v_mfma_scale_f32_32x32x64_f8f6f4",
    2: "v_mfma_f32_16x16x32_fp8_fp8",
    3: "v_mfma_f32_32x32x16_fp8_fp8",
    4: "v_mfma_f32_32x32x16_f16 (control: codes converted exactly to fp16)",
}


def fp8lin_gemm_fwd_mfma_probe(xq, sx, wq, sw, form: int, out=None, stream=None):
    """Diagnostic: fp8_gemm_fwd's product on matrix-core form `form` (see
    MFMA_PROBE_FORMS), fp32 output [M,N]."""
    M, K = xq.shape
    N = wq.shape[0]
    _expect(xq, "xq", torch.uint8, (M, K))
    _expect(sx, "sx", torch.float32, (M, K // GROUP))
    _expect(wq, "wq", torch.uint8, (N, K))
    _expect(sw, "sw", torch.float32, (N // GROUP, K // GROUP))
    y = out if out is not None else _empty((M, N), torch.float32, xq)
    _expect(y, "y", torch.float32, (M, N))
    _check(lib().fp8lin_gemm_fwd_mfma_probe(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), int(form),
                                            _stream(stream)), "fp8lin_gemm_fwd_mfma_probe")
    return y
