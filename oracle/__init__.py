"""CPU oracle for the FP8 block-scaled quantized linear layer (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never touches it, and it shares no code with them.

The arithmetic lives in ``fp8_oracle.c`` (plain C, fp32 quantization exactly as
defined, fp64 GEMM); this module only marshals numpy arrays through ctypes.
What is computed follows the Jet-RL technical summary (gist.science, paper
2601.14243), section "Quantization scheme": 1x128 activation groups, 128x128
weight blocks, FP8 forward/DGrad/WGrad GEMMs with WGrad grouped along tokens,
BF16 gradients, FP8 saved activations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GROUP = 128

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_quant_act.argtypes = [u16p, i64, i64, u8p, f32p]
        L.oracle_quant_weight.argtypes = [u16p, i64, i64, u8p, f32p]
        L.oracle_quant_transpose_bf16.argtypes = [u16p, i64, i64, u8p, f32p]
        L.oracle_quant_transpose_fp8.argtypes = [u8p, f32p, i64, i64, u8p, f32p]
        L.oracle_dequant_rowgroup.argtypes = [u8p, f32p, i64, i64, f64p]
        L.oracle_dequant_block.argtypes = [u8p, f32p, i64, i64, f64p]
        L.oracle_gemm.argtypes = [i64, i64, i64, f64p, i64, i64, f64p, i64, i64, f64p]
        L.oracle_rmsnorm_bf16.argtypes = [u16p, u16p, i64, i64, ctypes.c_float, u16p, f32p]
        L.oracle_swiglu_bf16.argtypes = [u16p, u16p, i64, i64, i64, u16p, u8p]
        L.oracle_swiglu_bwd_bf16.argtypes = [u16p, u16p, u16p, i64, i64, i64, u16p, u8p]
        L.oracle_rmsnorm_bwd.argtypes = [u16p, u16p, f32p, u16p, i64, i64, u16p, f32p]
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_mxfp4_quant.argtypes = [u16p, i64, i64, u8p, u8p]
        L.oracle_dequant_mxfp4.argtypes = [u8p, u8p, i64, i64, f64p]
        L.oracle_num_threads.restype = ctypes.c_int
        for f in ("oracle_quant_act", "oracle_quant_weight", "oracle_quant_transpose_bf16",
                  "oracle_quant_transpose_fp8", "oracle_dequant_rowgroup",
                  "oracle_dequant_block", "oracle_gemm", "oracle_rmsnorm_bf16",
                  "oracle_swiglu_bf16", "oracle_swiglu_bwd_bf16", "oracle_rmsnorm_bwd",
                  "oracle_mxfp4_quant", "oracle_dequant_mxfp4"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _bits16(x: np.ndarray) -> np.ndarray:
    """bf16 input given as uint16 bit patterns (numpy has no bf16)."""
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 tensors are passed as uint16 bit patterns"
    return x


# ------------------------------------------------------------------ format

def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (NaN for 0x7F/0xFF)."""
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([L.oracle_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def e4m3_encode_scalar(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def f64_to_bf16(x) -> np.ndarray:
    L = lib()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.array([L.oracle_f64_to_bf16(float(v)) for v in flat], dtype=np.uint16)
    return out.reshape(np.shape(x))


# ------------------------------------------------------------ quantization

def quant_act(x_bf16: np.ndarray):
    """1x128 row-group quant: x [M,K] bf16 bits -> (q u8 [M,K], s f32 [M,K/128])."""
    x = _bits16(x_bf16)
    M, K = x.shape
    assert K % GROUP == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // GROUP), np.float32)
    lib().oracle_quant_act(_ptr(x, ctypes.c_uint16), M, K, _ptr(q, ctypes.c_uint8),
                           _ptr(s, ctypes.c_float))
    return q, s


def quant_weight(w_bf16: np.ndarray):
    """128x128 block quant: w [N,K] -> (q u8 [N,K], s f32 [N/128, K/128])."""
    w = _bits16(w_bf16)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // GROUP, K // GROUP), np.float32)
    lib().oracle_quant_weight(_ptr(w, ctypes.c_uint16), N, K, _ptr(q, ctypes.c_uint8),
                              _ptr(s, ctypes.c_float))
    return q, s


def quant_transpose_bf16(x_bf16: np.ndarray):
    """128-along-T quant, transposed: x [T,C] -> (qT u8 [C,T], sT f32 [C, T/128])."""
    x = _bits16(x_bf16)
    T, C = x.shape
    assert T % GROUP == 0
    qT = np.empty((C, T), np.uint8)
    sT = np.empty((C, T // GROUP), np.float32)
    lib().oracle_quant_transpose_bf16(_ptr(x, ctypes.c_uint16), T, C, _ptr(qT, ctypes.c_uint8),
                                      _ptr(sT, ctypes.c_float))
    return qT, sT


def quant_transpose_fp8(q: np.ndarray, s_row: np.ndarray):
    """Requantize a saved FP8 tensor 128-along-T: q [T,C], s_row [T,C/128] ->
    (qT [C,T], sT [C,T/128]).  Parity unpinned beyond shared invariants."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s_row = np.ascontiguousarray(s_row, dtype=np.float32)
    T, C = q.shape
    assert T % GROUP == 0 and C % GROUP == 0 and s_row.shape == (T, C // GROUP)
    qT = np.empty((C, T), np.uint8)
    sT = np.empty((C, T // GROUP), np.float32)
    lib().oracle_quant_transpose_fp8(_ptr(q, ctypes.c_uint8), _ptr(s_row, ctypes.c_float), T, C,
                                     _ptr(qT, ctypes.c_uint8), _ptr(sT, ctypes.c_float))
    return qT, sT


# ----------------------------------------------------- producer operators

def rmsnorm_bf16(x_bf16: np.ndarray, gamma_bf16: np.ndarray, eps: float):
    """RMSNorm of bf16 rows: x [M,K], gamma [K] -> (y bf16 bits [M,K], rstd f32 [M]).

    fp64 sum of squares (tree per 128-group, groups ascending), r = 1/sqrt(ss/K + eps)
    in fp64, rstd = fp32(r), y = bf16(fp32(fp32(x * rstd) * gamma))."""
    x = _bits16(x_bf16)
    g = _bits16(gamma_bf16)
    M, K = x.shape
    assert K % GROUP == 0 and g.shape == (K,)
    y = np.empty((M, K), np.uint16)
    r = np.empty((M,), np.float32)
    lib().oracle_rmsnorm_bf16(_ptr(x, ctypes.c_uint16), _ptr(g, ctypes.c_uint16), M, K, float(eps),
                              _ptr(y, ctypes.c_uint16), _ptr(r, ctypes.c_float))
    return y, r


def swiglu_bf16(gate_bf16: np.ndarray, up_bf16: np.ndarray):
    """SwiGLU of bf16 tensors [M,F]: h = bf16(silu(g) * u), evaluated in fp64.

    Returns (h bf16 bits [M,F], near_tie bool [M,F]); near_tie marks elements
    whose fp64 value lies within 2^-44 (relative) of a bf16 rounding midpoint,
    where either bf16 neighbour is a correct result."""
    g = _bits16(gate_bf16)
    u = _bits16(up_bf16)
    assert g.shape == u.shape and g.ndim == 2
    M, F = g.shape
    h = np.empty((M, F), np.uint16)
    t = np.empty((M, F), np.uint8)
    lib().oracle_swiglu_bf16(_ptr(g, ctypes.c_uint16), _ptr(u, ctypes.c_uint16), F, M, F,
                             _ptr(h, ctypes.c_uint16), _ptr(t, ctypes.c_uint8))
    return h, t.astype(bool)


def rmsnorm_bwd(x_bf16: np.ndarray, gamma_bf16: np.ndarray, rstd: np.ndarray, dy_bf16: np.ndarray):
    """RMSNorm backward: x, dy bf16 [M,K], gamma bf16 [K], rstd f32 [M] (the
    forward's) -> (dx bf16 bits [M,K], dgamma f32 [K]), fp64 in a fixed order."""
    x, g, d = _bits16(x_bf16), _bits16(gamma_bf16), _bits16(dy_bf16)
    r = np.ascontiguousarray(rstd, dtype=np.float32)
    M, K = x.shape
    assert K % GROUP == 0 and g.shape == (K,) and d.shape == (M, K) and r.shape == (M,)
    dx = np.empty((M, K), np.uint16)
    dg = np.empty((K,), np.float32)
    lib().oracle_rmsnorm_bwd(_ptr(x, ctypes.c_uint16), _ptr(g, ctypes.c_uint16), _ptr(r, ctypes.c_float),
                             _ptr(d, ctypes.c_uint16), M, K, _ptr(dx, ctypes.c_uint16), _ptr(dg, ctypes.c_float))
    return dx, dg


def swiglu_bwd_bf16(gate_bf16: np.ndarray, up_bf16: np.ndarray, dh_bf16: np.ndarray):
    """Backward of h = silu(g) * u for bf16 [M,F] g, u and dh, evaluated in fp64:
    returns (dgu bf16 bits [M,2F] = [d_gate | d_up], near_tie bool [M,2F])."""
    g, u, d = _bits16(gate_bf16), _bits16(up_bf16), _bits16(dh_bf16)
    assert g.shape == u.shape == d.shape and g.ndim == 2
    M, F = g.shape
    out = np.empty((M, 2 * F), np.uint16)
    t = np.empty((M, 2 * F), np.uint8)
    lib().oracle_swiglu_bwd_bf16(_ptr(g, ctypes.c_uint16), _ptr(u, ctypes.c_uint16), _ptr(d, ctypes.c_uint16),
                                 F, M, F, _ptr(out, ctypes.c_uint16), _ptr(t, ctypes.c_uint8))
    return out, t.astype(bool)


def rmsnorm_quant(x_bf16: np.ndarray, gamma_bf16: np.ndarray, eps: float):
    """RMSNorm followed by 1x128 quantization of its bf16 output:
    -> (q u8 [M,K], s f32 [M,K/128], rstd f32 [M])."""
    y, r = rmsnorm_bf16(x_bf16, gamma_bf16, eps)
    q, s = quant_act(y)
    return q, s, r


def swiglu_quant(gate_bf16: np.ndarray, up_bf16: np.ndarray):
    """SwiGLU followed by 1x128 quantization of its bf16 output:
    -> (q u8 [M,F], s f32 [M,F/128], near_tie bool [M,F])."""
    h, t = swiglu_bf16(gate_bf16, up_bf16)
    q, s = quant_act(h)
    return q, s, t


# ------------------------------------------------------------- dequantize

def dequant_rowgroup(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    R, C = q.shape
    assert s.shape == (R, C // GROUP)
    out = np.empty((R, C), np.float64)
    lib().oracle_dequant_rowgroup(_ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float), R, C,
                                  _ptr(out, ctypes.c_double))
    return out


def dequant_block(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    R, C = q.shape
    assert s.shape == (R // GROUP, C // GROUP)
    out = np.empty((R, C), np.float64)
    lib().oracle_dequant_block(_ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float), R, C,
                               _ptr(out, ctypes.c_double))
    return out


# ------------------------------------------------------------------- GEMM

def gemm(A: np.ndarray, B: np.ndarray, a_trans: bool = False, b_trans: bool = False) -> np.ndarray:
    """fp64 C[m,n] = sum_k A(m,k) B(n,k), ascending k.

    A is [M,K] (or [K,M] with a_trans), B is [N,K] (or [K,N] with b_trans);
    transposition is expressed with strides, no data is moved."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    if a_trans:
        K, M = A.shape
        sam, sak = 1, M
    else:
        M, K = A.shape
        sam, sak = K, 1
    if b_trans:
        K2, N = B.shape
        sbn, sbk = 1, N
    else:
        N, K2 = B.shape
        sbn, sbk = K2, 1
    assert K == K2
    C = np.empty((M, N), np.float64)
    lib().oracle_gemm(M, N, K, _ptr(A, ctypes.c_double), sam, sak, _ptr(B, ctypes.c_double),
                      sbn, sbk, _ptr(C, ctypes.c_double))
    return C


def gemm_fwd(xq, sx, wq, sw) -> np.ndarray:
    """Forward / rollout: Y[m,n] = sum_k dec(Xq)sx * dec(Wq)sw (fp64)."""
    return gemm(dequant_rowgroup(xq, sx), dequant_block(wq, sw))


def gemm_dgrad(dyq, sdy, wq, sw) -> np.ndarray:
    """DGrad: dX[t,k] = sum_n dec(dYq)sdy * dec(Wq)sw, contraction over W's rows."""
    return gemm(dequant_rowgroup(dyq, sdy), dequant_block(wq, sw), b_trans=True)


def gemm_wgrad(dyTq, sdyT, xTq, sxT) -> np.ndarray:
    """WGrad: dW[n,k] = sum_t dec(dY^T q)sdyT * dec(X^T q)sxT, groups along T."""
    return gemm(dequant_rowgroup(dyTq, sdyT), dequant_rowgroup(xTq, sxT))


def gemm_metric(c_gpu: np.ndarray, c_ref: np.ndarray, rms_ref: float | None = None) -> float:
    """max |C_gpu - C_ref| / (|C_ref| + 0.01 * rms(C_ref)); pass if <= 1e-2."""
    c_ref = np.asarray(c_ref, dtype=np.float64)
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    if c_ref.size == 0:
        return 0.0
    if rms_ref is None:
        rms_ref = float(np.sqrt(np.mean(c_ref * c_ref)))
    den = np.abs(c_ref) + 0.01 * rms_ref
    num = np.abs(c_gpu - c_ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(num == 0, 0.0, num / den)
    return float(np.max(r))


# ------------------------------------------------------ 4-bit weights (MXFP4)

MX_BLOCK = 32


def e2m1_decode(codes) -> np.ndarray:
    """fp64 values of 4-bit E2M1 codes (0..15)."""
    L = lib()
    table = np.array([L.oracle_e2m1_decode(i) for i in range(16)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def mxfp4_quant(w_bf16: np.ndarray):
    """MXFP4 weight quant (OCP MX v1.0 reading of QeRL's 4-bit weights):
    w [N,K] bf16 bits -> (codes u8 [N,K/2], two per byte, even k in the low
    nibble; scales u8 [N,K/32], E8M0 = E + 127)."""
    w = _bits16(w_bf16)
    N, K = w.shape
    assert K % MX_BLOCK == 0
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // MX_BLOCK), np.uint8)
    lib().oracle_mxfp4_quant(_ptr(w, ctypes.c_uint16), N, K, _ptr(codes, ctypes.c_uint8),
                             _ptr(scales, ctypes.c_uint8))
    return codes, scales


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N, K2 = codes.shape
    K = 2 * K2
    assert scales.shape == (N, K // MX_BLOCK)
    out = np.empty((N, K), np.float64)
    lib().oracle_dequant_mxfp4(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), N, K,
                               _ptr(out, ctypes.c_double))
    return out


def gemm_fwd_w4(xq, sx, w4, s4) -> np.ndarray:
    """4-bit-weight rollout GEMM: Y[m,n] = sum_k dec(Xq)sx * e2m1(W4) 2^E (fp64)."""
    return gemm(dequant_rowgroup(xq, sx), dequant_mxfp4(w4, s4))


def num_threads() -> int:
    return int(lib().oracle_num_threads())
