"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no part of the method's arithmetic (no amax, scale, encode
or GEMM); it only draws tensors.  Both the CPU oracle and the HIP path receive
the very same bf16 bit patterns from here.

Recipe (per tensor): ``numpy.random.Generator(PCG64(SeedSequence([seed, tid])))``
with tid 1 for X, 2 for W, 3 for dY and 4 for the outlier-column draw;
``standard_normal(float32) * sigma``; outlier columns of X are multiplied by 50;
fp32 -> bf16 with round-to-nearest-even on the host.

The workloads stand in for the models the Jet-RL summary evaluates (Llama3.1-8B,
Qwen2.5-7B, Qwen3-8B-Base, and 32B-class rollouts): only their MLP shapes are
used, with Gaussian activations carrying a few outlier channels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TID_X, TID_W, TID_DY, TID_OUTLIER, TID_NORM = 1, 2, 3, 4, 5


def rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.  Inputs are
    finite Gaussian draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def n_outliers(K: int) -> int:
    """0.1 % of the channels, at least one."""
    return max(1, int(round(0.001 * K)))


def gaussian_bf16(shape, sigma: float, seed: int, tid: int,
                  outlier_cols: np.ndarray | None = None, outlier_mult: float = 50.0) -> np.ndarray:
    g = rng(seed, tid)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    if outlier_cols is not None and len(outlier_cols):
        a[..., outlier_cols] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(a)


def outlier_columns(K: int, n: int, seed: int) -> np.ndarray:
    return np.sort(rng(seed, TID_OUTLIER).choice(K, size=n, replace=False))


def activations(M: int, K: int, seed: int = 0, n_out: int | None = None) -> np.ndarray:
    """X ~ N(0,1) [M,K] with outlier columns x50, as bf16 bits."""
    n = n_outliers(K) if n_out is None else n_out
    return gaussian_bf16((M, K), 1.0, seed, TID_X, outlier_columns(K, n, seed))


def weights(N: int, K: int, seed: int = 0, sigma: float = 0.02) -> np.ndarray:
    """W ~ N(0, 0.02) [N,K] as bf16 bits."""
    return gaussian_bf16((N, K), sigma, seed, TID_W)


def norm_weights(K: int, seed: int = 0, sigma: float = 0.1) -> np.ndarray:
    """RMSNorm gain gamma ~ 1 + N(0, 0.1) [K] as bf16 bits."""
    g = rng(seed, TID_NORM)
    a = np.float32(1.0) + g.standard_normal(size=(K,), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(a)


def grad_out(T: int, N: int, seed: int = 0, sigma: float = 1e-3) -> np.ndarray:
    """dY ~ N(0, 1e-3) [T,N] as bf16 bits."""
    return gaussian_bf16((T, N), sigma, seed, TID_DY)


def random_codes(shape, seed: int, tid: int) -> np.ndarray:
    """Uniform random finite E4M3 codes (the two NaN codes 0x7F/0xFF excluded)."""
    c = rng(seed, tid).integers(0, 254, size=shape, dtype=np.int64)
    c = c + (c >= 0x7F)                     # skip 0x7F
    return c.astype(np.uint8)


def random_scales(shape, seed: int, tid: int, lo: float = 1e-3, hi: float = 2e-2) -> np.ndarray:
    """Positive fp32 scales drawn uniformly from [lo, hi)."""
    return (lo + (hi - lo) * rng(seed, tid).random(size=shape)).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "forward", "backward", "producers", "mlp" or "mlp_train"
    # mlp: M tokens, N intermediate width F, K hidden width
    M: int             # tokens (T for backward)
    N: int
    K: int
    n_out: int         # outlier columns in X
    doc: str


WORKLOADS = {
    "tiny": Workload("tiny", "forward", 128, 1024, 1024, 4,
                     "forward quantized linear, X[128,1024] W[1024,1024]"),
    "decode": Workload("decode", "forward", 64, 14336, 4096, n_outliers(4096),
                       "8B-shaped MLP up-proj decode step, X[64,4096] W[14336,4096] pre-quantized"),
    "w4_decode": Workload("w4_decode", "forward", 64, 14336, 4096, n_outliers(4096),
                          "8B-shaped MLP up-proj rollout decode step on 4-bit MXFP4 weights, X[64,4096] FP8 1x128, "
                          "W[14336,4096] MXFP4 pre-quantized"),
    "decode_unified": Workload("decode_unified", "forward", 64, 14336, 4096, n_outliers(4096),
                               "8B-shaped MLP up-proj decode step on the unified kernel (rows bit-identical to "
                               "training-sized calls), X[64,4096] W[14336,4096] pre-quantized"),
    "prefill": Workload("prefill", "forward", 8192, 18944, 3584, n_outliers(3584),
                        "7B-shaped MLP prefill/actor forward, X[8192,3584] W[18944,3584]"),
    "backward": Workload("backward", "backward", 8192, 14336, 4096, n_outliers(4096),
                         "8B-shaped MLP backward, dY[8192,14336] X[8192,4096] W[14336,4096]"),
    "large": Workload("large", "forward", 16384, 27648, 5120, n_outliers(5120),
                      "32B-shaped MLP forward, X[16384,5120] W[27648,5120]"),
    "mlp": Workload("mlp", "mlp", 8192, 14336, 4096, n_outliers(4096),
                    "8B-shaped FP8 MLP block forward on 8192 tokens: RMSNorm->FP8, gate/up GEMM [28672,4096], "
                    "SwiGLU->FP8, down GEMM [4096,14336]"),
    "mlp_decode": Workload("mlp_decode", "mlp", 64, 14336, 4096, n_outliers(4096),
                           "8B-shaped FP8 MLP block rollout decode step on 64 tokens: RMSNorm->FP8, gate/up GEMM "
                           "[28672,4096], SwiGLU->FP8, down GEMM [4096,14336], weights pre-quantized and packed"),
    "mlp_train": Workload("mlp_train", "mlp_train", 8192, 14336, 4096, n_outliers(4096),
                          "8B-shaped FP8 MLP block training step on 8192 tokens: weight re-quantization from BF16 "
                          "masters (with transposed copies), forward (RMSNorm->FP8, gate/up "
                          "GEMM, SwiGLU->FP8, down GEMM) and backward through the three linear layers (dual "
                          "transpose-quant of dY, FP8-source requant of H and X, SwiGLU backward fused with the "
                          "dual quantization of its result, two DGrad and two WGrad GEMMs, RMSNorm backward)"),
    "producers": Workload("producers", "producers", 8192, 14336, 4096, n_outliers(4096),
                          "8B-shaped producers fused with 1x128 quantization: RMSNorm of X[8192,4096], "
                          "SwiGLU of the gate/up halves of one [8192,2x14336] projection output"),
}
