"""Pins of the oracle's fp64 block-scaled GEMMs (forward, DGrad, WGrad):
exact rationals on tiny shapes, numpy's float64 matmul, one-hot decoding of
every code, permutation closed forms, and lossless-quantization exact cases."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic

G = 128


def lib_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def close_to_matmul(C, A, B):
    """|C - A@B| within the fp64 summation bound (K+1) 2^-52 sum|a||b|."""
    K = A.shape[1]
    bound = (K + 1) * 2.0 ** -52 * (np.abs(A) @ np.abs(B))
    return np.all(np.abs(C - A @ B) <= bound)


def finite_codes(g, shape):
    c = g.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def rand_scales(g, shape):
    return (g.random(shape) * 0.02 + 1e-4).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 3, 256), (3, 2, 384)])
def test_fwd_exact_rationals(M, N, K):
    """Brute force in exact rational arithmetic (no rounding at all)."""
    g = np.random.default_rng(M * 100 + N * 10 + K)
    xq, wq = finite_codes(g, (M, K)), finite_codes(g, (128, K))
    sx, sw = rand_scales(g, (M, K // G)), rand_scales(g, (1, K // G))
    C = oracle.gemm_fwd(xq, sx, wq, sw)
    dx, dw = lib_decode(xq), lib_decode(wq)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(dx[m, k])) * Fraction(float(sx[m, k // G])) *
                        Fraction(float(dw[n, k])) * Fraction(float(sw[0, k // G])) for k in range(K))
            mag = sum(abs(Fraction(float(dx[m, k])) * Fraction(float(sx[m, k // G])) *
                          Fraction(float(dw[n, k])) * Fraction(float(sw[0, k // G]))) for k in range(K))
            assert abs(Fraction(C[m, n]) - exact) <= mag * Fraction(K + 1, 2 ** 52)


@pytest.mark.parametrize("M,N,K", [(7, 128, 128), (64, 256, 512), (129, 384, 256)])
def test_fwd_matches_numpy_matmul(M, N, K):
    """numpy's float64 matmul (BLAS) on operands dequantized with a library
    decoder and numpy broadcasting."""
    g = np.random.default_rng(M + N + K)
    xq, wq = finite_codes(g, (M, K)), finite_codes(g, (N, K))
    sx, sw = rand_scales(g, (M, K // G)), rand_scales(g, (N // G, K // G))
    C = oracle.gemm_fwd(xq, sx, wq, sw)
    A = lib_decode(xq) * np.repeat(sx.astype(np.float64), G, axis=1)
    B = lib_decode(wq) * np.repeat(np.repeat(sw.astype(np.float64), G, axis=0), G, axis=1)
    assert close_to_matmul(C, A, B.T)


def test_dgrad_wgrad_match_numpy_matmul():
    g = np.random.default_rng(5)
    T, N, K = 256, 384, 256
    dyq, sdy = finite_codes(g, (T, N)), rand_scales(g, (T, N // G))
    wq, sw = finite_codes(g, (N, K)), rand_scales(g, (N // G, K // G))
    dX = oracle.gemm_dgrad(dyq, sdy, wq, sw)
    A = lib_decode(dyq) * np.repeat(sdy.astype(np.float64), G, axis=1)
    B = lib_decode(wq) * np.repeat(np.repeat(sw.astype(np.float64), G, axis=0), G, axis=1)
    assert close_to_matmul(dX, A, B)
    dyTq, sdyT = finite_codes(g, (N, T)), rand_scales(g, (N, T // G))
    xTq, sxT = finite_codes(g, (K, T)), rand_scales(g, (K, T // G))
    dW = oracle.gemm_wgrad(dyTq, sdyT, xTq, sxT)
    A = lib_decode(dyTq) * np.repeat(sdyT.astype(np.float64), G, axis=1)
    B = lib_decode(xTq) * np.repeat(sxT.astype(np.float64), G, axis=1)
    assert close_to_matmul(dW, A, B.T)


def test_one_hot_decodes_every_code():
    """X = one-hot rows, W holds every finite code: Y reproduces each code's
    value exactly (pins decoding, subnormals included)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 codes
    N, K = 256, 256
    wq = np.zeros((N, K), np.uint8)
    wq[: codes.size, 0] = codes
    sw = np.ones((N // G, K // G), np.float32)
    xq = np.zeros((1, K), np.uint8)
    xq[0, 0] = 0x38                      # 1.0
    sx = np.ones((1, K // G), np.float32)
    y = oracle.gemm_fwd(xq, sx, wq, sw)[0, : codes.size]
    assert np.array_equal(y, lib_decode(codes))


def test_dgrad_permutation_closed_form():
    """W = a permutation matrix in 128x128 blocks with power-of-two block
    scales: dX = dY W is dY with permuted, exactly rescaled columns."""
    g = np.random.default_rng(8)
    T, N = 129, 256
    K = N
    perm = g.permutation(N)
    wq = np.zeros((N, K), np.uint8)
    wq[np.arange(N), perm] = 0x38                                   # 1.0
    sw = (2.0 ** g.integers(-3, 4, size=(N // G, K // G))).astype(np.float32)
    dyq, sdy = finite_codes(g, (T, N)), rand_scales(g, (T, N // G))
    dX = oracle.gemm_dgrad(dyq, sdy, wq, sw)
    dy = lib_decode(dyq) * np.repeat(sdy.astype(np.float64), G, axis=1)
    expect = np.zeros((T, K))
    for n in range(N):
        expect[:, perm[n]] = dy[:, n] * float(sw[n // G, perm[n] // G])
    assert np.array_equal(dX, expect)


def test_lossless_quantization_reproduces_bf16_product():
    """Inputs whose groups hold +-448*2^e and otherwise E4M3 values times 2^e
    quantize losslessly; quantize -> GEMM then equals the exact product of the
    BF16 inputs, and its bf16 rounding matches the rounding of the exact
    rational result."""
    g = np.random.default_rng(21)
    M, N, K = 3, 128, 256
    mags = lib_decode(np.arange(0, 127, dtype=np.uint8))

    def lossless(rows, cols, block):
        v = g.choice(mags, size=(rows, cols)) * np.where(g.random((rows, cols)) < .5, -1.0, 1.0)
        e = g.integers(-6, 6, size=(rows // block[0] + 1, cols // G + 1))
        for r in range(rows):
            for c0 in range(0, cols, G):
                if r % block[0] == 0:
                    v[r, c0 + g.integers(0, G)] = 448.0
                v[r, c0:c0 + G] *= 2.0 ** e[r // block[0], c0 // G]
        return v

    x = lossless(M, K, (1, G))
    w = lossless(N, K, (G, G))
    xb, wb = synthetic.f32_to_bf16_bits(x), synthetic.f32_to_bf16_bits(w)
    assert np.array_equal(synthetic.bf16_bits_to_f32(xb), x.astype(np.float32))
    xq, sx = oracle.quant_act(xb)
    wq, sw = oracle.quant_weight(wb)
    C = oracle.gemm_fwd(xq, sx, wq, sw)
    for m in range(M):
        for n in range(0, N, 17):
            exact = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(K))
            assert Fraction(C[m, n]) == exact            # small integers x 2^e: fp64-exact
    ref_bits = oracle.f64_to_bf16(C)
    exact_bits = torch.from_numpy(C.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ref_bits.view(np.int16), exact_bits)


def test_gemm_metric_definition():
    ref = np.array([[1.0, -2.0], [0.0, 4.0]])
    rms = np.sqrt(np.mean(ref ** 2))
    gpu = ref.copy()
    assert oracle.gemm_metric(gpu, ref) == 0.0
    gpu[1, 0] = 0.01 * 0.01 * rms                     # error relative to 0.01*rms only
    assert abs(oracle.gemm_metric(gpu, ref) - 0.01) < 1e-12
    gpu = ref * (1 + 0.02)
    assert abs(oracle.gemm_metric(gpu, ref) - 0.02 * 4 / (4 + 0.01 * rms)) < 1e-12
