"""Pins of the oracle's 4-bit MXFP4 weight format and the GEMM on it.

The QeRL page ("QeRL: Beyond Efficiency -- Quantization-enhanced Reinforcement
Learning for LLMs", abstract) gives its rollout weights as 4-bit NVFP4 and no
format details; the oracle reads them as OCP MXFP4 (E2M1 elements, 32
per block along K, one E8M0 power-of-two scale per block, scale exponent
floor(log2(amax)) - 2, round to nearest with ties to even, saturation at 6).
Each test checks the oracle against something other than itself: the value
table of the element format, exact rational arithmetic, closed-form cases and
the rounding error bound.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic

# E2M1 magnitudes for codes 0..7 (OCP MX v1.0 element table)
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
        Fraction(6)]


def bf16(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def bf16_value(bits):
    return Fraction(float((np.uint32(bits) << np.uint32(16)).view(np.float32)))


def code_of(codes, n, k):
    byte = int(codes[n, k // 2])
    return byte & 15 if k % 2 == 0 else byte >> 4


def brute_block(vals):
    """(E, codes) of one 32-block by exact rationals: E = largest e with
    2^e <= amax, minus 2, clamped; each code the nearest E2M1 value to v/2^E,
    ties to the even code, sign kept."""
    amax = max(abs(v) for v in vals)
    if amax == 0:
        E = -127
    else:
        e = 0
        while Fraction(2) ** e > amax:
            e -= 1
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        E = min(max(e - 2, -127), 127)
    out = []
    for v in vals:
        q = abs(v) / Fraction(2) ** E
        best = min(range(8), key=lambda c: (abs(q - E2M1[c]), c & 1))
        neg = v < 0 or (v == 0 and math.copysign(1.0, float(v)) < 0)
        out.append(best | (8 if neg else 0))
    return E, out


def check_against_brute(w_bits):
    codes, scales = oracle.mxfp4_quant(w_bits)
    N, K = w_bits.shape
    for n in range(N):
        for b in range(K // 32):
            vals = [bf16_value(w_bits[n, 32 * b + i]) for i in range(32)]
            # keep the sign of negative zeros (Fraction drops it)
            E, want = brute_block(vals)
            for i in range(32):
                if w_bits[n, 32 * b + i] == 0x8000:
                    want[i] = 8
            assert scales[n, b] == E + 127, (n, b, scales[n, b], E)
            got = [code_of(codes, n, 32 * b + i) for i in range(32)]
            assert got == want, (n, b, got, want)


def test_e2m1_value_table():
    got = oracle.e2m1_decode(np.arange(16))
    want = [float(v) for v in E2M1] + [-float(v) for v in E2M1]
    assert got.tolist() == want
    assert math.copysign(1.0, got[8]) < 0


def test_quant_matches_exact_rationals_random():
    rng = np.random.default_rng(3)
    rows = []
    for scale in (1e-3, 0.02, 1.0, 37.0, 3e4):
        rows.append(rng.normal(0, scale, 128))
    r = rng.normal(0, 1, 128)
    r[rng.random(128) < 0.2] = 0.0
    rows.append(r)
    rows.append(rng.uniform(-1, 1, 128) * 2.0 ** rng.integers(-20, 20, 128))
    check_against_brute(bf16(np.stack(rows)))


def test_every_midpoint_ties_to_even():
    # amax = 4 * 2^E fixes E; the other elements sit on the seven midpoints
    E = -3
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]
    row = np.zeros(32, np.float64)
    row[0] = 4.0
    for i, m in enumerate(mids):
        row[1 + i] = m
        row[9 + i] = -m
    w = bf16(row * 2.0 ** E)[None, :]
    codes, scales = oracle.mxfp4_quant(w)
    assert scales[0, 0] == E + 127
    assert code_of(codes, 0, 0) == 6
    for i, c in enumerate(want):
        assert code_of(codes, 0, 1 + i) == c, mids[i]
        assert code_of(codes, 0, 9 + i) == (c | 8), -mids[i]
    check_against_brute(w)


def test_saturation_and_block_maximum():
    # amax in [4, 8) * 2^E: 7.5 and 6.5 saturate to 6, 5.5 rounds to 6
    w = bf16(np.array([7.5, 6.5, 5.5, -7.75, 1.0] + [0.0] * 27) * 2.0 ** 5)[None, :]
    codes, scales = oracle.mxfp4_quant(w)
    assert scales[0, 0] == 5 + 127
    assert [code_of(codes, 0, k) for k in range(5)] == [7, 7, 7, 15, 2]


def test_zero_and_negative_zero_blocks():
    w = np.zeros((2, 64), np.uint16)
    w[1, ::3] = 0x8000
    codes, scales = oracle.mxfp4_quant(w)
    assert (scales == 0).all()                       # E = -127
    assert all(code_of(codes, 0, k) == 0 for k in range(64))
    assert all(code_of(codes, 1, k) == (8 if k % 3 == 0 else 0) for k in range(64))


def test_scale_exponent_clamps_at_e8m0_minimum():
    # amax = 2^-133 (a bf16 subnormal): floor(log2) - 2 = -135 -> -127
    w = np.zeros((1, 32), np.uint16)
    w[0, 0] = 0x0001                                 # 2^-133
    w[0, 1] = 0x0040                                 # 2^-127
    codes, scales = oracle.mxfp4_quant(w)
    assert scales[0, 0] == 0
    # 2^-127 / 2^-127 = 1 -> code 2; 2^-133 / 2^-127 = 2^-6 -> 0
    assert code_of(codes, 0, 1) == 2 and code_of(codes, 0, 0) == 0
    check_against_brute(w)


def test_largest_bf16_block():
    w = bf16(np.array([3.0e38, -1.0e38] + [1.0] * 30, np.float32))[None, :]
    codes, scales = oracle.mxfp4_quant(w)
    E = int(scales[0, 0]) - 127
    assert E == math.frexp(float(bf16_value(w[0, 0])))[1] - 1 - 2 == 125
    check_against_brute(w)


def test_nibble_order():
    row = np.zeros(32)
    row[0], row[3] = 1.0, -3.0
    row[31] = 4.0                                    # E = 0
    codes, scales = oracle.mxfp4_quant(bf16(row)[None, :])
    assert codes[0, 0] == 0x02                       # k = 0 low, k = 1 high
    assert codes[0, 1] == 0xD0                       # k = 2 low (0), k = 3 high (-3 = 0xD)
    assert codes[0, 15] == 0x60                      # k = 31 high nibble (4 = code 6)


def test_dequant_error_bound():
    """|w - deq| <= half an E2M1 step times 2^E below 6*2^E; at most 2 * 2^E when
    saturated (|w| < 8 * 2^E)."""
    w = synthetic.weights(64, 512, seed=4)
    codes, scales = oracle.mxfp4_quant(w)
    deq = oracle.dequant_mxfp4(codes, scales)
    wf = (w.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127).repeat(32, axis=1)
    q = np.abs(wf) / X
    half_step = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    bound = np.where(q <= 6, half_step, 2.0) * X
    assert np.all(np.abs(wf - deq) <= bound)
    assert np.all(q < 8)                             # amax / 2^E < 8 by the scale rule
    # every block's amax lands in [4, 8) * 2^E
    amax = np.abs(wf).reshape(64, 16, 32).max(axis=2)
    ratio = amax / np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))


def test_gemm_w4_exact_small_case():
    """Dyadic operands whose products and sums are exact in fp64: the GEMM on
    dequantized operands equals the exact rational sum."""
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 256
    xq = rng.integers(0, 256, (M, K)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x38                   # no NaN codes
    sx = np.ldexp(1.0, rng.integers(-4, 4, (M, K // 128))).astype(np.float32)
    w4 = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    s4 = rng.integers(120, 134, (N, K // 32)).astype(np.uint8)
    y = oracle.gemm_fwd_w4(xq, sx, w4, s4)
    xdec = oracle.e4m3_decode(xq)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                c = int(w4[n, k // 2])
                c = c & 15 if k % 2 == 0 else c >> 4
                wv = E2M1[c & 7] * (-1 if c & 8 else 1) * Fraction(2) ** (int(s4[n, k // 32]) - 127)
                acc += Fraction(float(xdec[m, k])) * Fraction(float(sx[m, k // 128])) * wv
            assert Fraction(float(y[m, n])) == acc, (m, n)


def test_gemm_w4_close_to_bf16_product():
    """A quantization-error sanity bound: the 4-bit GEMM stays within the
    propagated half-step error of the product of the unquantized values."""
    M, N, K = 8, 32, 512
    x = synthetic.activations(M, K, seed=2, n_out=1)
    w = synthetic.weights(N, K, seed=2)
    xq, sx = oracle.quant_act(x)
    w4, s4 = oracle.mxfp4_quant(w)
    y = oracle.gemm_fwd_w4(xq, sx, w4, s4)
    xd = oracle.dequant_rowgroup(xq, sx)
    wf = (w.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    exact = xd @ wf.T
    wd = oracle.dequant_mxfp4(w4, s4)
    bound = np.abs(xd) @ np.abs(wf - wd).T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-12) + 1e-300)
