"""GPU parity of the forward GEMM on many-tile shapes (fp8_gemm_fwd above 64
rows: 128 x 128 tiles, more tiles than CUs) against the fp64 oracle: the
accuracy metric max |C - C_ref| / (|C_ref| + 0.01 rms(C_ref)) <= 1e-2 on
ragged and many-tile shapes (partial last row tile, N an odd multiple of 128),
exact cases bit for bit, power-of-two scale changes bit for bit, all-zero row
groups and weight blocks, row scales spanning 2^80, and the 32B shape's data
on sampled rows."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, bf16_to_dev, f32_to_dev, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
G = 128
TOL = 1e-2


def tiles(M, N):
    """Tiles of 256 x 256: every shape below has at least 256 of them, i.e.
    at least four times as many 128 x 128 tiles as the GPU has CUs."""
    return -(-M // 256) * -(-N // 256)


def codes_scales(shape_q, shape_s, seed, tid):
    return synthetic.random_codes(shape_q, seed, tid), synthetic.random_scales(shape_s, seed, tid + 100)


def rows_sample(M, n, seed):
    g = np.random.default_rng(seed)
    rows = set(g.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1}
    # rows of the last (ragged) tile and around tile edges
    rows |= {min(M - 1, 255), min(M - 1, 256), (M - 1) // 256 * 256}
    return np.array(sorted(rows))


def check_rows(y_dev, xq, sx, wq, sw, rows, what):
    yg = host(y_dev[torch.from_numpy(rows).to(DEV)])
    ref = oracle.gemm_fwd(xq[rows], sx[rows], wq, sw)
    err = oracle.gemm_metric(bf16_bits_to_f64(yg), ref)
    assert err <= TOL, "%s: metric %.3e" % (what, err)
    return err


@pytest.mark.parametrize("M,N,K", [(2048, 8192, 512), (4359, 4096, 384), (2000, 8320, 256), (1100, 16512, 1152),
                                   (300, 65536, 128)])
def test_large_random_codes_sampled(M, N, K):
    """Random codes over the whole E4M3 range and random scales; ragged M
    (partial last row tile), N an odd multiple of 128 (half-empty last column
    tile), K from one group to nine."""
    assert tiles(M, N) >= 256
    xq, sx = codes_scales((M, K), (M, K // G), M + 3 * K, 81)
    wq, sw = codes_scales((N, K), (N // G, K // G), N + 5 * K, 82)
    say("gemm_fwd many tiles", M, N, K)
    y = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    check_rows(y, xq, sx, wq, sw, rows_sample(M, 20, M + N), "large %dx%dx%d" % (M, N, K))


def test_large_rows_independent_of_call():
    """A row's bits do not depend on the rows it is computed with: 200 rows
    alone and inside a 2048-row call give the same output; repeated calls give
    the same bits."""
    M, N, K = 2048, 8192, 1024
    xq, sx = codes_scales((M, K), (M, K // G), 9, 83)
    wq, sw = codes_scales((N, K), (N // G, K // G), 10, 84)
    dw, dsw = u8_to_dev(wq), f32_to_dev(sw)
    say("gemm_fwd many tiles, row independence")
    y_big = host(fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), dw, dsw))
    y_small = host(fl.fp8_gemm_fwd(u8_to_dev(xq[:200]), f32_to_dev(sx[:200]), dw, dsw))
    assert np.array_equal(y_big[:200], y_small)
    assert np.array_equal(y_big, host(fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), dw, dsw)))


def test_large_exact_lossless_bitwise():
    """Lossless inputs (E4M3 values with +-448 in every group, so every scale
    is 1): all partial sums are exact in fp32 and the bf16 output equals the
    oracle's bit for bit."""
    g = np.random.default_rng(15)
    M, N, K = 1024, 16384, 512
    small = oracle.e4m3_decode(np.arange(0x30, 0x48, dtype=np.uint8))     # 0.5 .. 3.75
    x = g.choice(small, (M, K)) * np.where(g.random((M, K)) < .5, -1, 1)
    w = g.choice(small, (N, K)) * np.where(g.random((N, K)) < .5, -1, 1)
    x[:, ::G] = 448.0
    w[:, ::G] = 448.0
    xb, wb = synthetic.f32_to_bf16_bits(x), synthetic.f32_to_bf16_bits(w)
    say("gemm_fwd many tiles exact")
    xq, sx = fl.fp8_quant_act(bf16_to_dev(xb))
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(wb))
    y = host(fl.fp8_gemm_fwd(xq, sx, wq, sw))
    rows = rows_sample(M, 24, 3)
    oq, os_ = oracle.quant_act(xb[rows])
    wq2, sw2 = oracle.quant_weight(wb)
    ref = oracle.gemm_fwd(oq, os_, wq2, sw2)
    assert np.array_equal(ref, x[rows] @ w.T)
    assert np.array_equal(y[rows], oracle.f64_to_bf16(ref))


def test_large_power_of_two_scaling_is_exact():
    """Scaling all X scales by 2^3 and all W scales by 2^-1 scales Y by 4 bit
    for bit."""
    M, N, K = 2048, 8192, 512
    xq, sx = codes_scales((M, K), (M, K // G), 1, 85)
    wq, sw = codes_scales((N, K), (N // G, K // G), 2, 86)
    dx, dw = u8_to_dev(xq), u8_to_dev(wq)
    say("gemm_fwd many tiles pow2 scaling")
    y0 = host(fl.fp8_gemm_fwd(dx, f32_to_dev(sx), dw, f32_to_dev(sw)))
    y1 = host(fl.fp8_gemm_fwd(dx, f32_to_dev(sx * 8), dw, f32_to_dev(sw / 2)))
    assert np.array_equal(bf16_bits_to_f64(y1), bf16_bits_to_f64(y0) * 4)


def test_large_zero_groups_and_blocks():
    """All-zero row groups (scale 0, codes +-0, including a whole zero row and
    a row whose first groups are zero) and all-zero weight blocks; an all-zero
    row gives exact zeros."""
    M, N, K = 2048, 8192, 768
    xq, sx = codes_scales((M, K), (M, K // G), 3, 87)
    wq, sw = codes_scales((N, K), (N // G, K // G), 4, 88)
    r = np.random.default_rng(4)
    for m in r.choice(M, 300, replace=False):
        gz = r.choice(K // G, r.integers(1, K // G), replace=False)
        for g_ in gz:
            xq[m, g_ * G:(g_ + 1) * G] = np.where(r.random(G) < 0.5, 0x00, 0x80)
            sx[m, g_] = 0
    xq[7] = 0
    sx[7] = 0
    xq[300, :2 * G] = 0
    sx[300, :2] = 0
    for nb, g_ in [(3, 0), (3, 1), (40, 5), (63, 2)]:
        wq[nb * G:(nb + 1) * G, g_ * G:(g_ + 1) * G] = 0x80
        sw[nb, g_] = 0
    say("gemm_fwd many tiles zero groups")
    y = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    rows = np.array(sorted({7, 300} | set(rows_sample(M, 20, 5).tolist())))
    check_rows(y, xq, sx, wq, sw, rows, "zero groups")
    assert not host(y[7]).any()


def test_large_wide_scale_range():
    """Rows whose group scales span 2^80 (one group 2^40 up, the next 2^40
    down) still meet the metric: each group's partial sum is promoted with
    its own scale product."""
    M, N, K = 2048, 8192, 512
    xq, sx = codes_scales((M, K), (M, K // G), 5, 89)
    wq, sw = codes_scales((N, K), (N // G, K // G), 6, 90)
    wide = np.array([3, 260, 261, 1500, 2047])
    sx[wide, 0] *= np.float32(2.0 ** 40)
    sx[wide, 1] *= np.float32(2.0 ** -40)
    say("gemm_fwd many tiles wide scale range")
    y = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    rows = np.array(sorted(set(wide.tolist()) | {0, 255, 700, 1024}))
    check_rows(y, xq, sx, wq, sw, rows, "wide scale range")


def test_large_workload_data_sampled():
    """The 32B MLP shape's data (X with 5 outlier channels x50, W ~ N(0, 0.02))
    through the GPU quantizers and the forward GEMM, sampled rows."""
    M, N, K = 16384, 27648, 5120
    x = synthetic.activations(M, K, seed=0, n_out=synthetic.n_outliers(K))
    w = synthetic.weights(N, K, seed=0)
    say("gemm_fwd 32B data")
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    y = fl.fp8_gemm_fwd(xq, sx, wq, sw)
    rows = rows_sample(M, 16, 11)
    oq, os_ = oracle.quant_act(x[rows])
    owq, osw = oracle.quant_weight(w)
    del w
    yg = host(y[torch.from_numpy(rows).to(DEV)])
    err = oracle.gemm_metric(bf16_bits_to_f64(yg), oracle.gemm_fwd(oq, os_, owq, osw))
    assert err <= TOL, err
