"""GPU parity of the block-scaled FP8 GEMMs (forward, DGrad, WGrad) against the
fp64 CPU oracle.  Tolerance (stated by the project's definition of the layer):
max |C_gpu - C_ref| / (|C_ref| + 0.01 rms(C_ref)) <= 1e-2.  Exactly
representable cases must match the oracle's bf16 rounding bit for bit."""
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


def codes_scales(shape_q, shape_s, seed, tid):
    return synthetic.random_codes(shape_q, seed, tid), synthetic.random_scales(shape_s, seed, tid + 100)


def check_metric(y_gpu_bits, ref, what, rms=None):
    err = oracle.gemm_metric(bf16_bits_to_f64(y_gpu_bits), ref, rms)
    assert err <= TOL, "%s: metric %.3e > %.0e" % (what, err, TOL)
    return err


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (7, 256, 256), (64, 384, 1024), (65, 128, 512),
                                   (129, 256, 384), (300, 384, 1024), (1000, 256, 256)])
def test_fwd_random_codes(M, N, K):
    xq, sx = codes_scales((M, K), (M, K // G), M * 7 + K, 11)
    wq, sw = codes_scales((N, K), (N // G, K // G), N * 3 + K, 12)
    say("gemm_fwd", M, N, K)
    y = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    check_metric(host(y), oracle.gemm_fwd(xq, sx, wq, sw), "fwd %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(4359, 4096, 384), (4359, 4096, 128), (2048, 8192, 256)])
def test_fwd_many_tiles_sampled(M, N, K):
    """More 256x128 tiles than workgroups: each workgroup runs several tiles
    back to back with its step ring crossing tile boundaries (K/128 >= 2),
    or one tile each (K = 128); checked on sampled rows incl. the ragged tail."""
    xq, sx = codes_scales((M, K), (M, K // G), M + K, 41)
    wq, sw = codes_scales((N, K), (N // G, K // G), N + K, 42)
    say("gemm_fwd many tiles", M, N, K)
    y = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    rows = sampled_rows(M, n=24, seed=3)
    yg = host(y[torch.from_numpy(rows).to(DEV)])
    check_metric(yg, oracle.gemm_fwd(xq[rows], sx[rows], wq, sw), "fwd many tiles %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("N,K,T", [(4500, 2048, 256), (4500, 2048, 384)])
def test_wgrad_many_tiles_sampled(N, K, T):
    dyTq, sdyT = codes_scales((N, T), (N, T // G), N + T, 43)
    xTq, sxT = codes_scales((K, T), (K, T // G), K + T, 44)
    say("gemm_wgrad many tiles", N, K, T)
    dw = fl.fp8_gemm_wgrad(u8_to_dev(dyTq), f32_to_dev(sdyT), u8_to_dev(xTq), f32_to_dev(sxT))
    rows = sampled_rows(N, n=24, seed=4)
    dwg = host(dw[torch.from_numpy(rows).to(DEV)])
    check_metric(dwg, oracle.gemm_wgrad(dyTq[rows], sdyT[rows], xTq, sxT), "wgrad many tiles")


@pytest.mark.parametrize("M,N,K", [(1, 128, 512), (17, 256, 1024), (64, 384, 2048), (64, 128, 1536),
                                   (33, 128, 16384), (64, 256, 15872), (64, 512, 14336), (40, 128, 768),
                                   (64, 128, 256), (3, 256, 17408)])
def test_fwd_decode_shapes(M, N, K):
    """At most 64 rows: the streaming decode kernels (K/128 a multiple of 4 up
    to 128 groups), the K-split fallback and the generic tile, across group
    counts on both sides of each kernel's limits."""
    xq, sx = codes_scales((M, K), (M, K // G), M * 13 + K, 21)
    wq, sw = codes_scales((N, K), (N // G, K // G), N * 5 + K, 22)
    say("gemm_fwd decode shape", M, N, K)
    y = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    check_metric(host(y), oracle.gemm_fwd(xq, sx, wq, sw), "fwd %dx%dx%d" % (M, N, K))


def pack_reference(wq: np.ndarray) -> np.ndarray:
    """The decode layout written out from its definition: for each 64-row
    block, 256-column chunk, matrix wave w = ct + 2 kp + 4 kq, q and lane
    (m + 32 kh): the 16 codes of row 32 ct + m at chunk piece 8 kp + 4 kh + 2 kq + q."""
    N, K = wq.shape
    nch = K // 256
    out = np.empty(N * K, np.uint8)
    i = 0
    for nb in range(N // 64):
        for c in range(nch):
            for w in range(8):
                ct, kp, kq = w & 1, (w >> 1) & 1, w >> 2
                for q in range(2):
                    for lane in range(64):
                        m, kh = lane & 31, lane >> 5
                        pc = 8 * kp + 4 * kh + 2 * kq + q
                        out[i:i + 16] = wq[nb * 64 + 32 * ct + m, c * 256 + 16 * pc: c * 256 + 16 * pc + 16]
                        i += 16
    return out.reshape(N, K)


@pytest.mark.parametrize("N,K", [(128, 256), (256, 768)])
def test_weight_pack_layout(N, K):
    wq = synthetic.random_codes((N, K), N + K, 61)
    say("weight pack", N, K)
    assert np.array_equal(host(fl.fp8_weight_pack(u8_to_dev(wq))), pack_reference(wq))


@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (17, 256, 768), (64, 384, 2048), (33, 256, 3584),
                                   (64, 14336, 4096), (5, 128, 5120), (64, 512, 16384), (40, 128, 1024)])
def test_fwd_packed_matches_unpacked(M, N, K):
    """The decode kernel on the packed layout computes the same bits as the
    forward GEMM on the unpacked codes (unrolled widths 3584/4096/5120 and the
    run-time loop), and stays within the tolerance of the oracle."""
    xq, sx = codes_scales((M, K), (M, K // G), M * 5 + K, 62)
    wq, sw = codes_scales((N, K), (N // G, K // G), N * 3 + K, 63)
    say("gemm_fwd_packed", M, N, K)
    xd, sxd, wd, swd = u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw)
    y = host(fl.fp8_gemm_fwd_packed(xd, sxd, fl.fp8_weight_pack(wd), swd))
    assert np.array_equal(y, host(fl.fp8_gemm_fwd(xd, sxd, wd, swd)))
    if N * K <= 4096 * 4096:
        check_metric(y, oracle.gemm_fwd(xq, sx, wq, sw), "fwd packed %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(64, 4096, 14336), (64, 4096, 4096), (17, 1024, 2048), (1, 256, 4096),
                                   (64, 4096, 3584), (33, 512, 5120), (64, 14336, 4096)])
def test_fwd_packed_splitk(M, N, K):
    """The split-K decode GEMM: within the tolerance of the oracle (the 8B down
    projection 64x4096x14336 included, split ranges of unequal length at
    K = 3584), deterministic, rows bit-identical across batch sizes, and
    bit-identical to the unsplit kernel when no split is made (N >= 8192)."""
    xq, sx = codes_scales((M, K), (M, K // G), M * 7 + K, 64)
    wq, sw = codes_scales((N, K), (N // G, K // G), N * 5 + K, 65)
    say("gemm_fwd_packed_splitk", M, N, K)
    xd, sxd, wd, swd = u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw)
    wp = fl.fp8_weight_pack(wd)
    need = fl.fp8_gemm_fwd_packed_splitk_workspace(M, N, K)
    ws = torch.full((max(need // 4, 1),), float("nan"), dtype=torch.float32, device=DEV)   # contents ignored
    y = host(fl.fp8_gemm_fwd_packed_splitk(xd, sxd, wp, swd, workspace=ws))
    assert np.array_equal(y, host(fl.fp8_gemm_fwd_packed_splitk(xd, sxd, wp, swd, workspace=ws)))
    if need == 0:
        assert np.array_equal(y, host(fl.fp8_gemm_fwd_packed(xd, sxd, wp, swd)))
    rows = slice(M // 3, M // 3 + 1)
    y1 = host(fl.fp8_gemm_fwd_packed_splitk(xd[rows].contiguous(), sxd[rows].contiguous(), wp, swd))
    assert np.array_equal(y1, y[rows])
    if N * K <= 4096 * 14336:
        check_metric(y, oracle.gemm_fwd(xq, sx, wq, sw), "fwd packed split-K %dx%dx%d" % (M, N, K))
    if need > 0:
        with pytest.raises(fl.Fp8LinError, match="FP8LIN_ERR_ARG"):
            fl._check(fl.lib().fp8_gemm_fwd_packed_splitk(
                fl._ptr(xd), fl._ptr(sxd), fl._ptr(wp), fl._ptr(swd), M, N, K, fl._ptr(torch.empty_like(
                    torch.zeros((M, N), dtype=torch.bfloat16, device=DEV))), fl._ptr(ws), need - 4,
                fl._stream(None)), "splitk")


def test_fwd_one_hot_every_code():
    """Pins MFMA operand decoding and the fragment/output layouts: W holds every
    finite code once in column 0 of its group; X is one-hot at that column."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    N, K, M = 256, 256, 3
    wq = np.zeros((N, K), np.uint8)
    wq[: codes.size, 5] = codes
    wq[: codes.size, 130] = codes[::-1]
    sw = np.ones((N // G, K // G), np.float32)
    xq = np.zeros((M, K), np.uint8)
    xq[0, 5] = 0x38                               # 1.0
    xq[1, 130] = 0x38
    xq[2, 5] = 0x30                               # 0.5
    sx = np.ones((M, K // G), np.float32)
    say("gemm_fwd one-hot")
    y = host(fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw)))
    ref = oracle.f64_to_bf16(oracle.gemm_fwd(xq, sx, wq, sw))
    assert np.array_equal(y, ref)


def test_fwd_exact_lossless_bitwise():
    """Lossless-quantizing inputs (E4M3 values x 2^e per group, each group
    holding +-448 2^e): partial sums are small integers times a power of two,
    exact in fp32 in any order, so GPU and oracle bf16 bits must agree."""
    g = np.random.default_rng(5)
    M, N, K = 96, 256, 512
    small = oracle.e4m3_decode(np.arange(0x30, 0x48, dtype=np.uint8))     # 0.5 .. 3.75
    x = g.choice(small, (M, K)) * np.where(g.random((M, K)) < .5, -1, 1)
    w = g.choice(small, (N, K)) * np.where(g.random((N, K)) < .5, -1, 1)
    x[:, ::G] = 448.0
    w[:, ::G] = 448.0
    xb, wb = synthetic.f32_to_bf16_bits(x), synthetic.f32_to_bf16_bits(w)
    say("gemm_fwd exact")
    xq, sx = fl.fp8_quant_act(bf16_to_dev(xb))
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(wb))
    y = host(fl.fp8_gemm_fwd(xq, sx, wq, sw))
    oq, os_ = oracle.quant_act(xb)
    wq2, sw2 = oracle.quant_weight(wb)
    ref = oracle.gemm_fwd(oq, os_, wq2, sw2)
    assert np.array_equal(ref, x @ w.T)
    assert np.array_equal(y, oracle.f64_to_bf16(ref))


def test_fwd_end_to_end_tiny_config():
    """Forward quantized linear on the tiny config: X [128,1024] ~N(0,1) with 4
    outlier columns x50, W [1024,1024] ~N(0,0.02): GPU quantizers + GEMM vs the
    oracle chain."""
    x = synthetic.activations(128, 1024, seed=0, n_out=4)
    w = synthetic.weights(1024, 1024, seed=0)
    say("forward tiny end-to-end")
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    y = host(fl.fp8_gemm_fwd(xq, sx, wq, sw))
    ref = oracle.gemm_fwd(*oracle.quant_act(x), *oracle.quant_weight(w))
    check_metric(y, ref, "tiny end-to-end")


def test_fwd_degenerate():
    say("gemm_fwd degenerate")
    e = torch.empty((0, 256), dtype=torch.uint8, device=DEV)
    wq = u8_to_dev(synthetic.random_codes((128, 256), 0, 1))
    sw = f32_to_dev(np.ones((1, 2), np.float32))
    y = fl.fp8_gemm_fwd(e, torch.empty((0, 2), dtype=torch.float32, device=DEV), wq, sw)
    assert y.shape == (0, 128)
    xq = torch.empty((5, 0), dtype=torch.uint8, device=DEV)
    wq0 = torch.empty((128, 0), dtype=torch.uint8, device=DEV)
    y = fl.fp8_gemm_fwd(xq, torch.empty((5, 0), dtype=torch.float32, device=DEV), wq0,
                        torch.empty((1, 0), dtype=torch.float32, device=DEV),
                        out=torch.full((5, 128), 3.0, dtype=torch.bfloat16, device=DEV))
    assert torch.all(y == 0).item()


def test_fwd_power_of_two_scaling_is_exact():
    """Scaling all X scales by 2^i and all W scales by 2^j scales Y by 2^(i+j)
    bit for bit (no over/underflow here)."""
    M, N, K = 130, 256, 512
    xq, sx = codes_scales((M, K), (M, K // G), 1, 11)
    wq, sw = codes_scales((N, K), (N // G, K // G), 2, 12)
    say("gemm_fwd pow2 scaling")
    y0 = host(fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw)))
    y1 = host(fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx * 8), u8_to_dev(wq), f32_to_dev(sw / 2)))
    assert np.array_equal(bf16_bits_to_f64(y1), bf16_bits_to_f64(y0) * 4)


def test_fwd_rows_independent_of_batch():
    """A row's result does not depend on the other rows of the call: bit for
    bit among decode-sized calls (<= 64 rows) and among large calls; across
    the two kernels (different group summation order) within the metric."""
    M, N, K = 512, 256, 1024
    xq, sx = codes_scales((M, K), (M, K // G), 3, 11)
    wq, sw = codes_scales((N, K), (N // G, K // G), 4, 12)
    say("gemm_fwd batch invariance")
    run = lambda a, b: host(fl.fp8_gemm_fwd(u8_to_dev(xq[a:b]), f32_to_dev(sx[a:b]), u8_to_dev(wq), f32_to_dev(sw)))
    y_all = run(0, M)
    y_mid = run(100, 300)
    assert np.array_equal(y_mid, y_all[100:300])
    y_64 = run(128, 192)
    y_1 = run(130, 131)
    y_7 = run(125, 132)
    assert np.array_equal(y_1, y_64[2:3]) and np.array_equal(y_7[3:7], y_64[0:4])   # rows 128..131
    ref = oracle.gemm_fwd(xq[128:192], sx[128:192], wq, sw)
    check_metric(y_64, ref, "decode rows")
    assert oracle.gemm_metric(bf16_bits_to_f64(y_64), bf16_bits_to_f64(y_all[128:192])) <= TOL


def test_fwd_unified_rows_bitwise_across_batch_sizes():
    """fp8_gemm_fwd_unified: every row's bits are the same whether it is
    computed alone (rollout decode), in a decode-sized batch or in a large
    training batch, and equal to fp8_gemm_fwd's above 64 rows; the result meets
    the accuracy metric against the oracle."""
    M, N, K = 600, 512, 1536
    xq, sx = codes_scales((M, K), (M, K // G), 5, 13)
    wq, sw = codes_scales((N, K), (N // G, K // G), 6, 14)
    dw, dsw = u8_to_dev(wq), f32_to_dev(sw)
    run = lambda f, a, b: host(f(u8_to_dev(xq[a:b]), f32_to_dev(sx[a:b]), dw, dsw))
    say("gemm_fwd_unified batch invariance")
    y_all = run(fl.fp8_gemm_fwd, 0, M)                 # > 64 rows: the large kernel
    for a, b in ((0, M), (0, 1), (37, 38), (100, 107), (130, 194), (599, 600), (200, 265), (250, 600)):
        assert np.array_equal(run(fl.fp8_gemm_fwd_unified, a, b), y_all[a:b]), (a, b)
    check_metric(run(fl.fp8_gemm_fwd_unified, 130, 194), oracle.gemm_fwd(xq[130:194], sx[130:194], wq, sw),
                 "unified decode rows")


def test_fwd_unified_bitwise_full_decode_shape():
    """The 8B up-projection (N = 14336, K = 4096): rollout batches of 64 and 1
    rows on the 64 x 64 tiles give the bits of a 200-row call on the 128 x 128
    tiles."""
    M, N, K = 200, 14336, 4096
    xq, sx = codes_scales((M, K), (M, K // G), 7, 15)
    wq, sw = codes_scales((N, K), (N // G, K // G), 8, 16)
    dw, dsw = u8_to_dev(wq), f32_to_dev(sw)
    run = lambda a, b: host(fl.fp8_gemm_fwd_unified(u8_to_dev(xq[a:b]), f32_to_dev(sx[a:b]), dw, dsw))
    say("gemm_fwd_unified full decode shape")
    y_all = run(0, M)
    for a, b in ((0, 64), (64, 65), (136, 200), (199, 200)):
        assert np.array_equal(run(a, b), y_all[a:b]), (a, b)


@pytest.mark.parametrize("K", [128, 256, 384, 512, 640])
def test_fwd_unified_short_contractions(K):
    """The 64 x 64 tiles keep four steps in flight; with fewer groups than that
    (K = 128 .. 384) and on the last steps of a longer contraction, each step
    must still be waited for before it is read.  Ten repeated 64-row and 5-row
    calls give the bits of the 128 x 128 tiles' rows, with every call's output
    prefilled with a different pattern."""
    M, N = 192, 8192
    xq, sx = codes_scales((M, K), (M, K // G), K + 3, 17)
    wq, sw = codes_scales((N, K), (N // G, K // G), K + 4, 18)
    dw, dsw = u8_to_dev(wq), f32_to_dev(sw)
    say("gemm_fwd_unified short contraction K =", K)
    y_all = host(fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), dw, dsw))
    for a, b in ((64, 128), (100, 105)):
        xa, sa = u8_to_dev(xq[a:b]), f32_to_dev(sx[a:b])
        for rep in range(10):
            out = torch.full((b - a, N), float(rep - 5), dtype=torch.bfloat16, device=DEV)
            got = host(fl.fp8_gemm_fwd_unified(xa, sa, dw, dsw, out=out))
            assert np.array_equal(got, y_all[a:b]), (K, a, b, rep)


@pytest.mark.parametrize("kind,M,N,K", [("fwd", 64, 14336, 4096), ("fwd", 300, 1024, 1024),
                                        ("dgrad", 300, 1024, 512), ("wgrad", 512, 384, 1024)])
def test_gemm_deterministic(kind, M, N, K):
    """No atomics and a fixed summation order: repeated calls give the same
    bits (decode streaming kernel, NT tiles, DGrad and WGrad paths)."""
    a, sa = codes_scales((M, K), (M, K // G), M + N + K, 51)
    if kind == "fwd":
        b, sb = codes_scales((N, K), (N // G, K // G), N + K, 52)
        fn = fl.fp8_gemm_fwd
    elif kind == "dgrad":                       # dY [T=M, N=K here], W [K, N]
        b, sb = codes_scales((K, N), (K // G, N // G), N + K, 53)
        fn = fl.fp8_gemm_dgrad
    else:                                       # dY^T [M, T=K], X^T [N, T=K]
        b, sb = codes_scales((N, K), (N, K // G), N + K, 54)
        fn = fl.fp8_gemm_wgrad
    args = [u8_to_dev(a), f32_to_dev(sa), u8_to_dev(b), f32_to_dev(sb)]
    say("gemm determinism", kind, M, N, K)
    first = host(fn(*args))
    for _ in range(3):
        assert np.array_equal(host(fn(*args)), first)


# -------------------------------------------------------------------- DGrad

@pytest.mark.parametrize("T,N,K", [(1, 128, 128), (7, 256, 128), (64, 384, 256), (129, 256, 384),
                                   (300, 1024, 256)])
def test_dgrad_random_codes(T, N, K):
    dyq, sdy = codes_scales((T, N), (T, N // G), T + N, 21)
    wq, sw = codes_scales((N, K), (N // G, K // G), N + K, 22)
    say("gemm_dgrad", T, N, K)
    dx = fl.fp8_gemm_dgrad(u8_to_dev(dyq), f32_to_dev(sdy), u8_to_dev(wq), f32_to_dev(sw))
    check_metric(host(dx), oracle.gemm_dgrad(dyq, sdy, wq, sw), "dgrad %dx%dx%d" % (T, N, K))


def test_dgrad_permutation_exact():
    """W = a permutation in 128x128 blocks with power-of-two scales: dX is dY
    with permuted, rescaled columns, exactly."""
    g = np.random.default_rng(8)
    T, N = 200, 256
    perm = g.permutation(N)
    wq = np.zeros((N, N), np.uint8)
    wq[np.arange(N), perm] = 0x38
    sw = (2.0 ** g.integers(-3, 4, size=(N // G, N // G))).astype(np.float32)
    dyq = synthetic.random_codes((T, N), 5, 23)
    sdy = (2.0 ** g.integers(-8, 8, size=(T, N // G))).astype(np.float32)
    say("gemm_dgrad permutation")
    dx = host(fl.fp8_gemm_dgrad(u8_to_dev(dyq), f32_to_dev(sdy), u8_to_dev(wq), f32_to_dev(sw)))
    assert np.array_equal(dx, oracle.f64_to_bf16(oracle.gemm_dgrad(dyq, sdy, wq, sw)))


@pytest.mark.parametrize("T,N,K", [(5, 128, 256), (200, 256, 384), (1000, 512, 256)])
def test_dgrad_via_transposed_weight(T, N, K):
    """DGrad as the forward GEMM on fp8_weight_transpose's copy of W: the same
    sums as the oracle's DGrad (a6), and the copy itself is exactly W^T."""
    dyq, sdy = codes_scales((T, N), (T, N // G), T + N, 25)
    wq, sw = codes_scales((N, K), (N // G, K // G), N + K, 26)
    say("weight transpose + fwd as dgrad", T, N, K)
    wqT, swT = fl.fp8_weight_transpose(u8_to_dev(wq), f32_to_dev(sw))
    assert np.array_equal(host(wqT), wq.T) and np.array_equal(host(swT), sw.T)
    dx = fl.fp8_gemm_dgrad_t(u8_to_dev(dyq), f32_to_dev(sdy), wqT, swT)
    check_metric(host(dx), oracle.gemm_dgrad(dyq, sdy, wq, sw), "dgrad(wT) %dx%dx%d" % (T, N, K))
    same = fl.fp8_gemm_fwd(u8_to_dev(dyq), f32_to_dev(sdy), wqT, swT)
    assert np.array_equal(host(dx), host(same))


# -------------------------------------------------------------------- WGrad

@pytest.mark.parametrize("N,K,T", [(1, 1, 128), (5, 77, 256), (64, 128, 128), (130, 200, 384),
                                   (256, 384, 1024)])
def test_wgrad_random_codes(N, K, T):
    dyTq, sdyT = codes_scales((N, T), (N, T // G), N + T, 31)
    xTq, sxT = codes_scales((K, T), (K, T // G), K + T, 32)
    say("gemm_wgrad", N, K, T)
    dw = fl.fp8_gemm_wgrad(u8_to_dev(dyTq), f32_to_dev(sdyT), u8_to_dev(xTq), f32_to_dev(sxT))
    check_metric(host(dw), oracle.gemm_wgrad(dyTq, sdyT, xTq, sxT), "wgrad %dx%dx%d" % (N, K, T))


def test_wgrad_swap_roles_transposes():
    N, K, T = 192, 256, 512
    a, sa = codes_scales((N, T), (N, T // G), 9, 33)
    b, sb = codes_scales((K, T), (K, T // G), 10, 34)
    say("gemm_wgrad swap")
    d1 = host(fl.fp8_gemm_wgrad(u8_to_dev(a), f32_to_dev(sa), u8_to_dev(b), f32_to_dev(sb)))
    d2 = host(fl.fp8_gemm_wgrad(u8_to_dev(b), f32_to_dev(sb), u8_to_dev(a), f32_to_dev(sa)))
    err = oracle.gemm_metric(bf16_bits_to_f64(d2).T, bf16_bits_to_f64(d1))
    assert err <= TOL


def test_backward_end_to_end_small():
    """The backward flow on the GPU: dY -> dual quant (1x128 rows + 128-along-T
    transposed), saved FP8 X -> transpose-requant, DGrad and WGrad, against the
    oracle chain."""
    T, N, K = 256, 384, 256
    dy = synthetic.grad_out(T, N, seed=1)
    x = synthetic.activations(T, K, seed=1, n_out=1)
    w = synthetic.weights(N, K, seed=1)
    say("backward end-to-end small")
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    dyTq, sdyT, dyq, sdy = fl.fp8_quant_transpose(bf16_to_dev(dy), dual=True)
    xTq, sxT = fl.fp8_quant_transpose(xq, sx)
    dx = host(fl.fp8_gemm_dgrad(dyq, sdy, wq, sw))
    dw = host(fl.fp8_gemm_wgrad(dyTq, sdyT, xTq, sxT))
    owq, osw = oracle.quant_weight(w)
    oxq, osx = oracle.quant_act(x)
    check_metric(dx, oracle.gemm_dgrad(*oracle.quant_act(dy), owq, osw), "dX")
    check_metric(dw, oracle.gemm_wgrad(*oracle.quant_transpose_bf16(dy), *oracle.quant_transpose_fp8(oxq, osx)),
                 "dW")


# -------------------------------------------- full sizes, sampled rows

def sampled_rows(M, n=12, seed=0):
    g = np.random.default_rng(seed)
    rows = set(g.choice(M, size=min(n, M), replace=False).tolist())
    rows |= {0, M - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("name,M,N,K", [("decode 8B up-proj", 64, 14336, 4096),
                                        ("prefill 7B", 8192, 18944, 3584),
                                        ("large 32B", 16384, 27648, 5120)])
def test_fwd_full_size_sampled(name, M, N, K):
    """Full-size forward (GPU quantizers + GEMM, as timed by the bench), checked
    on sampled rows that the oracle computes one by one."""
    x = synthetic.activations(M, K, seed=0)
    w = synthetic.weights(N, K, seed=0)
    say("gemm_fwd full", name)
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    y = fl.fp8_gemm_fwd(xq, sx, wq, sw)
    rows = sampled_rows(M)
    yg = host(y[torch.from_numpy(rows).to(DEV)])
    if M <= 64:
        # the decode step as timed: packed weight layout
        yp = fl.fp8_gemm_fwd_packed(xq, sx, fl.fp8_weight_pack(wq), sw)
        assert np.array_equal(host(yp), host(y))
        del yp
    del y, xq, sx, wq, sw
    torch.cuda.empty_cache()
    oxq, osx = oracle.quant_act(x[rows])
    owq, osw = oracle.quant_weight(w)
    ref = oracle.gemm(oracle.dequant_rowgroup(oxq, osx), oracle.dequant_block(owq, osw))
    check_metric(yg, ref, name)


def test_backward_full_size_sampled():
    """8B-shaped backward (T=8192, N=14336, K=4096): DGrad rows and WGrad rows
    sampled against the oracle."""
    T, N, K = 8192, 14336, 4096
    dy = synthetic.grad_out(T, N, seed=0)
    x = synthetic.activations(T, K, seed=0)
    w = synthetic.weights(N, K, seed=0)
    say("backward full: quantize")
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    dyTq, sdyT, dyq, sdy = fl.fp8_quant_transpose(bf16_to_dev(dy), dual=True)
    xTq, sxT = fl.fp8_quant_transpose(xq, sx)
    say("backward full: dgrad")
    dx = fl.fp8_gemm_dgrad(dyq, sdy, wq, sw)
    say("backward full: dgrad on the transposed weight")
    wqT, swT = fl.fp8_weight_transpose(wq, sw)
    dx_t = fl.fp8_gemm_dgrad_t(dyq, sdy, wqT, swT)
    del wqT, swT
    say("backward full: wgrad")
    dw = fl.fp8_gemm_wgrad(dyTq, sdyT, xTq, sxT)
    rows_t = sampled_rows(T, seed=1)
    rows_n = sampled_rows(N, seed=2)
    dxg = host(dx[torch.from_numpy(rows_t).to(DEV)])
    dxg_t = host(dx_t[torch.from_numpy(rows_t).to(DEV)])
    del dx_t
    dwg = host(dw[torch.from_numpy(rows_n).to(DEV)])
    del dx, dw, wq, sw, xq, sx, dyTq, sdyT, dyq, sdy, xTq, sxT
    torch.cuda.empty_cache()
    owq, osw = oracle.quant_weight(w)
    dyq_o, sdy_o = oracle.quant_act(dy[rows_t])
    ref_dx = oracle.gemm(oracle.dequant_rowgroup(dyq_o, sdy_o), oracle.dequant_block(owq, osw), b_trans=True)
    check_metric(dxg, ref_dx, "dgrad full")
    check_metric(dxg_t, ref_dx, "dgrad full (transposed weight)")
    dyTq_o, sdyT_o = oracle.quant_act(np.ascontiguousarray(dy[:, rows_n].T))
    oxq, osx = oracle.quant_act(x)
    xTq_o, sxT_o = oracle.quant_transpose_fp8(oxq, osx)
    ref_dw = oracle.gemm(oracle.dequant_rowgroup(dyTq_o, sdyT_o), oracle.dequant_rowgroup(xTq_o, sxT_o))
    check_metric(dwg, ref_dw, "wgrad full")
