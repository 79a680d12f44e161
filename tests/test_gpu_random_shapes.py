"""Randomized parity: for each seed, random shapes and value scales drawn
from the seed, every quantizer and producer (forward and backward)
bit-exact against the CPU oracle (near-tie elements of the SwiGLU forms
checked against both valid roundings) and every GEMM form within the 1e-2
metric.  The fixed-shape tests pin the
workloads' sizes and the edge cases; this tier covers the shapes between
them (ragged rows, any number of 128-groups, scales from 1e-4 to 1)."""
import numpy as np
import pytest

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import bf16_bits_to_f64, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev
from test_gpu_mlp_bwd import check_swiglu_bwd_quant, compare_swiglu_bwd
from test_gpu_producers import compare_swiglu, gamma_for, run_rmsnorm, run_rmsnorm_bwd

pytestmark = pytest.mark.gpu
G = 128
TOL = 1e-2


def same(a, b, what):
    bad = first_mismatch(a, b)
    assert bad is None, "%s: first mismatch at %s" % (what, bad)


def within_metric(y, ref, what):
    m = oracle.gemm_metric(bf16_bits_to_f64(host(y)), ref)
    assert m <= TOL, (what, m)


@pytest.mark.parametrize("seed", range(9000, 9048))
def test_random_shapes(seed):
    r = np.random.default_rng(seed)
    say("random shapes, seed", seed)
    # 1x128 and 128x128 quantization, transposed dual quantization
    M, K = int(r.integers(1, 400)), G * int(r.integers(1, 40))
    x = synthetic.activations(M, K, seed=seed, n_out=int(r.integers(0, 6)))
    q, s = fl.fp8_quant_act(bf16_to_dev(x))
    oq, os_ = oracle.quant_act(x)
    same(host(q), oq, "quant_act %dx%d" % (M, K))
    same(host(s).view(np.uint32), os_.view(np.uint32), "quant_act scales")
    N = G * int(r.integers(1, 12))
    w = synthetic.weights(N, K, seed=seed, sigma=float(10.0 ** r.uniform(-3, 0)))
    q, s = fl.fp8_quant_weight(bf16_to_dev(w))
    oq, os_ = oracle.quant_weight(w)
    same(host(q), oq, "quant_weight %dx%d" % (N, K))
    same(host(s).view(np.uint32), os_.view(np.uint32), "quant_weight scales")
    T, C = G * int(r.integers(1, 5)), G * int(r.integers(1, 10))
    xt = synthetic.activations(T, C, seed=seed + 1000, n_out=2)
    qT, sT, qr, sr = fl.fp8_quant_transpose(bf16_to_dev(xt), dual=True)
    oqT, osT = oracle.quant_transpose_bf16(xt)
    same(host(qT), oqT, "quant_transpose %dx%d" % (T, C))
    same(host(sT).view(np.uint32), osT.view(np.uint32), "quant_transpose scales")
    oq, os_ = oracle.quant_act(xt)
    same(host(qr), oq, "quant_transpose dual rows")
    same(host(sr).view(np.uint32), os_.view(np.uint32), "quant_transpose dual row scales")

    # producers: RMSNorm and SwiGLU fused with the quantization, SwiGLU backward
    Mr, Kr = int(r.integers(1, 200)), G * int(r.integers(1, 64))
    run_rmsnorm(synthetic.activations(Mr, Kr, seed=seed + 7, n_out=int(r.integers(0, 4))), gamma_for(Kr, seed),
                float(r.choice([1e-6, 1e-5, 0.0])), "random %d" % seed)
    Mb, Kb = int(r.integers(1, 400)), G * int(r.integers(1, 64))
    run_rmsnorm_bwd(Mb, Kb, seed, "random %d" % seed, with_dgamma=bool(r.integers(0, 4)))
    Ms, F = int(r.integers(1, 160)), G * int(r.integers(1, 24))
    gate = synthetic.gaussian_bf16((Ms, F), float(r.uniform(0.3, 6.0)), seed, 11)
    up = synthetic.gaussian_bf16((Ms, F), float(r.uniform(0.1, 3.0)), seed, 12)
    q, s = fl.fp8_swiglu_quant(bf16_to_dev(gate), bf16_to_dev(up))
    compare_swiglu(q, s, gate, up, "swiglu %dx%d" % (Ms, F))
    dh = synthetic.gaussian_bf16((Ms, F), float(10.0 ** r.uniform(-4, 0)), seed, 13)
    compare_swiglu_bwd(fl.fp8_swiglu_bwd(bf16_to_dev(gate), bf16_to_dev(up), bf16_to_dev(dh)), gate, up, dh,
                       "swiglu_bwd %dx%d" % (Ms, F))
    Tq = G * int(r.integers(1, 3))
    check_swiglu_bwd_quant(synthetic.gaussian_bf16((Tq, F), float(r.uniform(0.3, 6.0)), seed, 14),
                           synthetic.gaussian_bf16((Tq, F), 1.0, seed, 15),
                           synthetic.gaussian_bf16((Tq, F), 1e-2, seed, 16), "swiglu_bwd_quant %dx%d" % (Tq, F))

    # GEMMs: forward (both entry points), DGrad, WGrad
    Mg, Ng, Kg = int(r.integers(1, 300)), G * int(r.integers(1, 8)), G * int(r.integers(1, 12))
    xq, sx = synthetic.random_codes((Mg, Kg), seed, 21), synthetic.random_scales((Mg, Kg // G), seed, 22)
    wq, sw = synthetic.random_codes((Ng, Kg), seed, 23), synthetic.random_scales((Ng // G, Kg // G), seed, 24)
    ref = oracle.gemm_fwd(xq, sx, wq, sw)
    args = (u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    within_metric(fl.fp8_gemm_fwd(*args), ref, "fwd %dx%dx%d" % (Mg, Ng, Kg))
    within_metric(fl.fp8_gemm_fwd_unified(*args), ref, "fwd unified %dx%dx%d" % (Mg, Ng, Kg))
    Td = int(r.integers(1, 300))
    dyq, sdy = synthetic.random_codes((Td, Ng), seed, 25), synthetic.random_scales((Td, Ng // G), seed, 26)
    within_metric(fl.fp8_gemm_dgrad(u8_to_dev(dyq), f32_to_dev(sdy), u8_to_dev(wq), f32_to_dev(sw)),
                  oracle.gemm_dgrad(dyq, sdy, wq, sw), "dgrad %dx%dx%d" % (Td, Ng, Kg))
    Tw, Nw, Kw = G * int(r.integers(1, 4)), int(r.integers(1, 300)), 4 * int(r.integers(1, 100))
    aT, saT = synthetic.random_codes((Nw, Tw), seed, 27), synthetic.random_scales((Nw, Tw // G), seed, 28)
    bT, sbT = synthetic.random_codes((Kw, Tw), seed, 29), synthetic.random_scales((Kw, Tw // G), seed, 30)
    within_metric(fl.fp8_gemm_wgrad(u8_to_dev(aT), f32_to_dev(saT), u8_to_dev(bT), f32_to_dev(sbT)),
                  oracle.gemm_wgrad(aT, saT, bT, sbT), "wgrad %dx%dx%d" % (Nw, Kw, Tw))


@pytest.mark.parametrize("seed", range(9100, 9132))
def test_random_shapes_rollout_and_fused(seed):
    """The rollout GEMMs (decode layout, split over K with a workspace and
    without), 4-bit weights, the FP8-source transpose, DGrad on the transposed
    weight, and the one-call linear and MLP forward against their parts."""
    r = np.random.default_rng(seed)
    say("random shapes (rollout and fused), seed", seed)
    # decode layout and split-K: M <= 64, K % 256 == 0
    M, N, K = int(r.integers(1, 65)), G * int(r.integers(1, 40)), 256 * int(r.integers(1, 24))
    xq, sx = synthetic.random_codes((M, K), seed, 41), synthetic.random_scales((M, K // G), seed, 42)
    wq, sw = synthetic.random_codes((N, K), seed, 43), synthetic.random_scales((N // G, K // G), seed, 44)
    ref = oracle.gemm_fwd(xq, sx, wq, sw)
    dx, dsx, dw, dsw = u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw)
    wp = fl.fp8_weight_pack(dw)
    y_packed = fl.fp8_gemm_fwd_packed(dx, dsx, wp, dsw)
    within_metric(y_packed, ref, "packed %dx%dx%d" % (M, N, K))
    same(host(y_packed), host(fl.fp8_gemm_fwd(dx, dsx, dw, dsw)), "packed vs unpacked bits")
    y_split = fl.fp8_gemm_fwd_packed_splitk(dx, dsx, wp, dsw)
    within_metric(y_split, ref, "split-K %dx%dx%d" % (M, N, K))
    if fl.fp8_gemm_fwd_packed_splitk_workspace(M, N, K) <= 4 << 20:
        same(host(fl.fp8_gemm_fwd_packed_splitk_noalloc(dx, dsx, wp, dsw)), host(y_split), "noalloc vs workspace")

    # 4-bit weights: quantizer bit-exact, GEMM within the metric
    N4, K4 = int(r.integers(1, 300)), G * int(r.integers(1, 40))
    w = synthetic.weights(N4, K4, seed=seed, sigma=float(10.0 ** r.uniform(-3, 0)))
    c4, s4 = fl.fp8_mxfp4_quant_weight(bf16_to_dev(w))
    oc4, os4 = oracle.mxfp4_quant(w)
    same(host(c4), oc4, "mxfp4 codes %dx%d" % (N4, K4))
    same(host(s4), os4, "mxfp4 scales")
    M4 = int(r.integers(1, 200))
    xq4, sx4 = synthetic.random_codes((M4, K4), seed, 45), synthetic.random_scales((M4, K4 // G), seed, 46)
    within_metric(fl.fp8_gemm_fwd_w4(u8_to_dev(xq4), f32_to_dev(sx4), c4, s4), oracle.gemm_fwd_w4(xq4, sx4, oc4, os4),
                  "w4 %dx%dx%d" % (M4, N4, K4))

    # transpose of saved FP8 activations; DGrad on the transposed weight
    T, C = G * int(r.integers(1, 5)), G * int(r.integers(1, 10))
    xa = synthetic.activations(T, C, seed=seed + 2000, n_out=2)
    q, s = fl.fp8_quant_act(bf16_to_dev(xa))
    qT, sT = fl.fp8_quant_transpose(q, s)
    oqT, osT = oracle.quant_transpose_fp8(host(q), host(s))
    same(host(qT), oqT, "quant_transpose fp8 %dx%d" % (T, C))
    same(host(sT).view(np.uint32), osT.view(np.uint32), "quant_transpose fp8 scales")
    Nd, Kd, Td = G * int(r.integers(1, 8)), G * int(r.integers(1, 8)), int(r.integers(1, 300))
    wd, swd = synthetic.random_codes((Nd, Kd), seed, 47), synthetic.random_scales((Nd // G, Kd // G), seed, 48)
    wdT, swdT = fl.fp8_weight_transpose(u8_to_dev(wd), f32_to_dev(swd))
    same(host(wdT), wd.T, "weight transpose codes")
    same(host(swdT).view(np.uint32), np.ascontiguousarray(swd.T).view(np.uint32), "weight transpose scales")
    dyq, sdy = synthetic.random_codes((Td, Nd), seed, 49), synthetic.random_scales((Td, Nd // G), seed, 50)
    within_metric(fl.fp8_gemm_dgrad_t(u8_to_dev(dyq), f32_to_dev(sdy), wdT, swdT), oracle.gemm_dgrad(dyq, sdy, wd, swd),
                  "dgrad_t %dx%dx%d" % (Td, Nd, Kd))

    # one-call forms, bit-identical to the calls they enqueue
    Ml, Kl, Nl = int(r.integers(1, 200)), G * int(r.integers(1, 16)), G * int(r.integers(1, 8))
    xl = bf16_to_dev(synthetic.activations(Ml, Kl, seed=seed + 3000, n_out=1))
    wl, swl = u8_to_dev(synthetic.random_codes((Nl, Kl), seed, 51)), f32_to_dev(synthetic.random_scales((Nl // G, Kl // G), seed, 52))
    y, ql, sl = fl.fp8_linear_fwd(xl, wl, swl)
    q2, s2 = fl.fp8_quant_act(xl)
    same(host(ql), host(q2), "linear_fwd codes")
    same(host(y), host(fl.fp8_gemm_fwd(q2, s2, wl, swl)), "linear_fwd output")
    Tm, Km, Fm = int(r.integers(1, 160)), G * int(r.integers(1, 12)), G * int(r.integers(1, 12))
    xm = bf16_to_dev(synthetic.activations(Tm, Km, seed=seed + 4000, n_out=1))
    gm = bf16_to_dev(synthetic.norm_weights(Km, seed=seed))
    wgu, sgu = fl.fp8_quant_weight(bf16_to_dev(synthetic.weights(2 * Fm, Km, seed=seed + 1)))
    wdn, sdn = fl.fp8_quant_weight(bf16_to_dev(synthetic.weights(Km, Fm, seed=seed + 2)))
    o = fl.fp8_mlp_fwd(xm, gm, wgu, sgu, wdn, sdn)
    xq1, sx1, r1 = fl.fp8_rmsnorm_quant(xm, gm)
    gu1 = fl.fp8_gemm_fwd(xq1, sx1, wgu, sgu)
    hq1, sh1 = fl.fp8_swiglu_quant(gu1[:, :Fm], gu1[:, Fm:])
    for name, a, b in (("xq", o["xq"], xq1), ("rstd", o["rstd"], r1), ("gu", o["gu"], gu1), ("hq", o["hq"], hq1),
                       ("sh", o["sh"], sh1), ("y", o["y"], fl.fp8_gemm_fwd(hq1, sh1, wdn, sdn))):
        same(host(a).view(np.uint8), host(b).view(np.uint8), "mlp_fwd %s (%dx%dx%d)" % (name, Tm, Km, Fm))
