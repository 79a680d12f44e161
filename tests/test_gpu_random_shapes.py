"""Randomized parity: for each seed, random shapes and value scales drawn
from the seed, every quantizer and producer bit-exact against the CPU oracle
(near-tie elements of the SwiGLU forms checked against both valid roundings)
and every GEMM form within the 1e-2 metric.  The fixed-shape tests pin the
workloads' sizes and the edge cases; this tier covers the shapes between
them (ragged rows, any number of 128-groups, scales from 1e-4 to 1)."""
import numpy as np
import pytest

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import bf16_bits_to_f64, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev
from test_gpu_mlp_bwd import check_swiglu_bwd_quant, compare_swiglu_bwd
from test_gpu_producers import compare_swiglu, gamma_for, run_rmsnorm

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
