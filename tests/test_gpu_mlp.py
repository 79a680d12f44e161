"""GPU tests of the forward FP8 MLP block (fp8_mlp_fwd): RMSNorm -> gate/up
GEMM -> SwiGLU -> down GEMM in one call.

Each stage must be bit-identical to the separate entry point, and each is
checked against the oracle on its own GPU inputs: the FP8 input of the first
GEMM bit-exact, the gate/up output within the GEMM metric, the SwiGLU
quantization bit-exact on the GPU's gate/up output (valid roundings at
near-ties), the down projection within the metric on the GPU's FP8 H.  The
block's output is also compared end to end with the all-oracle chain; there
the two chains round the gate/up product separately (fp32 vs fp64
accumulation), which can move a SwiGLU code by one step, so that comparison is
on the rms-relative error, 1e-2."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev
from near_tie import check_rowq_near_ties

pytestmark = pytest.mark.gpu
G = 128
TOL = 1e-2


def make_block(T, K, F, seed):
    x = synthetic.activations(T, K, seed=seed, n_out=synthetic.n_outliers(K))
    gamma = synthetic.norm_weights(K, seed=seed)
    wgu = synthetic.weights(2 * F, K, seed=seed)
    wdown = synthetic.weights(K, F, seed=seed + 1)
    return x, gamma, wgu, wdown


def oracle_chain(x, gamma, owgu, osgu, owd, osd, eps):
    xq, sx, rstd = oracle.rmsnorm_quant(x, gamma, eps)
    gu = oracle.f64_to_bf16(oracle.gemm_fwd(xq, sx, owgu, osgu))
    F = gu.shape[1] // 2
    hq, sh, _ = oracle.swiglu_quant(np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]))
    y = oracle.gemm_fwd(hq, sh, owd, osd)
    return xq, sx, rstd, gu, y


def same(a, b, what):
    bad = first_mismatch(a, b)
    assert bad is None, "%s: first mismatch at %s (%d total)" % (what, bad[0], bad[3])


def run_block(T, K, F, seed, rows=None, eps=1e-6):
    x, gamma, wgu, wdown = make_block(T, K, F, seed)
    owgu, osgu = oracle.quant_weight(wgu)
    owd, osd = oracle.quant_weight(wdown)
    say("mlp_fwd", T, K, F)
    dx, dg = bf16_to_dev(x), bf16_to_dev(gamma)
    wgu_q, sgu = u8_to_dev(owgu), f32_to_dev(osgu)
    wd_q, sd = u8_to_dev(owd), f32_to_dev(osd)
    out = fl.fp8_mlp_fwd(dx, dg, wgu_q, sgu, wd_q, sd, eps=eps)
    # stage by stage against the separate entry points
    xq, sx, r = fl.fp8_rmsnorm_quant(dx, dg, eps)
    gu = fl.fp8_gemm_fwd(xq, sx, wgu_q, sgu)
    hq, sh = fl.fp8_swiglu_quant(gu[:, :F], gu[:, F:])
    y = fl.fp8_gemm_fwd(hq, sh, wd_q, sd)
    for name, a, b in (("xq", out["xq"], xq), ("sx", out["sx"], sx), ("rstd", out["rstd"], r),
                       ("gu", out["gu"], gu), ("hq", out["hq"], hq), ("sh", out["sh"], sh), ("y", out["y"], y)):
        same(host(a).view(np.uint8), host(b).view(np.uint8), "stage " + name)
    # against the oracle on (sampled) rows: every stage is row-independent
    sel = np.arange(T) if rows is None else rows
    oxq, osx, orstd, ogu, oy = oracle_chain(np.ascontiguousarray(x[sel]), gamma, owgu, osgu, owd, osd, eps)
    same(host(out["xq"])[sel], oxq, "xq vs oracle")
    same(host(out["sx"])[sel].view(np.uint32), osx.view(np.uint32), "sx vs oracle")
    same(host(out["rstd"])[sel].view(np.uint32), orstd.view(np.uint32), "rstd vs oracle")
    ref_gu = oracle.gemm_fwd(oxq, osx, owgu, osgu)
    err_gu = oracle.gemm_metric(bf16_bits_to_f64(host(out["gu"])[sel]), ref_gu)
    assert err_gu <= TOL, err_gu
    # each later stage on its GPU inputs: SwiGLU quantization on the GPU's gu
    # (bit for bit, valid roundings at near-ties), the down GEMM on the GPU's hq
    gu_g = host(out["gu"])[sel]
    h, near = oracle.swiglu_bf16(np.ascontiguousarray(gu_g[:, :F]), np.ascontiguousarray(gu_g[:, F:]))
    check_rowq_near_ties(h, near, host(out["hq"])[sel], host(out["sh"])[sel], "SwiGLU quantization")
    err_y = oracle.gemm_metric(bf16_bits_to_f64(host(out["y"])[sel]),
                               oracle.gemm_fwd(host(out["hq"])[sel], host(out["sh"])[sel], owd, osd))
    assert err_y <= TOL, err_y
    yg = bf16_bits_to_f64(host(out["y"])[sel])
    rel = float(np.sqrt(np.mean((yg - oy) ** 2)) / np.sqrt(np.mean(oy * oy)))
    gu_same = float(np.mean(host(out["gu"])[sel] == ogu))
    hq_same = float(np.mean(host(out["hq"])[sel] == oracle.swiglu_quant(
        np.ascontiguousarray(ogu[:, :F]), np.ascontiguousarray(ogu[:, F:]))[0]))
    print("[mlp %dx%dx%d] gate/up metric %.2e, gu equal %.5f, hq equal %.6f, y rms-rel %.2e"
          % (T, K, F, err_gu, gu_same, hq_same, rel))
    assert rel <= TOL, rel


@pytest.mark.parametrize("T,K,F", [(100, 256, 384), (64, 512, 640), (5, 1024, 1536)])
def test_mlp_fwd_small(T, K, F):
    run_block(T, K, F, seed=T)


def test_mlp_fwd_8B_sampled_rows():
    """One 8B layer's MLP (hidden 4096, intermediate 14336) on 8192 tokens;
    the oracle chain runs on 12 sampled rows."""
    rows = np.array([0, 1, 777, 2048, 3000, 4095, 4096, 5555, 6001, 7000, 8190, 8191])
    run_block(8192, 4096, 14336, seed=0, rows=rows)


def test_mlp_fwd_degenerate():
    say("mlp_fwd degenerate")
    K, F = 256, 128
    x = torch.zeros((0, K), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(K, dtype=torch.bfloat16, device=DEV)
    wgu = torch.zeros((2 * F, K), dtype=torch.uint8, device=DEV)
    sgu = torch.zeros((2 * F // G, K // G), dtype=torch.float32, device=DEV)
    wd = torch.zeros((K, F), dtype=torch.uint8, device=DEV)
    sd = torch.zeros((K // G, F // G), dtype=torch.float32, device=DEV)
    out = fl.fp8_mlp_fwd(x, g, wgu, sgu, wd, sd)
    assert out["y"].shape == (0, K)
