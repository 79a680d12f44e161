"""GPU tests of the SwiGLU backward (fp8_swiglu_bwd) and of the MLP block's
backward chain (fp8_mlp_bwd).

fp8_swiglu_bwd must be bit-identical to the oracle wherever the exact
derivative is not next to a BF16 midpoint (the oracle flags such elements;
groups of 128 holding one are reported and skipped).  The chain is compared
with the oracle chain computed from the same inputs on the CPU: stage inputs
differ by the bf16 roundings of GEMM outputs (fp32 vs fp64 accumulation), so
its tolerance is on the rms-relative error, 1e-2; the per-call parity of
every call in the chain is covered by the other GPU tests."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
G = 128
TOL = 1e-2


def compare_swiglu_bwd(out, gate, up, dh, what):
    ref, near = oracle.swiglu_bwd_bf16(gate, up, dh)
    got = host(out)
    M, F2 = ref.shape
    keep = ~near
    if near.any():
        print("[%s] %d near-tie element(s) skipped" % (what, near.sum()))
    bad = first_mismatch(got[keep], ref[keep])
    assert bad is None, "%s: first mismatch at flat %s gpu=%#x ref=%#x (%d total)" % (what, bad[0], bad[1], bad[2],
                                                                                     bad[3])


@pytest.mark.parametrize("M,F", [(1, 128), (37, 1024), (64, 14336), (300, 640)])
def test_swiglu_bwd_shapes(M, F):
    gate = synthetic.activations(M, F, seed=F + 3, n_out=max(1, F // 1024))
    up = synthetic.activations(M, F, seed=F + 4, n_out=0)
    dh = synthetic.grad_out(M, F, seed=F + 5)
    say("swiglu_bwd", M, F)
    out = fl.fp8_swiglu_bwd(bf16_to_dev(gate), bf16_to_dev(up), bf16_to_dev(dh))
    compare_swiglu_bwd(out, gate, up, dh, "%dx%d" % (M, F))


def test_swiglu_bwd_halves_and_special_values():
    M, F = 40, 512
    rng = np.random.default_rng(3)
    gu = synthetic.activations(M, 2 * F, seed=8, n_out=3)
    g32 = synthetic.bf16_bits_to_f32(gu)
    g32[0, :F] = 0.0
    g32[1, :F] = rng.uniform(60, 800, F) * np.where(rng.random(F) < 0.5, -1, 1)
    g32[2, :F] = -1.2784645                        # near the zero of silu'
    gu = synthetic.f32_to_bf16_bits(g32)
    dh = synthetic.grad_out(M, F, seed=9)
    say("swiglu_bwd halves")
    t = bf16_to_dev(gu)
    out = fl.fp8_swiglu_bwd(t[:, :F], t[:, F:], bf16_to_dev(dh))
    compare_swiglu_bwd(out, np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]), dh, "halves")


def test_swiglu_bwd_full_size():
    M, F = 8192, 14336
    gu = synthetic.activations(M, 2 * F, seed=1, n_out=synthetic.n_outliers(2 * F))
    dh = synthetic.grad_out(M, F, seed=2)
    say("swiglu_bwd full", M, F)
    t = bf16_to_dev(gu)
    out = fl.fp8_swiglu_bwd(t[:, :F], t[:, F:], bf16_to_dev(dh))
    compare_swiglu_bwd(out, np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]), dh, "8B")


def check_swiglu_bwd_quant(gate, up, dh, what, gu_dev=None):
    """Fused kernel vs the oracle chain (SwiGLU backward, then both
    quantizations) and vs the two unfused GPU calls."""
    T, F = gate.shape
    if gu_dev is None:
        g_d, u_d = bf16_to_dev(gate), bf16_to_dev(up)
    else:
        g_d, u_d = gu_dev[:, :F], gu_dev[:, F:]
    d_d = bf16_to_dev(dh)
    say("swiglu_bwd_quant", what, T, F)
    qT, sT, q, s = fl.fp8_swiglu_bwd_quant(g_d, u_d, d_d)
    uqT, usT, uq, us = fl.fp8_quant_transpose(fl.fp8_swiglu_bwd(g_d, u_d, d_d), dual=True)
    for name, a, b in (("dguTq", qT, uqT), ("sdguT", sT, usT), ("dguq", q, uq), ("sdgu", s, us)):
        bad = first_mismatch(host(a).view(np.uint8), host(b).view(np.uint8))
        assert bad is None, "%s %s vs unfused: %s" % (what, name, bad)
    dgu, near = oracle.swiglu_bwd_bf16(gate, up, dh)
    oq, os_ = oracle.quant_act(dgu)
    oqT, osT = oracle.quant_transpose_bf16(dgu)
    row_ok = ~near.reshape(T, 2 * F // G, G).any(axis=2)            # [T, 2F/128]
    col_ok = ~near.T.reshape(2 * F, T // G, G).any(axis=2)          # [2F, T/128]
    if near.any():
        print("[%s] %d near-tie element(s): their groups skipped" % (what, near.sum()))
    hq, hs, hqT, hsT = host(q), host(s), host(qT), host(sT)
    assert np.array_equal(hs.view(np.uint32)[row_ok], os_.view(np.uint32)[row_ok])
    assert np.array_equal(hq.reshape(T, -1, G)[row_ok], oq.reshape(T, -1, G)[row_ok])
    assert np.array_equal(hsT.view(np.uint32)[col_ok], osT.view(np.uint32)[col_ok])
    assert np.array_equal(hqT.reshape(2 * F, -1, G)[col_ok], oqT.reshape(2 * F, -1, G)[col_ok])


@pytest.mark.parametrize("T,F", [(128, 128), (256, 640), (384, 1024)])
def test_swiglu_bwd_quant_shapes(T, F):
    gate = synthetic.activations(T, F, seed=F + 6, n_out=max(1, F // 512))
    up = synthetic.activations(T, F, seed=F + 7, n_out=0)
    dh = synthetic.grad_out(T, F, seed=F + 8)
    check_swiglu_bwd_quant(gate, up, dh, "%dx%d" % (T, F))


def test_swiglu_bwd_quant_8B():
    """8192 tokens x 14336, gate and up as the halves of the saved [T, 2F] output."""
    T, F = 8192, 14336
    gu = synthetic.activations(T, 2 * F, seed=1, n_out=synthetic.n_outliers(2 * F))
    dh = synthetic.grad_out(T, F, seed=2)
    check_swiglu_bwd_quant(np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]), dh, "8B",
                           gu_dev=bf16_to_dev(gu))


def test_swiglu_bwd_degenerate():
    say("swiglu_bwd empty")
    z = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    assert fl.fp8_swiglu_bwd(z, z, z).shape == (0, 512)


# --------------------------------------------------------- backward chain

def rms_rel(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.sqrt(np.mean((np.asarray(got, np.float64) - ref) ** 2)) / np.sqrt(np.mean(ref * ref)))


def oracle_block_fwd_bwd(x, gamma, wgu, wdown, dy, eps):
    """The whole block, forward and backward, through the oracle."""
    owgu, osgu = oracle.quant_weight(wgu)
    owd, osd = oracle.quant_weight(wdown)
    xq, sx, _ = oracle.rmsnorm_quant(x, gamma, eps)
    gu = oracle.f64_to_bf16(oracle.gemm_fwd(xq, sx, owgu, osgu))
    F = gu.shape[1] // 2
    g, u = np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:])
    hq, sh, _ = oracle.swiglu_quant(g, u)
    dyq, sdy = oracle.quant_act(dy)
    dyTq, sdyT = oracle.quant_transpose_bf16(dy)
    hTq, shT = oracle.quant_transpose_fp8(hq, sh)
    dw_down = oracle.gemm_wgrad(dyTq, sdyT, hTq, shT)
    dh = oracle.f64_to_bf16(oracle.gemm_dgrad(dyq, sdy, owd, osd))
    dgu, _ = oracle.swiglu_bwd_bf16(g, u, dh)
    dguq, sdgu = oracle.quant_act(dgu)
    dguTq, sdguT = oracle.quant_transpose_bf16(dgu)
    xTq, sxT = oracle.quant_transpose_fp8(xq, sx)
    dw_gu = oracle.gemm_wgrad(dguTq, sdguT, xTq, sxT)
    dxn = oracle.gemm_dgrad(dguq, sdgu, owgu, osgu)
    _, rstd = oracle.rmsnorm_bf16(x, gamma, eps)
    dx, dgamma = oracle.rmsnorm_bwd(x, gamma, rstd, oracle.f64_to_bf16(dxn))
    return ({"dxn": dxn, "dw_gu": dw_gu, "dw_down": dw_down, "dh": dh, "dgu": dgu, "dx": dx, "dgamma": dgamma},
            (owgu, osgu, owd, osd))


@pytest.mark.parametrize("T,K,F", [(256, 256, 384), (384, 512, 256)])
def test_mlp_backward_chain_small(T, K, F):
    eps = 1e-6
    x = synthetic.activations(T, K, seed=T, n_out=2)
    gamma = synthetic.norm_weights(K, seed=T)
    wgu = synthetic.weights(2 * F, K, seed=T)
    wdown = synthetic.weights(K, F, seed=T + 1)
    dy = synthetic.grad_out(T, K, seed=T)
    ref, (owgu, osgu, owd, osd) = oracle_block_fwd_bwd(x, gamma, wgu, wdown, dy, eps)
    say("mlp fwd+bwd chain", T, K, F)
    wgu_q, sgu = u8_to_dev(owgu), f32_to_dev(osgu)
    wd_q, sd = u8_to_dev(owd), f32_to_dev(osd)
    saved = fl.fp8_mlp_fwd(bf16_to_dev(x), bf16_to_dev(gamma), wgu_q, sgu, wd_q, sd, eps=eps)
    wguT, sguT = fl.fp8_weight_transpose(wgu_q, sgu)
    wdT, sdT = fl.fp8_weight_transpose(wd_q, sd)
    grads = fl.fp8_mlp_bwd(bf16_to_dev(dy), saved, wguT, sguT, wdT, sdT, x=bf16_to_dev(x),
                           gamma=bf16_to_dev(gamma))
    errs = {}
    for k in ("dh", "dxn", "dw_gu", "dw_down", "dx"):
        want = ref[k] if ref[k].dtype == np.float64 else bf16_bits_to_f64(ref[k])
        errs[k] = rms_rel(bf16_bits_to_f64(host(grads[k])), want)
    errs["dgamma"] = rms_rel(host(grads["dgamma"]).astype(np.float64), ref["dgamma"].astype(np.float64))
    print("[mlp bwd %dx%dx%d] rms-relative errors %s" % (T, K, F, errs))
    assert max(errs.values()) <= TOL, errs


def test_mlp_backward_8B_sampled_rows():
    """One 8B layer (T 8192, hidden 4096, intermediate 14336): the DGrad path
    (dh, dxn) of sampled token rows against the oracle, which needs only
    those rows of every operand; dw_down and dw_gu checked for finiteness and
    scale (the WGrad kernels' own full-size parity is tested elsewhere)."""
    T, K, F = 8192, 4096, 14336
    eps = 1e-6
    rows = np.array([0, 5, 1000, 4097, 8191])
    x = synthetic.activations(T, K, seed=0, n_out=synthetic.n_outliers(K))
    gamma = synthetic.norm_weights(K, seed=0)
    wgu = synthetic.weights(2 * F, K, seed=0)
    wdown = synthetic.weights(K, F, seed=1)
    dy = synthetic.grad_out(T, K, seed=0)
    owgu, osgu = oracle.quant_weight(wgu)
    owd, osd = oracle.quant_weight(wdown)
    say("mlp fwd+bwd 8B")
    wgu_q, sgu = u8_to_dev(owgu), f32_to_dev(osgu)
    wd_q, sd = u8_to_dev(owd), f32_to_dev(osd)
    saved = fl.fp8_mlp_fwd(bf16_to_dev(x), bf16_to_dev(gamma), wgu_q, sgu, wd_q, sd, eps=eps)
    wguT, sguT = fl.fp8_weight_transpose(wgu_q, sgu)
    wdT, sdT = fl.fp8_weight_transpose(wd_q, sd)
    grads = fl.fp8_mlp_bwd(bf16_to_dev(dy), saved, wguT, sguT, wdT, sdT)
    # oracle on the sampled rows (every DGrad-path stage is row-local)
    xs, dys = np.ascontiguousarray(x[rows]), np.ascontiguousarray(dy[rows])
    xq, sx, _ = oracle.rmsnorm_quant(xs, gamma, eps)
    gu = oracle.f64_to_bf16(oracle.gemm_fwd(xq, sx, owgu, osgu))
    g, u = np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:])
    dyq, sdy = oracle.quant_act(dys)
    dh = oracle.f64_to_bf16(oracle.gemm_dgrad(dyq, sdy, owd, osd))
    dgu, _ = oracle.swiglu_bwd_bf16(g, u, dh)
    dguq, sdgu = oracle.quant_act(dgu)
    dxn = oracle.gemm_dgrad(dguq, sdgu, owgu, osgu)
    errs = {"dh": rms_rel(bf16_bits_to_f64(host(grads["dh"])[rows]), bf16_bits_to_f64(dh)),
            "dxn": rms_rel(bf16_bits_to_f64(host(grads["dxn"])[rows]), dxn)}
    print("[mlp bwd 8B] rms-relative errors on sampled rows %s" % errs)
    assert max(errs.values()) <= TOL, errs
    for k in ("dw_gu", "dw_down"):
        w = bf16_bits_to_f64(host(grads[k]))
        assert np.all(np.isfinite(w)) and np.sqrt(np.mean(w * w)) > 0, k


def test_mlp_train_step_graph_replays():
    """The block's forward and backward, the split-K decode GEMM and the RMSNorm
    backward captured in one HIP graph: every replay (new inputs, eager work
    between replays) equals the eager calls bit for bit."""
    T, K, F = 256, 512, 512                                     # F % 256 == 0 for the decode layout
    owgu, osgu = oracle.quant_weight(synthetic.weights(2 * F, K, seed=3))
    owd, osd = oracle.quant_weight(synthetic.weights(K, F, seed=4))
    wgu_q, sgu, wd_q, sd = u8_to_dev(owgu), f32_to_dev(osgu), u8_to_dev(owd), f32_to_dev(osd)
    wguT, sguT = fl.fp8_weight_transpose(wgu_q, sgu)
    wdT, sdT = fl.fp8_weight_transpose(wd_q, sd)
    wdp = fl.fp8_weight_pack(wd_q)
    gamma = bf16_to_dev(synthetic.norm_weights(K, seed=3))
    x = bf16_to_dev(synthetic.activations(T, K, seed=3))
    dy = bf16_to_dev(synthetic.grad_out(T, K, seed=3))
    hq64 = torch.empty((64, F), dtype=torch.uint8, device=DEV)
    sh64 = torch.empty((64, F // G), dtype=torch.float32, device=DEV)
    wsk = torch.empty((max(fl.fp8_gemm_fwd_packed_splitk_workspace(64, K, F) // 4, 1),), dtype=torch.float32,
                      device=DEV)

    def step():
        saved = fl.fp8_mlp_fwd(x, gamma, wgu_q, sgu, wd_q, sd)
        grads = fl.fp8_mlp_bwd(dy, saved, wguT, sguT, wdT, sdT, x=x, gamma=gamma)
        hq64.copy_(saved["hq"][:64])
        sh64.copy_(saved["sh"][:64])
        ydec = fl.fp8_gemm_fwd_packed_splitk(hq64, sh64, wdp, sd, workspace=wsk)
        return [saved["y"], saved["gu"], saved["hq"], grads["dxn"], grads["dw_gu"], grads["dw_down"],
                grads["dx"], grads["dgamma"], ydec]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("mlp train step graph capture")
    with torch.cuda.stream(s):
        step()                                                  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = step()
    for r in range(3):
        x.copy_(bf16_to_dev(synthetic.activations(T, K, seed=60 + r)))
        dy.copy_(bf16_to_dev(synthetic.grad_out(T, K, seed=60 + r)))
        torch.cuda.synchronize()
        say("mlp train step graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in outs]
        want = [host(t) for t in step()]
        for i, (a, b) in enumerate(zip(got, want)):
            bad = first_mismatch(a.view(np.uint8), b.view(np.uint8))
            assert bad is None, "replay %d output %d: %s" % (r, i, bad)
