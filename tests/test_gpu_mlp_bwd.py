"""GPU tests of the SwiGLU backward (fp8_swiglu_bwd) and of the MLP block's
backward chain (fp8_mlp_bwd).

fp8_swiglu_bwd must be bit-identical to the oracle wherever the exact
derivative is not next to a BF16 midpoint; on the elements the oracle flags as
such, the GPU's value must be one of the BF16 values next to the oracle's, and
a quantized group holding one must be the quantization of one of its valid
roundings.  In the chain, stage inputs differ from the all-oracle chain's by
the bf16 roundings of GEMM outputs (fp32 vs fp64 accumulation), so each stage
is checked against the oracle run on that stage's GPU inputs (quantizers and
elementwise operators bit for bit, GEMMs with the 1e-2 metric), and the end to
end rms-relative error of the chain is checked beside that."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev
from near_tie import check_bf16_near_ties, check_colq_near_ties, check_rowq_near_ties

pytestmark = pytest.mark.gpu
G = 128
TOL = 1e-2


def compare_swiglu_bwd(out, gate, up, dh, what):
    ref, near = oracle.swiglu_bwd_bf16(gate, up, dh)
    if near.any():
        print("[%s] %d near-tie element(s): checked against both BF16 neighbours" % (what, near.sum()))
    check_bf16_near_ties(host(out), ref, near, what)


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
    hq, hs, hqT, hsT = host(q), host(s), host(qT), host(sT)
    nr = check_rowq_near_ties(dgu, near, hq, hs, what + " rows")
    nc = check_colq_near_ties(dgu, near, hqT, hsT, what + " columns")
    if near.any():
        print("[%s] %d near-tie element(s) in %d row and %d column group(s): each matched one valid rounding"
              % (what, near.sum(), nr, nc))


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


def metric(got_bits, ref, what):
    g = bf16_bits_to_f64(got_bits)
    err = oracle.gemm_metric(g, ref)
    assert err <= TOL, "%s: metric %.3e" % (what, err)
    return err


def same_bits(a, b, what):
    bad = first_mismatch(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    assert bad is None, "%s: first mismatch %s" % (what, bad)


def gpu_stages(dy, saved, F):
    """The backward chain's intermediates from the same C calls fp8_mlp_bwd
    makes (device tensors)."""
    dyTq, sdyT, dyq, sdy = fl.fp8_quant_transpose(dy, dual=True)
    hTq, shT = fl.fp8_quant_transpose(saved["hq"], saved["sh"])
    gu = saved["gu"]
    return {"dyTq": dyTq, "sdyT": sdyT, "dyq": dyq, "sdy": sdy, "hTq": hTq, "shT": shT,
            "xT": fl.fp8_quant_transpose(saved["xq"], saved["sx"]), "gate": gu[:, :F], "up": gu[:, F:]}


@pytest.mark.parametrize("T,K,F", [(256, 256, 384), (384, 512, 256)])
def test_mlp_backward_chain_small(T, K, F):
    """Every stage of the block's backward against the oracle run on that
    stage's GPU inputs: quantizers and the SwiGLU/RMSNorm backward bit for
    bit (valid roundings at near-ties), every GEMM within the metric; the
    chain's outputs equal the separate calls bit for bit; end to end the
    chain stays within 1e-2 rms of the all-oracle chain."""
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
    xd, gd, dyd = bf16_to_dev(x), bf16_to_dev(gamma), bf16_to_dev(dy)
    saved = fl.fp8_mlp_fwd(xd, gd, wgu_q, sgu, wd_q, sd, eps=eps)
    wguT, sguT = fl.fp8_weight_transpose(wgu_q, sgu)
    wdT, sdT = fl.fp8_weight_transpose(wd_q, sd)
    grads = fl.fp8_mlp_bwd(dyd, saved, wguT, sguT, wdT, sdT, x=xd, gamma=gd)
    st = gpu_stages(dyd, saved, F)
    # quantizers of dY and of the saved FP8 H and X
    same_bits(host(st["dyq"]), oracle.quant_act(dy)[0], "dYq")
    same_bits(host(st["dyTq"]), oracle.quant_transpose_bf16(dy)[0], "dY^T q")
    same_bits(host(st["sdyT"]), oracle.quant_transpose_bf16(dy)[1], "dY^T scales")
    hq, sh = host(saved["hq"]), host(saved["sh"])
    ohTq, ohT = oracle.quant_transpose_fp8(hq, sh)
    same_bits(host(st["hTq"]), ohTq, "H^T q")
    same_bits(host(st["shT"]), ohT, "H^T scales")
    xq, sx = host(saved["xq"]), host(saved["sx"])
    oxTq, osxT = oracle.quant_transpose_fp8(xq, sx)
    same_bits(host(st["xT"][0]), oxTq, "X^T q")
    same_bits(host(st["xT"][1]), osxT, "X^T scales")
    # the down projection's gradients on the GPU's operands
    metric(host(grads["dw_down"]), oracle.gemm_wgrad(host(st["dyTq"]), host(st["sdyT"]), ohTq, ohT), "dW_down")
    metric(host(grads["dh"]), oracle.gemm_dgrad(host(st["dyq"]), host(st["sdy"]), owd, osd), "dh")
    # SwiGLU backward fused with both quantizations, on the GPU's gate/up and dh
    gate = np.ascontiguousarray(host(st["gate"]))
    up = np.ascontiguousarray(host(st["up"]))
    dh = host(grads["dh"])
    dguTq, sdguT, dguq, sdgu = fl.fp8_swiglu_bwd_quant(st["gate"], st["up"], grads["dh"])
    dgu, near = oracle.swiglu_bwd_bf16(gate, up, dh)
    check_rowq_near_ties(dgu, near, host(dguq), host(sdgu), "dGU rows")
    check_colq_near_ties(dgu, near, host(dguTq), host(sdguT), "dGU columns")
    # the gate/up projection's gradients on the GPU's operands
    metric(host(grads["dw_gu"]), oracle.gemm_wgrad(host(dguTq), host(sdguT), oxTq, osxT), "dW_gu")
    metric(host(grads["dxn"]), oracle.gemm_dgrad(host(dguq), host(sdgu), owgu, osgu), "dxn")
    # the chain's GEMM outputs are those of the separate calls
    same_bits(host(grads["dw_gu"]), host(fl.fp8_gemm_wgrad(dguTq, sdguT, *st["xT"])), "chain dW_gu")
    same_bits(host(grads["dxn"]), host(fl.fp8_gemm_dgrad_t(dguq, sdgu, wguT, sguT)), "chain dxn")
    # RMSNorm backward on the GPU's rstd and dxn
    odx, odg = oracle.rmsnorm_bwd(x, gamma, host(saved["rstd"]), host(grads["dxn"]))
    same_bits(host(grads["dx"]), odx, "dx")
    same_bits(host(grads["dgamma"]), odg, "dgamma")
    # end to end against the all-oracle chain (stage inputs differ by roundings)
    errs = {}
    for k in ("dh", "dxn", "dw_gu", "dw_down", "dx"):
        want = ref[k] if ref[k].dtype == np.float64 else bf16_bits_to_f64(ref[k])
        errs[k] = rms_rel(bf16_bits_to_f64(host(grads[k])), want)
    errs["dgamma"] = rms_rel(host(grads["dgamma"]).astype(np.float64), ref["dgamma"].astype(np.float64))
    print("[mlp bwd %dx%dx%d] end-to-end rms-relative errors %s" % (T, K, F, errs))
    assert max(errs.values()) <= TOL, errs


def test_mlp_backward_8B_sampled_rows():
    """One 8B layer (T 8192, hidden 4096, intermediate 14336), stage by stage
    on sampled rows, each stage on the GPU's own inputs: dh and dxn (token
    rows), dW_down and dW_gu (weight rows, each needing its row of the
    transposed gradient and the whole transposed activation), the fused
    SwiGLU backward quantization and the RMSNorm backward's dx (token rows)."""
    T, K, F = 8192, 4096, 14336
    eps = 1e-6
    rows = np.array([0, 5, 1000, 4097, 8191])
    wrows_down = np.array([0, 77, 2048, 4095])                  # rows of dW_down [K, F]
    wrows_gu = np.array([0, 1000, 14335, 14336, 28671])         # rows of dW_gu [2F, K] (gate and up halves)
    x = synthetic.activations(T, K, seed=0, n_out=synthetic.n_outliers(K))
    gamma = synthetic.norm_weights(K, seed=0)
    wgu = synthetic.weights(2 * F, K, seed=0)
    wdown = synthetic.weights(K, F, seed=1)
    dy = synthetic.grad_out(T, K, seed=0)
    owgu, osgu = oracle.quant_weight(wgu)
    owd, osd = oracle.quant_weight(wdown)
    del wgu, wdown
    say("mlp fwd+bwd 8B")
    wgu_q, sgu = u8_to_dev(owgu), f32_to_dev(osgu)
    wd_q, sd = u8_to_dev(owd), f32_to_dev(osd)
    xd, gd, dyd = bf16_to_dev(x), bf16_to_dev(gamma), bf16_to_dev(dy)
    saved = fl.fp8_mlp_fwd(xd, gd, wgu_q, sgu, wd_q, sd, eps=eps)
    wguT, sguT = fl.fp8_weight_transpose(wgu_q, sgu)
    wdT, sdT = fl.fp8_weight_transpose(wd_q, sd)
    grads = fl.fp8_mlp_bwd(dyd, saved, wguT, sguT, wdT, sdT, x=xd, gamma=gd)
    st = gpu_stages(dyd, saved, F)
    dguTq, sdguT, dguq, sdgu = fl.fp8_swiglu_bwd_quant(st["gate"], st["up"], grads["dh"])
    same_bits(host(grads["dw_gu"]), host(fl.fp8_gemm_wgrad(dguTq, sdguT, *st["xT"])), "chain dW_gu")
    same_bits(host(grads["dxn"]), host(fl.fp8_gemm_dgrad_t(dguq, sdgu, wguT, sguT)), "chain dxn")
    # token rows: DGrad path, SwiGLU backward quantization, RMSNorm backward
    dyq, sdy = host(st["dyq"])[rows], host(st["sdy"])[rows]
    same_bits(dyq, oracle.quant_act(np.ascontiguousarray(dy[rows]))[0], "dYq rows")
    metric(host(grads["dh"])[rows], oracle.gemm_dgrad(dyq, sdy, owd, osd), "dh rows")
    gate = np.ascontiguousarray(host(st["gate"])[rows])
    up = np.ascontiguousarray(host(st["up"])[rows])
    dgu, near = oracle.swiglu_bwd_bf16(gate, up, host(grads["dh"])[rows])
    check_rowq_near_ties(dgu, near, host(dguq)[rows], host(sdgu)[rows], "dGU rows")
    metric(host(grads["dxn"])[rows], oracle.gemm_dgrad(host(dguq)[rows], host(sdgu)[rows], owgu, osgu), "dxn rows")
    odx, _ = oracle.rmsnorm_bwd(np.ascontiguousarray(x[rows]), gamma, host(saved["rstd"])[rows],
                                host(grads["dxn"])[rows])
    same_bits(host(grads["dx"])[rows], odx, "dx rows")
    # weight rows: WGrad on the GPU's transposed operands
    hTq, shT = host(st["hTq"]), host(st["shT"])
    metric(host(grads["dw_down"])[wrows_down],
           oracle.gemm_wgrad(host(st["dyTq"])[wrows_down], host(st["sdyT"])[wrows_down], hTq, shT),
           "dW_down rows")
    del hTq, shT
    xTq, sxT = host(st["xT"][0]), host(st["xT"][1])
    metric(host(grads["dw_gu"])[wrows_gu],
           oracle.gemm_wgrad(host(dguTq)[wrows_gu], host(sdguT)[wrows_gu], xTq, sxT), "dW_gu rows")


def test_mlp_train_step_graph_replays():
    """The block's forward and backward, the RMSNorm backward and split-K
    decode GEMMs (one the kernel does not split, one it splits four ways,
    through the workspace entry and the allocation-free entry) captured in
    one HIP graph: every replay (new inputs, eager work between replays)
    equals the eager calls bit for bit, and the two split entries agree."""
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
    # a decode GEMM the split-K kernel really splits (K2 / 256 = 8 chunks, 8
    # column blocks: 4 splits), through the workspace entry and the
    # allocation-free one
    N2, K2 = 512, 2048
    assert fl.fp8_gemm_fwd_packed_splitk_workspace(64, N2, K2) == 4 * 64 * N2 * 4
    x2 = bf16_to_dev(synthetic.activations(64, K2, seed=5))
    ow2, os2 = oracle.quant_weight(synthetic.weights(N2, K2, seed=5))
    w2p, s2 = fl.fp8_weight_pack(u8_to_dev(ow2)), f32_to_dev(os2)
    ws2 = torch.empty((fl.fp8_gemm_fwd_packed_splitk_workspace(64, N2, K2) // 4,), dtype=torch.float32, device=DEV)

    def step():
        saved = fl.fp8_mlp_fwd(x, gamma, wgu_q, sgu, wd_q, sd)
        grads = fl.fp8_mlp_bwd(dy, saved, wguT, sguT, wdT, sdT, x=x, gamma=gamma)
        hq64.copy_(saved["hq"][:64])
        sh64.copy_(saved["sh"][:64])
        ydec = fl.fp8_gemm_fwd_packed_splitk(hq64, sh64, wdp, sd, workspace=wsk)
        x2q, x2s = fl.fp8_quant_act(x2)
        y2 = fl.fp8_gemm_fwd_packed_splitk(x2q, x2s, w2p, s2, workspace=ws2)
        y2na = fl.fp8_gemm_fwd_packed_splitk_noalloc(x2q, x2s, w2p, s2)
        return [saved["y"], saved["gu"], saved["hq"], grads["dxn"], grads["dw_gu"], grads["dw_down"],
                grads["dx"], grads["dgamma"], ydec, y2, y2na]

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
        x2.copy_(bf16_to_dev(synthetic.activations(64, K2, seed=70 + r)))
        torch.cuda.synchronize()
        say("mlp train step graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in outs]
        want = [host(t) for t in step()]
        for i, (a, b) in enumerate(zip(got, want)):
            bad = first_mismatch(a.view(np.uint8), b.view(np.uint8))
            assert bad is None, "replay %d output %d: %s" % (r, i, bad)
        assert np.array_equal(got[-1], got[-2])
