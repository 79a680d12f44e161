"""GPU parity of the 4-bit (MXFP4) rollout path against the CPU oracle.

fp8_mxfp4_quant_weight: codes and scales bit-exact (small and ragged shapes,
adversarial blocks: zeros, negative zeros, every rounding midpoint,
saturation, subnormal and huge magnitudes, and the full 8B up-projection
weight).  fp8_gemm_fwd_w4: max|Y - Y_ref| / (|Y_ref| + 0.01 rms(Y_ref)) <= 1e-2
against the oracle's fp64 GEMM on the same codes, over ragged M/N, several
64-row slabs, K from one group to 4096, blocks of very different scales in one
group, and the full decode shape on sampled columns; plus the chain GPU
quantizers -> GPU GEMM against the oracle chain, and the rollout step
replayed from a HIP graph."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-2


def bf16(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def assert_same(gpu, ref, what):
    bad = first_mismatch(gpu, ref)
    assert bad is None, "%s: first mismatch at %s gpu=%r ref=%r (%d total)" % (what, bad[0], bad[1], bad[2], bad[3])


def run_quant(w, what):
    say("mxfp4_quant", what, w.shape)
    c, s = fl.fp8_mxfp4_quant_weight(bf16_to_dev(w))
    oc, os_ = oracle.mxfp4_quant(w)
    assert_same(host(c), oc, what + " codes")
    assert_same(host(s), os_, what + " scales")
    return c, s, oc, os_


@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (33, 4096), (130, 1024), (3, 16384)])
def test_mxfp4_quant_shapes(N, K):
    run_quant(synthetic.weights(N, K, seed=N + K), "%dx%d" % (N, K))


def test_mxfp4_quant_adversarial_blocks():
    rng = np.random.default_rng(7)
    rows = []
    z = np.zeros(64)
    rows.append(z)
    nz = np.zeros(64, np.float32)
    nz[::3] = -0.0
    rows.append(nz)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    r = np.zeros(64)
    r[0] = 4.0
    r[1:8] = mids
    r[8:15] = -mids
    r[32] = 4.0
    r[33:40] = mids * 1.0000001
    r[40:47] = -mids * 0.9999999
    rows.append(r * 2.0 ** -9)
    sat = np.zeros(64)
    sat[:6] = [7.5, 6.5, 5.5, -7.75, 1.0, 5.0]
    sat[32:36] = [7.9, -7.9, 3.0, 0.1]
    rows.append(sat * 2.0 ** 12)
    rows.append(rng.normal(0, 1, 64) * 1e-38)        # bf16 subnormals and tiny normals
    rows.append(rng.normal(0, 1, 64) * 1e37)
    rows.append(rng.normal(0, 1, 64) * 2.0 ** rng.integers(-30, 30, 64))
    w = np.stack([bf16(x) for x in rows])
    w[1, ::3] = 0x8000
    w[4, 5] = 0x0001                                 # smallest bf16 subnormal
    w[5, 7] = 0x7F7F                                 # largest finite bf16
    run_quant(w, "adversarial")


def test_mxfp4_quant_full_size():
    run_quant(synthetic.weights(14336, 4096, seed=0), "8B up-proj W")


def test_mxfp4_quant_degenerate():
    say("mxfp4_quant empty")
    c, s = fl.fp8_mxfp4_quant_weight(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert c.shape == (0, 32) and s.shape == (0, 2)
    with pytest.raises(fl.Fp8LinError, match="FP8LIN_ERR_SHAPE"):
        fl.fp8_mxfp4_quant_weight(torch.zeros((2, 48), dtype=torch.bfloat16, device=DEV))


# ------------------------------------------------------------------ GEMM

def run_gemm(M, N, K, seed, what, w=None, cols=None):
    x = synthetic.activations(M, K, seed=seed, n_out=max(1, K // 1024))
    if w is None:
        w = synthetic.weights(N, K, seed=seed)
    xq, sx = oracle.quant_act(x)
    c, s = oracle.mxfp4_quant(w)
    say("gemm_fwd_w4", what, M, N, K)
    y = fl.fp8_gemm_fwd_w4(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(c), u8_to_dev(s))
    yg = bf16_bits_to_f64(host(y))
    if cols is None:
        ref = oracle.gemm_fwd_w4(xq, sx, c, s)
    else:
        ref = oracle.gemm_fwd_w4(xq, sx, np.ascontiguousarray(c[cols]), np.ascontiguousarray(s[cols]))
        yg = yg[:, cols]
    err = oracle.gemm_metric(yg, ref)
    print("[%s] metric %.3g" % (what, err))
    assert err <= TOL, "%s: metric %g" % (what, err)


@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (7, 100, 384), (64, 256, 4096), (65, 96, 1024),
                                   (130, 200, 512), (16, 1000, 2048), (3, 64, 16384), (1, 32, 256),
                                   (64, 64, 256), (40, 96, 7936), (64, 1, 512), (2, 33, 128)])
def test_gemm_w4_shapes(M, N, K):
    """Ragged M and N, one and several 64-row slabs and 64-column blocks, K
    from one 128-group to the largest supported; M <= 64 with K % 256 == 0
    takes the LDS-ring decode kernel (one chunk, an odd chunk count, the
    unrolled K = 4096 form), the rest the generic one."""
    run_gemm(M, N, K, seed=M + N + K, what="%dx%dx%d" % (M, N, K))


def test_gemm_w4_blocks_of_very_different_scale():
    """Within one column's 128-group the four 32-blocks span up to 2^40: the
    small blocks' terms are rounded in fp16 relative to the largest block."""
    N, K = 64, 512
    rng = np.random.default_rng(5)
    w = rng.normal(0, 1, (N, K))
    w *= 2.0 ** rng.integers(-20, 20, (N, K // 32)).repeat(32, axis=1)
    run_gemm(8, N, K, seed=9, what="spread scales", w=bf16(w))


def test_gemm_w4_full_decode_sampled_columns():
    """The decode shape X [64,4096], W [14336,4096] on 384 sampled columns
    (including the last block)."""
    cols = np.unique(np.concatenate([np.random.default_rng(1).choice(14336, 320, replace=False),
                                     np.arange(14336 - 64, 14336)]))
    run_gemm(64, 14336, 4096, seed=0, what="decode 8B", cols=cols)


def test_w4_chain_gpu_quantizers_vs_oracle_chain():
    """GPU activation quant + GPU MXFP4 weight quant + GPU GEMM against the
    oracle chain from the same BF16 inputs."""
    M, N, K = 37, 320, 1536
    x = synthetic.activations(M, K, seed=21, n_out=2)
    w = synthetic.weights(N, K, seed=21)
    say("w4 chain", M, N, K)
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    c, s = fl.fp8_mxfp4_quant_weight(bf16_to_dev(w))
    y = fl.fp8_gemm_fwd_w4(xq, sx, c, s)
    oxq, osx = oracle.quant_act(x)
    oc, os_ = oracle.mxfp4_quant(w)
    assert_same(host(xq), oxq, "chain xq")
    assert_same(host(c), oc, "chain codes")
    assert_same(host(s), os_, "chain scales")
    err = oracle.gemm_metric(bf16_bits_to_f64(host(y)), oracle.gemm_fwd_w4(oxq, osx, oc, os_))
    assert err <= TOL, err


def test_gemm_w4_degenerate():
    say("gemm_fwd_w4 degenerate")
    xq = torch.zeros((0, 256), dtype=torch.uint8, device=DEV)
    sx = torch.zeros((0, 2), dtype=torch.float32, device=DEV)
    c = torch.zeros((64, 128), dtype=torch.uint8, device=DEV)
    s = torch.zeros((64, 8), dtype=torch.uint8, device=DEV)
    assert fl.fp8_gemm_fwd_w4(xq, sx, c, s).shape == (0, 64)
    y = fl.fp8_gemm_fwd_w4(torch.zeros((3, 0), dtype=torch.uint8, device=DEV),
                           torch.zeros((3, 0), dtype=torch.float32, device=DEV),
                           torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                           torch.zeros((5, 0), dtype=torch.uint8, device=DEV))
    assert (host(y) == 0).all() and y.shape == (3, 5)
    with pytest.raises(fl.Fp8LinError, match="FP8LIN_ERR_SHAPE"):
        fl.fp8_gemm_fwd_w4(torch.zeros((2, 96), dtype=torch.uint8, device=DEV),
                           torch.zeros((2, 0), dtype=torch.float32, device=DEV),
                           torch.zeros((4, 48), dtype=torch.uint8, device=DEV),
                           torch.zeros((4, 3), dtype=torch.uint8, device=DEV))


def test_w4_rollout_step_graph_replays():
    """The rollout step (activation quantization + 4-bit GEMM) captured in a
    HIP graph: every replay, with eager work between replays, gives the eager
    result bit for bit."""
    M, N, K = 64, 2048, 4096
    x = bf16_to_dev(synthetic.activations(M, K, seed=31, n_out=4))
    c, s = fl.fp8_mxfp4_quant_weight(bf16_to_dev(synthetic.weights(N, K, seed=31)))
    xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    say("w4 graph replays", M, N, K)

    def step():
        fl.fp8_quant_act(x, out=(xq, sx))
        fl.fp8_gemm_fwd_w4(xq, sx, c, s, out=y)

    step()
    ref = host(y).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for i in range(4):
        y.zero_()
        xq.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref), "replay %d" % i
