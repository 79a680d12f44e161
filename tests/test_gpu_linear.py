"""GPU parity of fp8_linear_fwd, the one-call forward / rollout step
(1x128 activation quantization followed by the forward GEMM).

Its outputs must be bit-identical to fp8_quant_act followed by fp8_gemm_fwd,
the codes and scales bit-identical to the oracle's quantizer, and y within the
GEMM tolerance of the oracle: max |y - ref| / (|ref| + 0.01 rms(ref)) <= 1e-2."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, bf16_to_dev, first_mismatch, host, say

pytestmark = pytest.mark.gpu
G = 128
TOL = 1e-2


def separate(xd, wq, sw):
    xq, sx = fl.fp8_quant_act(xd)
    return fl.fp8_gemm_fwd(xq, sx, wq, sw), xq, sx


def assert_same(a, b, what):
    a, b = host(a), host(b)
    assert a.shape == b.shape, what
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "%s: first mismatch %s" % (
        what, first_mismatch(a, b))


# decode-sized (streaming kernel, K-split and generic small-M paths) and
# prefill-sized row counts, with ragged M
@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (17, 256, 1024), (64, 384, 2048), (33, 128, 768),
                                   (64, 128, 384), (65, 256, 512), (300, 384, 1024)])
def test_linear_fwd_matches_separate_and_oracle(M, N, K):
    x = synthetic.activations(M, K, seed=M + K)
    w = synthetic.weights(N, K, seed=M + K)
    xd = bf16_to_dev(x)
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    say("linear_fwd", M, N, K)
    y, xq, sx = fl.fp8_linear_fwd(xd, wq, sw)
    y2, xq2, sx2 = separate(xd, wq, sw)
    assert_same(xq, xq2, "xq")
    assert_same(sx, sx2, "sx")
    assert_same(y, y2, "y")
    oxq, osx = oracle.quant_act(x)
    assert np.array_equal(host(xq), oxq)
    assert np.array_equal(host(sx).view(np.uint32), osx.view(np.uint32))
    owq, osw = oracle.quant_weight(w)
    err = oracle.gemm_metric(bf16_bits_to_f64(host(y)), oracle.gemm_fwd(oxq, osx, owq, osw))
    assert err <= TOL, "metric %.3e" % err


def test_linear_fwd_graph_replays():
    """The call captured in a HIP graph: every replay, with new inputs and
    eager work between replays, equals the eager separate path."""
    M, N, K = 64, 4096, 2048
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(synthetic.weights(N, K, seed=9)))
    xd = bf16_to_dev(synthetic.activations(M, K, seed=9))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // G), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("linear_fwd graph capture")
    with torch.cuda.stream(s):
        fl.fp8_linear_fwd(xd, wq, sw, out=(y, xq, sx))            # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fl.fp8_linear_fwd(xd, wq, sw, out=(y, xq, sx))
    for r in range(4):
        xd.copy_(bf16_to_dev(synthetic.activations(M, K, seed=50 + r)))
        torch.cuda.synchronize()
        say("linear_fwd graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        y2, xq2, sx2 = separate(xd, wq, sw)
        assert_same(y, y2, "replay %d y" % r)
        assert_same(xq, xq2, "replay %d xq" % r)


def test_linear_fwd_empty_and_degenerate():
    wq0, sw0 = fl.fp8_quant_weight(bf16_to_dev(synthetic.weights(256, 512, seed=1)))
    say("linear_fwd M=0")
    y, xq, sx = fl.fp8_linear_fwd(torch.empty((0, 512), dtype=torch.bfloat16, device=DEV), wq0, sw0)
    assert y.shape == (0, 256) and xq.shape == (0, 512)
    say("linear_fwd N=0")
    x = synthetic.activations(5, 512, seed=2)
    wq_e = torch.empty((0, 512), dtype=torch.uint8, device=DEV)
    sw_e = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    y, xq, sx = fl.fp8_linear_fwd(bf16_to_dev(x), wq_e, sw_e)
    oxq, osx = oracle.quant_act(x)
    assert y.shape == (5, 0)
    assert np.array_equal(host(xq), oxq)
    assert np.array_equal(host(sx).view(np.uint32), osx.view(np.uint32))
    say("linear_fwd K=0")
    wq_k = torch.empty((256, 0), dtype=torch.uint8, device=DEV)
    sw_k = torch.empty((2, 0), dtype=torch.float32, device=DEV)
    y = torch.full((5, 256), 3.0, dtype=torch.bfloat16, device=DEV)
    fl.fp8_linear_fwd(torch.empty((5, 0), dtype=torch.bfloat16, device=DEV), wq_k, sw_k,
                      out=(y, torch.empty((5, 0), dtype=torch.uint8, device=DEV),
                           torch.empty((5, 0), dtype=torch.float32, device=DEV)))
    assert not host(y).any()
