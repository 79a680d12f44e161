"""Guard bands (canaries) around every output of the GEMMs, the transposing
quantizers and the producer operators: each output is a view inside a larger
buffer filled with a known pattern, and after the call the pattern outside the
view must be intact, while the view holds exactly what an unguarded call
writes.  Shapes are ragged where the entry point allows it, so the kernels'
tail handling runs next to the guards."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import synthetic
from gpu_util import DEV, bf16_to_dev, f32_to_dev, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
G = 128
PAD = 4096                      # bytes of guard on each side (keeps 16-byte alignment)
FILL = {torch.uint8: 0xA5, torch.bfloat16: float("nan"), torch.float32: -7.25, torch.float64: -3.5}


class Guarded:
    """An output tensor of `shape` inside a buffer with PAD bytes of pattern
    before and after it."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.pad = PAD // torch.tensor([], dtype=dtype).element_size()
        self.buf = torch.full((self.n + 2 * self.pad,), FILL[dtype], dtype=dtype, device=DEV)
        self.ref = self.buf.clone()
        self.t = self.buf[self.pad:self.pad + self.n].view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        a = self.buf.view(torch.uint8).cpu().numpy()
        b = self.ref.view(torch.uint8).cpu().numpy()
        p = PAD
        assert np.array_equal(a[:p], b[:p]), "%s: guard before the output overwritten" % what
        assert np.array_equal(a[len(a) - p:], b[len(b) - p:]), "%s: guard after the output overwritten" % what


def run(what, shapes, call, plain):
    """call(outs) writes into guarded outputs; plain() returns the same
    outputs from an unguarded call (None for a workspace); both must agree bit
    for bit."""
    say("guard bands", what)
    gs = [Guarded(s, d) for s, d in shapes]
    call([g.t for g in gs])
    for i, g in enumerate(gs):
        g.check("%s output %d" % (what, i))
    ref = plain()
    for i, (g, r) in enumerate(zip(gs, ref)):
        if r is None:                       # a workspace: contents unspecified
            continue
        assert np.array_equal(host(g.t).view(np.uint8), host(r).view(np.uint8)), \
            "%s output %d differs from an unguarded call" % (what, i)


def codes(shape, seed):
    return u8_to_dev(synthetic.random_codes(shape, seed, 1))


def scales(shape, seed):
    return f32_to_dev(synthetic.random_scales(shape, seed, 2))


u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16


@pytest.mark.parametrize("M,N,K", [(37, 384, 512), (130, 384, 640), (300, 1152, 256)])
def test_gemm_fwd_guards(M, N, K):
    xq, sx, wq, sw = codes((M, K), 1), scales((M, K // G), 1), codes((N, K), 2), scales((N // G, K // G), 2)
    run("gemm_fwd %dx%dx%d" % (M, N, K), [((M, N), bf)], lambda o: fl.fp8_gemm_fwd(xq, sx, wq, sw, out=o[0]),
        lambda: [fl.fp8_gemm_fwd(xq, sx, wq, sw)])
    run("gemm_fwd_unified %dx%dx%d" % (M, N, K), [((M, N), bf)],
        lambda o: fl.fp8_gemm_fwd_unified(xq, sx, wq, sw, out=o[0]), lambda: [fl.fp8_gemm_fwd_unified(xq, sx, wq, sw)])


@pytest.mark.parametrize("M,N,K", [(17, 1024, 2048), (64, 4096, 14336)])
def test_gemm_fwd_packed_guards(M, N, K):
    xq, sx, wq, sw = codes((M, K), 3), scales((M, K // G), 3), codes((N, K), 4), scales((N // G, K // G), 4)
    wp = fl.fp8_weight_pack(wq)
    run("gemm_fwd_packed", [((M, N), bf)], lambda o: fl.fp8_gemm_fwd_packed(xq, sx, wp, sw, out=o[0]),
        lambda: [fl.fp8_gemm_fwd_packed(xq, sx, wp, sw)])
    need = fl.fp8_gemm_fwd_packed_splitk_workspace(M, N, K)
    assert need > 0
    run("gemm_fwd_packed_splitk", [((M, N), bf), ((need // 4,), f32)],
        lambda o: fl.fp8_gemm_fwd_packed_splitk(xq, sx, wp, sw, workspace=o[1], out=o[0]),
        lambda: [fl.fp8_gemm_fwd_packed_splitk(xq, sx, wp, sw), None])
    run("gemm_fwd_packed_splitk_noalloc", [((M, N), bf)],
        lambda o: fl.fp8_gemm_fwd_packed_splitk_noalloc(xq, sx, wp, sw, out=o[0]),
        lambda: [fl.fp8_gemm_fwd_packed_splitk(xq, sx, wp, sw)])


def test_gemm_dgrad_guards():
    T, N, K = 130, 384, 256
    dyq, sdy, wq, sw = codes((T, N), 5), scales((T, N // G), 5), codes((N, K), 6), scales((N // G, K // G), 6)
    wqT, swT = fl.fp8_weight_transpose(wq, sw)
    run("gemm_dgrad", [((T, K), bf)], lambda o: fl.fp8_gemm_dgrad(dyq, sdy, wq, sw, out=o[0]),
        lambda: [fl.fp8_gemm_dgrad(dyq, sdy, wq, sw)])
    run("gemm_dgrad_t", [((T, K), bf)], lambda o: fl.fp8_gemm_dgrad_t(dyq, sdy, wqT, swT, out=o[0]),
        lambda: [fl.fp8_gemm_dgrad_t(dyq, sdy, wqT, swT)])
    run("weight_transpose", [((K, N), u8), ((K // G, N // G), f32)],
        lambda o: fl.fp8_weight_transpose(wq, sw, out=(o[0], o[1])), lambda: list(fl.fp8_weight_transpose(wq, sw)))


@pytest.mark.parametrize("N,K,T", [(200, 132, 256), (50, 136, 128), (300, 130, 384)])
def test_gemm_wgrad_guards(N, K, T):
    """The three WGrad paths: NT tiles, few rows, K % 4 != 0."""
    a, sa, b, sb = codes((N, T), 7), scales((N, T // G), 7), codes((K, T), 8), scales((K, T // G), 8)
    run("gemm_wgrad %dx%dx%d" % (N, K, T), [((N, K), bf)], lambda o: fl.fp8_gemm_wgrad(a, sa, b, sb, out=o[0]),
        lambda: [fl.fp8_gemm_wgrad(a, sa, b, sb)])


def test_gemm_w4_guards():
    M, N, K = 33, 384, 1024
    xq, sx = codes((M, K), 9), scales((M, K // G), 9)
    c4, s4 = fl.fp8_mxfp4_quant_weight(bf16_to_dev(synthetic.weights(N, K, seed=9)))
    run("gemm_fwd_w4", [((M, N), bf)], lambda o: fl.fp8_gemm_fwd_w4(xq, sx, c4, s4, out=o[0]),
        lambda: [fl.fp8_gemm_fwd_w4(xq, sx, c4, s4)])
    w = bf16_to_dev(synthetic.weights(N, K, seed=10))
    run("mxfp4_quant_weight", [((N, K // 2), u8), ((N, K // 32), u8)],
        lambda o: fl.fp8_mxfp4_quant_weight(w, out=(o[0], o[1])), lambda: list(fl.fp8_mxfp4_quant_weight(w)))


@pytest.mark.parametrize("T,C", [(256, 200), (384, 384)])
def test_quant_transpose_guards(T, C):
    x = bf16_to_dev(synthetic.activations(T, C, seed=T + C, n_out=1))
    run("quant_transpose bf16 %dx%d" % (T, C), [((C, T), u8), ((C, T // G), f32)],
        lambda o: fl.fp8_quant_transpose(x, out=(o[0], o[1], None, None)), lambda: list(fl.fp8_quant_transpose(x)))
    if C % G == 0:
        run("quant_transpose bf16 dual", [((C, T), u8), ((C, T // G), f32), ((T, C), u8), ((T, C // G), f32)],
            lambda o: fl.fp8_quant_transpose(x, dual=True, out=tuple(o)),
            lambda: list(fl.fp8_quant_transpose(x, dual=True)))
        q, s = fl.fp8_quant_act(x)
        run("quant_transpose fp8 source", [((C, T), u8), ((C, T // G), f32)],
            lambda o: fl.fp8_quant_transpose(q, s, out=(o[0], o[1], None, None)),
            lambda: list(fl.fp8_quant_transpose(q, s)))


def test_quant_weight_and_pack_guards():
    N, K = 256, 384
    w = bf16_to_dev(synthetic.weights(N, K, seed=11))
    run("quant_weight", [((N, K), u8), ((N // G, K // G), f32)],
        lambda o: fl.fp8_quant_weight(w, out=(o[0], o[1])), lambda: list(fl.fp8_quant_weight(w)))
    wq2 = codes((N, 512), 12)
    run("weight_pack", [((N, 512), u8)], lambda o: fl.fp8_weight_pack(wq2, out=o[0]),
        lambda: [fl.fp8_weight_pack(wq2)])


def test_producer_guards():
    M, K, F = 37, 640, 384
    x = bf16_to_dev(synthetic.activations(M, K, seed=12, n_out=1))
    gamma = bf16_to_dev(synthetic.norm_weights(K, seed=12))
    run("rmsnorm_quant", [((M, K), u8), ((M, K // G), f32), ((M,), f32)],
        lambda o: fl.fp8_rmsnorm_quant(x, gamma, 1e-6, out=tuple(o)), lambda: list(fl.fp8_rmsnorm_quant(x, gamma)))
    gu = bf16_to_dev(synthetic.activations(M, 2 * F, seed=13, n_out=1))
    run("swiglu_quant", [((M, F), u8), ((M, F // G), f32)],
        lambda o: fl.fp8_swiglu_quant(gu[:, :F], gu[:, F:], out=tuple(o)),
        lambda: list(fl.fp8_swiglu_quant(gu[:, :F], gu[:, F:])))
    dh = bf16_to_dev(synthetic.grad_out(M, F, seed=13))
    run("swiglu_bwd", [((M, 2 * F), bf)], lambda o: fl.fp8_swiglu_bwd(gu[:, :F], gu[:, F:], dh, out=o[0]),
        lambda: [fl.fp8_swiglu_bwd(gu[:, :F], gu[:, F:], dh)])
    T = 256
    guT = bf16_to_dev(synthetic.activations(T, 2 * F, seed=14, n_out=1))
    dhT = bf16_to_dev(synthetic.grad_out(T, F, seed=14))
    run("swiglu_bwd_quant", [((2 * F, T), u8), ((2 * F, T // G), f32), ((T, 2 * F), u8), ((T, 2 * F // G), f32)],
        lambda o: fl.fp8_swiglu_bwd_quant(guT[:, :F], guT[:, F:], dhT, out=tuple(o)),
        lambda: list(fl.fp8_swiglu_bwd_quant(guT[:, :F], guT[:, F:], dhT)))
    _, _, rstd = fl.fp8_rmsnorm_quant(x, gamma)
    dy = bf16_to_dev(synthetic.grad_out(M, K, seed=15, sigma=1.0))
    need = fl.fp8_rmsnorm_bwd_workspace(M, K)
    run("rmsnorm_bwd", [((M, K), bf), ((K,), f32), ((need // 8,), torch.float64)],
        lambda o: fl.fp8_rmsnorm_bwd(x, gamma, rstd, dy, workspace=o[2], out=(o[0], o[1])),
        lambda: list(fl.fp8_rmsnorm_bwd(x, gamma, rstd, dy)) + [None])
