"""GPU parity of the producer operators fused with 1x128 quantization
(fp8_rmsnorm_quant, fp8_swiglu_quant) against the CPU oracle: codes, scales
and rstd must be bit-identical, on small ragged shapes, adversarial rows and
the full-size 8B/32B-shaped tensors.  For SwiGLU an element whose exact value
lies next to a BF16 rounding midpoint (flagged by the oracle) may round either
way; a group holding one must equal the quantization of one of its valid
roundings."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_to_dev, first_mismatch, host, say
from near_tie import check_rowq_near_ties

pytestmark = pytest.mark.gpu
G = 128


def bf16(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def gamma_for(K, seed):
    g = np.random.default_rng(seed).uniform(0.25, 1.75, K).astype(np.float32)
    g[::17] *= -1.0
    return bf16(g)


def assert_same(gpu, ref, what):
    bad = first_mismatch(gpu, ref)
    assert bad is None, "%s: first mismatch at %s gpu=%r ref=%r (%d total)" % (what, bad[0], bad[1], bad[2], bad[3])


def run_rmsnorm(x, gamma, eps, what, with_rstd=True):
    say("rmsnorm_quant", what, x.shape, eps)
    q, s, r = fl.fp8_rmsnorm_quant(bf16_to_dev(x), bf16_to_dev(gamma), eps, rstd=with_rstd)
    oq, os_, orr = oracle.rmsnorm_quant(x, gamma, eps)
    assert_same(host(q), oq, what + " codes")
    assert_same(host(s).view(np.uint32), os_.view(np.uint32), what + " scales")
    if with_rstd:
        assert_same(host(r).view(np.uint32), orr.view(np.uint32), what + " rstd")
    else:
        assert r is None


@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (33, 1024), (7, 640), (17, 3584), (64, 4096),
                                 (9, 5120), (3, 8192), (2, 12288), (2, 16384)])
def test_rmsnorm_quant_shapes(M, K):
    """Every register-pass count (K up to 512, 1024, ..., 16384), K not a
    multiple of 512, row counts not a multiple of the 4 rows per workgroup."""
    x = synthetic.activations(M, K, seed=M + K, n_out=max(1, K // 1024))
    run_rmsnorm(x, gamma_for(K, K), 1e-6, "%dx%d" % (M, K), with_rstd=(M % 2 == 1))


def test_rmsnorm_quant_adversarial_rows():
    """Zero rows (eps > 0), rows of +-2^e, huge and tiny magnitudes, a single
    non-zero value, negative zeros, and eps = 0 on non-zero rows."""
    K = 1024
    rng = np.random.default_rng(5)
    rows = [np.zeros(K, np.float32), np.full(K, -0.0, np.float32),
            np.where(rng.random(K) < 0.5, -1.0, 1.0).astype(np.float32) * 2.0 ** -40,
            rng.normal(0, 1e30, K).astype(np.float32), rng.normal(0, 1e-30, K).astype(np.float32)]
    one = np.zeros(K, np.float32)
    one[700] = -3.5
    rows.append(one)
    mixed = rng.normal(0, 1, K).astype(np.float32)
    mixed[::5] = 0.0
    mixed[3] = 1e4
    rows.append(mixed)
    x = bf16(np.stack(rows))
    run_rmsnorm(x, gamma_for(K, 1), 1e-5, "adversarial")
    run_rmsnorm(x[2:], gamma_for(K, 2), 0.0, "adversarial eps=0")


@pytest.mark.parametrize("name,M,K", [("8B hidden", 8192, 4096), ("decode 8B", 64, 4096),
                                      ("7B hidden", 8192, 3584), ("32B hidden", 16384, 5120)])
def test_rmsnorm_quant_full_size(name, M, K):
    x = synthetic.activations(M, K, seed=0, n_out=synthetic.n_outliers(K))
    run_rmsnorm(x, gamma_for(K, 0), 1e-6, name)


def test_rmsnorm_quant_degenerate():
    say("rmsnorm_quant empty")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(256, dtype=torch.bfloat16, device=DEV)
    q, s, r = fl.fp8_rmsnorm_quant(x, g)
    assert q.shape == (0, 256) and s.shape == (0, 2) and r.shape == (0,)
    with pytest.raises(fl.Fp8LinError, match="FP8LIN_ERR_ARG"):
        fl.fp8_rmsnorm_quant(torch.ones((2, 256), dtype=torch.bfloat16, device=DEV), g, eps=-1.0)


# ------------------------------------------------------------------ SwiGLU

def compare_swiglu(q, s, gate, up, what):
    """Codes and scales bit-exact in every group without a near-tie element;
    a group holding some must be the quantization of the group with each
    flagged element at one of its candidate BF16 values (near_tie.py)."""
    h, near = oracle.swiglu_bf16(gate, up)
    n = check_rowq_near_ties(h, near, host(q), host(s), what)
    if n:
        print("[%s] %d group(s) hold a near-tie element; each matched one valid rounding" % (what, n))


@pytest.mark.parametrize("M,F", [(1, 128), (3, 384), (37, 1024), (64, 14336), (130, 2048)])
def test_swiglu_quant_shapes(M, F):
    gate = synthetic.activations(M, F, seed=F + 1, n_out=max(1, F // 1024))
    up = synthetic.activations(M, F, seed=F + 2, n_out=0)
    say("swiglu_quant", M, F)
    q, s = fl.fp8_swiglu_quant(bf16_to_dev(gate), bf16_to_dev(up))
    compare_swiglu(q, s, gate, up, "%dx%d" % (M, F))


def test_swiglu_quant_halves_of_one_tensor():
    """gate and up as the two halves of one [M, 2F] projection output (row
    stride 2F)."""
    M, F = 45, 1536
    gu = synthetic.activations(M, 2 * F, seed=77, n_out=3)
    say("swiglu_quant halves", M, F)
    t = bf16_to_dev(gu)
    q, s = fl.fp8_swiglu_quant(t[:, :F], t[:, F:])
    compare_swiglu(q, s, np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]), "halves")


def test_swiglu_quant_special_values():
    """Zeros of both signs, large positive and negative gates, tiny products
    that round into BF16 subnormals or to zero."""
    rng = np.random.default_rng(9)
    F = 1024
    gate = rng.normal(0, 1, (6, F)).astype(np.float32)
    up = rng.normal(0, 1, (6, F)).astype(np.float32)
    gate[0] = 0.0
    gate[1, ::2] = -0.0
    gate[2] = rng.uniform(60, 300, F) * np.where(rng.random(F) < 0.5, -1, 1)
    up[3] *= 1e-36
    gate[4] *= 1e-20
    up[5] = 0.0
    up[5, 7] = 2.0
    gb, ub = bf16(gate), bf16(up)
    say("swiglu_quant special")
    q, s = fl.fp8_swiglu_quant(bf16_to_dev(gb), bf16_to_dev(ub))
    compare_swiglu(q, s, gb, ub, "special")


def test_swiglu_quant_full_size():
    """8B MLP intermediate: gate, up [8192, 14336]."""
    M, F = 8192, 14336
    gate = synthetic.activations(M, F, seed=1, n_out=synthetic.n_outliers(F))
    up = synthetic.activations(M, F, seed=2, n_out=0)
    say("swiglu_quant full", M, F)
    q, s = fl.fp8_swiglu_quant(bf16_to_dev(gate), bf16_to_dev(up))
    compare_swiglu(q, s, gate, up, "8B intermediate")


def test_swiglu_quant_degenerate():
    say("swiglu_quant empty")
    z = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s = fl.fp8_swiglu_quant(z, z)
    assert q.shape == (0, 256) and s.shape == (0, 2)


# -------------------------------------------------------- RMSNorm backward

def run_rmsnorm_bwd(M, K, seed, what, with_dgamma=True):
    x = synthetic.activations(M, K, seed=seed, n_out=max(1, K // 1024))
    gamma = synthetic.norm_weights(K, seed=seed)
    dy = synthetic.grad_out(M, K, seed=seed, sigma=1.0)
    _, rstd = oracle.rmsnorm_bf16(x, gamma, 1e-6)           # the forward's rstd (oracle-made input)
    odx, odg = oracle.rmsnorm_bwd(x, gamma, rstd, dy)
    say("rmsnorm_bwd", what, M, K)
    dx, dg = fl.fp8_rmsnorm_bwd(bf16_to_dev(x), bf16_to_dev(gamma), torch.from_numpy(rstd).to(DEV), bf16_to_dev(dy),
                                dgamma=with_dgamma)
    assert_same(host(dx), odx, what + " dx")
    if with_dgamma:
        assert_same(host(dg).view(np.uint32), odg.view(np.uint32), what + " dgamma")
    else:
        assert dg is None


@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (130, 1024), (300, 4096), (9, 5120), (3, 3584),
                                 (129, 16384)])
def test_rmsnorm_bwd_shapes(M, K):
    """dx and dgamma bit-exact: every pass count, K not a multiple of 2048,
    token counts that leave a short last block of 128."""
    run_rmsnorm_bwd(M, K, M + K, "%dx%d" % (M, K), with_dgamma=(M != 9))


def test_rmsnorm_bwd_full_size():
    run_rmsnorm_bwd(8192, 4096, 0, "8B hidden")
