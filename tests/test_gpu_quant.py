"""GPU parity of the quantization kernels against the CPU oracle: codes and
scales must be bit-identical, on small ragged shapes, adversarial groups and
the full-size tensors of the 7B/8B/32B-shaped workloads."""
import ctypes
import json
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_to_dev, f32_to_dev, first_mismatch, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
G = 128


def check_quant(q_gpu, s_gpu, q_ref, s_ref, what):
    qg, sg = host(q_gpu), host(s_gpu)
    assert qg.shape == q_ref.shape and sg.shape == s_ref.shape
    bad = first_mismatch(qg, q_ref)
    assert bad is None, "%s codes: first mismatch at %s gpu=%#x ref=%#x (%d total)" % (
        what, bad[0], bad[1], bad[2], bad[3])
    bad = first_mismatch(sg.view(np.uint32), s_ref.view(np.uint32))
    assert bad is None, "%s scales: first mismatch at %s (%d total)" % (what, bad[0], bad[3])


# --------------------------------------------------------------- encoders

_ENC = {}


def _oracle_encode_many():
    """Vectorised oracle encode: the oracle's scalar encoder driven by a small
    C loop (tests/csrc/brute_e4m3.c), multithreaded."""
    if "f" not in _ENC:
        d = tempfile.mkdtemp()
        so = os.path.join(d, "libbrute.so")
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-o", so, os.path.join(os.path.dirname(__file__), "csrc", "brute_e4m3.c"), "-lm"])
        lib = ctypes.CDLL(so)
        lib.encode_many.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        fn = ctypes.cast(oracle.lib().oracle_e4m3_encode, ctypes.c_void_p)

        def run(v):
            out = np.empty(v.size, np.uint8)
            lib.encode_many(v.ctypes.data, v.size, fn, out.ctypes.data)
            return out
        _ENC["f"] = run
    return _ENC["f"]


def test_encoder_exhaustive_all_fp32():
    """The kernels' encoder (method 0: the hardware conversion on inputs
    clamped to +-448) equals the oracle on every finite fp32 bit pattern.  The
    unclamped hardware conversion (method 1) must agree with the oracle for
    every |v| <= 464: the fast quotient reaches 448 (1 + 2^-23) unclamped, and
    464 is the midpoint that rounds to 448.  Above 464 it returns the NaN code
    (counted, not an error: no kernel passes such values)."""
    enc = _oracle_encode_many()
    chunk = 1 << 28
    stats = {"hw_mismatch_total": 0, "hw_mismatch_le464": 0, "hw_examples": []}
    for c in range((1 << 32) // chunk):
        lo = c * chunk
        say("encoder exhaustive chunk", c, "of", (1 << 32) // chunk)
        bits = torch.arange(lo, lo + chunk, dtype=torch.int64, device=DEV)
        bits = torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32)
        x = bits.view(torch.float32)
        q0 = host(fl.fp8lin_encode_e4m3(x, method=0))
        q1 = host(fl.fp8lin_encode_e4m3(x, method=1))
        del bits, x
        hb = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32)
        finite = ((hb >> np.uint32(23)) & np.uint32(0xFF)) != np.uint32(0xFF)
        ref = enc(hb.view(np.float32))
        bad = np.nonzero((q0 != ref) & finite)[0]
        assert bad.size == 0, "encoder mismatch at fp32 bits %#x: gpu %#x ref %#x (%d in chunk)" % (
            hb[bad[0]], q0[bad[0]], ref[bad[0]], bad.size)
        hw_bad = np.nonzero((q1 != ref) & finite)[0]
        stats["hw_mismatch_total"] += int(hw_bad.size)
        if hw_bad.size:
            mags = np.abs(hb[hw_bad].view(np.float32))
            stats["hw_mismatch_le464"] += int(np.sum(mags <= 464.0))
            for i in hw_bad[:: max(1, hw_bad.size // 4)][:4]:
                stats["hw_examples"].append([hex(int(hb[i])), float(hb[i:i + 1].view(np.float32)[0]),
                                             hex(int(q1[i])), hex(int(ref[i]))])
    print("hardware cvt vs definition:", json.dumps(stats))
    assert stats["hw_mismatch_le464"] == 0, stats["hw_examples"]


def test_decoder_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    ref = oracle.e4m3_decode(codes).astype(np.float32)
    qd = u8_to_dev(codes)
    for method in (0, 2):
        say("decoder method", method)
        got = host(fl.fp8lin_decode_e4m3(qd, method=method))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), method
    hw = host(fl.fp8lin_decode_e4m3(qd, method=1))
    mism = [(hex(int(c)), float(h), float(r)) for c, h, r in zip(codes, hw, ref)
            if np.float32(h).view(np.uint32) != np.float32(r).view(np.uint32)]
    print("hardware decode mismatches:", len(mism), mism[:8])
    assert not mism, mism[:8]


# ----------------------------------------------------------- 1x128 groups

def adversarial_bf16(rows=12, cols=1024, seed=0):
    g = np.random.default_rng(seed)
    out = []
    mags = oracle.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    out.append(np.zeros(cols, np.float32))
    out.append(-np.zeros(cols, np.float32))
    r = np.zeros(cols, np.float32); r[3] = -7.0; r[cols - 5] = 1e-30; out.append(r)
    out.append(g.standard_normal(cols).astype(np.float32))
    out.append(g.standard_normal(cols).astype(np.float32) * np.float32(1e-38))     # subnormal bf16
    out.append(g.standard_normal(cols).astype(np.float32) * np.float32(1e-30))     # tiny scales
    out.append(g.standard_normal(cols).astype(np.float32) * np.float32(3e37))      # huge
    r = g.choice(mids, cols).astype(np.float32); r[::G] = 448.0; out.append(r)    # exact ties
    r = (g.choice(mags, cols) * 2.0 ** g.integers(-30, 30)).astype(np.float32); r[::G] = -448.0 * 2.0 ** 3
    out.append(r)
    r = g.standard_normal(cols).astype(np.float32); r[5::G] = -30.0; out.append(r)  # negative amax
    while len(out) < rows:
        out.append(g.standard_normal(cols).astype(np.float32) * np.float32(10.0 ** g.integers(-20, 20)))
    return synthetic.f32_to_bf16_bits(np.stack(out[:rows]))


@pytest.mark.parametrize("M,K", [(1, 128), (7, 256), (64, 1024), (129, 384), (300, 2048)])
def test_quant_act_small(M, K):
    x = synthetic.activations(M, K, seed=M + K, n_out=max(1, K // 256))
    say("quant_act", M, K)
    q, s = fl.fp8_quant_act(bf16_to_dev(x))
    check_quant(q, s, *oracle.quant_act(x), "quant_act %dx%d" % (M, K))


def test_quant_act_adversarial():
    x = adversarial_bf16()
    say("quant_act adversarial")
    q, s = fl.fp8_quant_act(bf16_to_dev(x))
    check_quant(q, s, *oracle.quant_act(x), "quant_act adversarial")


@pytest.mark.parametrize("name,M,K,kind", [
    ("decode X", 64, 4096, "x"), ("prefill X", 8192, 3584, "x"), ("large X", 16384, 5120, "x"),
    ("backward dY", 8192, 14336, "dy")])
def test_quant_act_full_size(name, M, K, kind):
    x = synthetic.activations(M, K, seed=0) if kind == "x" else synthetic.grad_out(M, K, seed=0)
    say("quant_act full", name)
    q, s = fl.fp8_quant_act(bf16_to_dev(x))
    check_quant(q, s, *oracle.quant_act(x), name)


def test_quant_act_empty_and_zero():
    say("quant_act empty")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s = fl.fp8_quant_act(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)
    z = np.zeros((3, 256), np.uint16)
    z[1] = 0x8000
    q, s = fl.fp8_quant_act(bf16_to_dev(z))
    check_quant(q, s, *oracle.quant_act(z), "zeros")


def test_quant_act_metamorphic():
    x = synthetic.activations(64, 1024, seed=3, n_out=4)
    say("quant_act metamorphic")
    q0, s0 = (host(t) for t in fl.fp8_quant_act(bf16_to_dev(x)))
    q1, s1 = (host(t) for t in fl.fp8_quant_act(bf16_to_dev(x ^ np.uint16(0x8000))))
    assert np.array_equal(q1, q0 ^ 0x80) and np.array_equal(s1, s0)
    xf = synthetic.bf16_bits_to_f32(x)
    for j in (-9, 5):
        q2, s2 = (host(t) for t in fl.fp8_quant_act(bf16_to_dev(synthetic.f32_to_bf16_bits(xf * 2.0 ** j))))
        assert np.array_equal(q2, q0) and np.array_equal(s2, (s0 * np.float32(2.0 ** j)).astype(np.float32))
    q3, s3 = (host(t) for t in fl.fp8_quant_act(bf16_to_dev(x[17:40])))
    assert np.array_equal(q3, q0[17:40]) and np.array_equal(s3, s0[17:40])


def test_quant_act_guard_bands():
    """Outputs are written inside their tensors only (canaries around them)."""
    M, K = 65, 384
    x = synthetic.activations(M, K, seed=8, n_out=2)
    qbuf = torch.full((M * K + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((M * K // G + 1024,), -7.0, dtype=torch.float32, device=DEV)
    q = qbuf[2048:2048 + M * K].view(M, K)
    s = sbuf[512:512 + M * K // G].view(M, K // G)
    say("quant_act guard bands")
    fl.fp8_quant_act(bf16_to_dev(x), out=(q, s))
    qh, sh = host(qbuf), host(sbuf)
    assert np.all(qh[:2048] == 0xA5) and np.all(qh[2048 + M * K:] == 0xA5)
    assert np.all(sh[:512] == -7.0) and np.all(sh[512 + M * K // G:] == -7.0)
    check_quant(q, s, *oracle.quant_act(x), "guarded")


# --------------------------------------------------------- 128x128 blocks

@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (1024, 1024)])
def test_quant_weight_small(N, K):
    w = synthetic.weights(N, K, seed=N + K)
    say("quant_weight", N, K)
    q, s = fl.fp8_quant_weight(bf16_to_dev(w))
    check_quant(q, s, *oracle.quant_weight(w), "quant_weight %dx%d" % (N, K))


def test_quant_weight_adversarial():
    w = np.concatenate([adversarial_bf16(12, 256, seed=1).repeat(11, axis=0)[:128],
                        synthetic.weights(128, 256, seed=2)])
    say("quant_weight adversarial")
    q, s = fl.fp8_quant_weight(bf16_to_dev(w))
    check_quant(q, s, *oracle.quant_weight(w), "quant_weight adversarial")


@pytest.mark.parametrize("name,N,K", [("8B up-proj W", 14336, 4096), ("7B W", 18944, 3584),
                                      ("32B W", 27648, 5120)])
def test_quant_weight_full_size(name, N, K):
    w = synthetic.weights(N, K, seed=0)
    say("quant_weight full", name)
    q, s = fl.fp8_quant_weight(bf16_to_dev(w))
    check_quant(q, s, *oracle.quant_weight(w), name)


# ------------------------------------------------- transpose along tokens

@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (14336, 4096)])
def test_weight_transpose(N, K):
    """fp8_weight_transpose of the GPU weight quantization equals the oracle's
    codes and block scales, transposed, bit for bit."""
    w = synthetic.weights(N, K, seed=N + K)
    say("weight transpose", N, K)
    wq, sw = fl.fp8_quant_weight(bf16_to_dev(w))
    wqT, swT = fl.fp8_weight_transpose(wq, sw)
    oq, osc = oracle.quant_weight(w)
    assert np.array_equal(host(wqT), np.ascontiguousarray(oq.T))
    assert np.array_equal(host(swT).view(np.uint32), np.ascontiguousarray(osc.T).view(np.uint32))


@pytest.mark.parametrize("T,C", [(128, 1), (128, 77), (256, 200), (384, 256), (128, 1000)])
def test_quant_transpose_bf16_small(T, C):
    x = synthetic.activations(T, C, seed=T + C, n_out=1)
    say("quant_transpose bf16", T, C)
    qT, sT = fl.fp8_quant_transpose(bf16_to_dev(x))
    check_quant(qT, sT, *oracle.quant_transpose_bf16(x), "transpose %dx%d" % (T, C))


def test_quant_transpose_bf16_adversarial():
    # each column is one adversarial pattern running down 3 token groups
    x = np.ascontiguousarray(adversarial_bf16(12, 128 * 3, seed=4).T)
    say("quant_transpose adversarial")
    qT, sT = fl.fp8_quant_transpose(bf16_to_dev(x))
    check_quant(qT, sT, *oracle.quant_transpose_bf16(x), "transpose adversarial")


@pytest.mark.parametrize("T,C", [(128, 128), (384, 512)])
def test_quant_transpose_dual_small(T, C):
    x = synthetic.grad_out(T, C, seed=T + C)
    say("quant_transpose dual", T, C)
    qT, sT, qr, sr = fl.fp8_quant_transpose(bf16_to_dev(x), dual=True)
    check_quant(qT, sT, *oracle.quant_transpose_bf16(x), "dual transposed")
    check_quant(qr, sr, *oracle.quant_act(x), "dual rows")


def test_quant_transpose_dual_full_dy():
    T, N = 8192, 14336
    dy = synthetic.grad_out(T, N, seed=0)
    say("quant_transpose dual full dY")
    qT, sT, qr, sr = fl.fp8_quant_transpose(bf16_to_dev(dy), dual=True)
    check_quant(qT, sT, *oracle.quant_transpose_bf16(dy), "dY^T")
    check_quant(qr, sr, *oracle.quant_act(dy), "dY rows")


@pytest.mark.parametrize("T,C", [(128, 128), (384, 256), (8192, 4096)])
def test_quant_transpose_fp8(T, C):
    """Saved-activation path: X bf16 -> 1x128 FP8 (the forward's saved
    activations) -> transposed 128-along-T requantization."""
    x = synthetic.activations(T, C, seed=0)
    xq, sx = oracle.quant_act(x)
    say("quant_transpose fp8", T, C)
    qT, sT = fl.fp8_quant_transpose(u8_to_dev(xq), f32_to_dev(sx))
    check_quant(qT, sT, *oracle.quant_transpose_fp8(xq, sx), "fp8 transpose %dx%d" % (T, C))


def test_saved_activation_flow_end_to_end():
    """GPU forward quantization feeds the GPU transpose-requant (the FP8 saved
    activations of the forward pass), compared with the oracle chain."""
    x = synthetic.activations(256, 512, seed=6)
    say("saved activation flow")
    xq, sx = fl.fp8_quant_act(bf16_to_dev(x))
    qT, sT = fl.fp8_quant_transpose(xq, sx)
    oq, os_ = oracle.quant_act(x)
    check_quant(qT, sT, *oracle.quant_transpose_fp8(oq, os_), "saved flow")
