"""Pins of the oracle's quantizers (1x128 groups, 128x128 blocks, 128-along-T
transposed groups) against library routines, invariants and special cases."""
import numpy as np
import pytest
import torch

import oracle
import synthetic

G = 128


def bf16(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f32(bits):
    return synthetic.bf16_bits_to_f32(bits)


def library_group_quant(vals_f32: np.ndarray):
    """Independent route for one group along the last axis, built only from
    numpy's IEEE float32 arithmetic and torch's float8_e4m3fn cast."""
    a = np.max(np.abs(vals_f32), axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        s = (a / np.float32(448.0)).astype(np.float32)
        t = (vals_f32 / s).astype(np.float32)
    t = np.clip(t, -448.0, 448.0)                      # only rounding can exceed 448
    zero = (a == 0)
    t = np.where(zero, vals_f32, t)                    # all-zero group: keep the signed zeros
    codes = torch.from_numpy(np.ascontiguousarray(t)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, np.where(zero, np.float32(0), s)[..., 0]


def adversarial_rows(seed=0):
    """Rows of 1024 bf16 values covering the corner cases of a group."""
    g = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(1024, np.float32))                          # all-zero groups
    r = np.zeros(1024, np.float32); r[5] = -3.0; r[300] = 1e-30; rows.append(r)   # single non-zero
    rows.append(-np.zeros(1024, np.float32))                          # all negative zeros
    rows.append(g.standard_normal(1024).astype(np.float32))           # plain Gaussian
    r = g.standard_normal(1024).astype(np.float32); r[::97] *= 50; rows.append(r)  # outliers
    rows.append(g.standard_normal(1024).astype(np.float32) * np.float32(1e-38))   # bf16 subnormals
    rows.append(g.standard_normal(1024).astype(np.float32) * np.float32(1e30))    # huge
    # E4M3 values times powers of two: lossless groups with exact ties nearby
    mags = torch.arange(0, 127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    r = g.choice(mags, 1024) * np.where(g.random(1024) < 0.5, -1, 1)
    r[::128] = 448.0
    rows.append((r * 2.0 ** g.integers(-20, 20)).astype(np.float32))
    # group amax attained only by a negative value
    r = g.standard_normal(1024).astype(np.float32); r[::128] = -20.0; rows.append(r)
    # midpoints of E4M3 values relative to a scale of exactly 1 (amax 448)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    r = g.choice(mids, 1024).astype(np.float32); r[::128] = 448.0; rows.append(r)
    return np.stack(rows)


def test_quant_act_matches_library_route():
    rows = adversarial_rows()
    x = np.concatenate([bf16(rows), synthetic.activations(64, 1024, seed=5, n_out=4)])
    q, s = oracle.quant_act(x)
    xf = f32(x).reshape(x.shape[0], -1, G)
    cq, cs = library_group_quant(xf)
    assert np.array_equal(q, cq.reshape(q.shape))
    assert np.array_equal(s.view(np.uint32), cs.astype(np.float32).view(np.uint32))


def _check_invariants(q, s, vals, group_view):
    """vals/q/s reshaped so that axis -1 is one group."""
    dec = oracle.e4m3_decode(q)
    nz = np.any(vals != 0, axis=-1)
    # every non-zero group reaches the maximum magnitude 448
    assert np.all(np.max(np.abs(dec), axis=-1)[nz] == 448.0)
    assert np.all(s[~nz] == 0)
    # never the NaN codes
    assert not np.any((q & 0x7F) == 0x7F)
    # per-element error: |dec*s - x| <= 1/2 ulp_E4M3(x/s) * s * (1 + 2^-19)
    sd = s.astype(np.float64)[..., None]
    t = np.abs(vals.astype(np.float64)) / np.where(sd == 0, 1, sd)
    e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    err = np.abs(dec * sd - vals)
    bound = 0.5 * ulp * sd * (1 + 2.0 ** -19)
    assert np.all(err <= bound)


def test_quant_act_invariants():
    rows = adversarial_rows(1)
    x = np.concatenate([bf16(rows), synthetic.activations(32, 1024, seed=2, n_out=4)])
    q, s = oracle.quant_act(x)
    vals = f32(x).astype(np.float64).reshape(x.shape[0], -1, G)
    _check_invariants(q.reshape(vals.shape), s, vals, None)


def test_quant_scale_covariance():
    """Scaling the input by 2^j keeps the codes and scales the scales by 2^j
    exactly (away from fp32 under/overflow)."""
    x = synthetic.activations(16, 1024, seed=9, n_out=4)
    q0, s0 = oracle.quant_act(x)
    for j in (-30, -3, 1, 7, 40):
        xj = bf16(f32(x) * np.float32(2.0 ** j))
        qj, sj = oracle.quant_act(xj)
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_quant_sign_flip():
    x = synthetic.activations(8, 512, seed=4, n_out=1)
    q0, s0 = oracle.quant_act(x)
    q1, s1 = oracle.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(q1, q0 ^ 0x80) and np.array_equal(s1, s0)


def test_quant_rows_independent():
    """1x128 groups lie inside a row: quantizing a slice of rows alone gives
    the same codes (the unified rollout/training flow relies on this)."""
    x = synthetic.activations(300, 1024, seed=3, n_out=4)
    q, s = oracle.quant_act(x)
    q2, s2 = oracle.quant_act(x[37:101])
    assert np.array_equal(q2, q[37:101]) and np.array_equal(s2, s[37:101])


def test_quant_weight_equals_row_quant_when_rows_share_amax():
    """Special case: if every 1x128 row-group of a 128x128 block contains the
    block's amax, block quantization equals row-group quantization."""
    g = np.random.default_rng(11)
    w = g.standard_normal((256, 384)).astype(np.float32)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * G:(bi + 1) * G, bj * G:(bj + 1) * G]
            amax = np.float32(np.max(np.abs(blk)) * 1.5)
            cols = g.integers(0, G, size=G)
            blk[np.arange(G), cols] = amax * np.where(g.random(G) < 0.5, -1, 1)
    wb = bf16(w)
    qb, sb = oracle.quant_weight(wb)
    qr, sr = oracle.quant_act(wb)
    assert np.array_equal(qb, qr)
    for bi in range(2):
        for bj in range(3):
            assert np.all(sr[bi * G:(bi + 1) * G, bj] == sb[bi, bj])


def test_quant_weight_block_permutation():
    """Permuting elements inside a block permutes its codes and keeps its
    scale; other blocks are untouched."""
    w = synthetic.weights(256, 256, seed=1)
    q, s = oracle.quant_weight(w)
    g = np.random.default_rng(2)
    perm = g.permutation(G * G)
    w2 = w.copy()
    blk = w2[:G, G:].reshape(-1)[perm].reshape(G, G)
    w2[:G, G:] = blk
    q2, s2 = oracle.quant_weight(w2)
    assert np.array_equal(q2[:G, G:], q[:G, G:].reshape(-1)[perm].reshape(G, G))
    assert np.array_equal(s2, s)
    assert np.array_equal(q2[G:], q[G:]) and np.array_equal(q2[:G, :G], q[:G, :G])


def test_quant_weight_invariants_and_library_route():
    w = np.concatenate([synthetic.weights(256, 384, seed=3),
                        bf16(adversarial_rows(4)[:, :384].repeat(13, axis=0)[:128])])
    q, s = oracle.quant_weight(w)
    # rearrange into blocks: [bi, bj, 128*128]
    def blocks(a):
        R, C = a.shape
        return a.reshape(R // G, G, C // G, G).transpose(0, 2, 1, 3).reshape(R // G, C // G, G * G)
    vals = blocks(f32(w).astype(np.float64))
    _check_invariants(blocks(q), s, vals, None)
    cq, cs = library_group_quant(blocks(f32(w)))
    assert np.array_equal(blocks(q), cq) and np.array_equal(s, cs)


@pytest.mark.parametrize("T,C", [(128, 1), (256, 77), (384, 256)])
def test_transpose_bf16_equals_act_quant_of_transpose(T, C):
    x = synthetic.activations(T, C, seed=T + C, n_out=1)
    qT, sT = oracle.quant_transpose_bf16(x)
    q, s = oracle.quant_act(np.ascontiguousarray(x.T))
    assert np.array_equal(qT, q) and np.array_equal(sT, s)


def test_transpose_fp8_invariants():
    """FP8-source transpose-requant: parity unpinned by the pages; only the
    invariants of the quantizer relative to v = fp32(dec(q) * s_row) apply."""
    x = synthetic.activations(384, 256, seed=12, n_out=2)
    xq, sx = oracle.quant_act(x)
    qT, sT = oracle.quant_transpose_fp8(xq, sx)
    v = (oracle.e4m3_decode(xq).astype(np.float32) * np.repeat(sx, G, axis=1)).astype(np.float32)
    vT = v.T.astype(np.float64).reshape(256, -1, G)
    _check_invariants(qT.reshape(vT.shape), sT, vT, None)
    # and it equals the BF16-free route: requantizing v with the library route
    cq, cs = library_group_quant(np.ascontiguousarray(v.T).reshape(256, -1, G))
    assert np.array_equal(qT.reshape(cq.shape), cq) and np.array_equal(sT, cs)


def test_quant_zero_and_empty():
    q, s = oracle.quant_act(np.zeros((0, 256), np.uint16))
    assert q.shape == (0, 256) and s.shape == (0, 2)
    x = np.zeros((2, 128), np.uint16)
    x[1] = 0x8000
    q, s = oracle.quant_act(x)
    assert np.all(q[0] == 0) and np.all(q[1] == 0x80) and np.all(s == 0)
