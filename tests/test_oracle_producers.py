"""Pins of the oracle's producer operators (RMSNorm and SwiGLU in front of a
linear layer, each followed by 1x128 quantization of its BF16 output).

The pages only name these operators (fused activation / RMSNorm kernels, FP8
activations produced fused with the previous operator); the oracle takes the
textbook forms with the precision of every step fixed.  The pins below check
it against exact rational arithmetic (Fraction / Decimal), library routines
(numpy fp32 products, torch's bf16 cast and silu) and closed forms.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch

import oracle
import synthetic

G = 128


def bf16(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f32(bits):
    return synthetic.bf16_bits_to_f32(bits)


def torch_bf16_bits(a_f32):
    """fp32 -> bf16 (round to nearest even) through torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def round_fraction(q: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Nearest value with `mant_bits` significant bits (exponent floor min_exp,
    i.e. gradual underflow), ties to even, of a rational q."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # now 2^e <= a < 2^(e+1)
    e = max(e, min_exp)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def midpoint_distance(q: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """|q - nearest rounding midpoint| / |q| for the given format."""
    a = abs(q)
    if a == 0:
        return Fraction(1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, min_exp)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = a / quantum
    frac = n - (n.numerator // n.denominator)
    return abs(frac - Fraction(1, 2)) * quantum / a


# ------------------------------------------------------------------ RMSNorm

def fp32_inv_sqrt(A: Fraction):
    """fp32 nearest to 1/sqrt(A) exactly (A > 0), and the relative distance of
    1/sqrt(A) from the rounding boundary it was closest to."""
    approx = np.float32(1.0 / math.sqrt(float(A)))
    c = [approx]
    for _ in range(3):
        c.insert(0, np.nextafter(c[0], np.float32(0)))
        c.append(np.nextafter(c[-1], np.float32(np.inf)))
    # r >= mid  <=>  mid^2 * A <= 1 ; the candidates bracket r
    best, margin = None, None
    for lo, hi in zip(c[:-1], c[1:]):
        mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
        t = mid * mid * A
        if t <= 1:
            best = hi                                # r >= mid: hi or beyond
        elif best is None:
            best = lo
        d = abs(t - 1)
        margin = d if margin is None else min(margin, d)
    return best, margin


def test_rmsnorm_rstd_is_rounded_exact_value():
    """rstd equals fp32 of the exact 1/sqrt(sum(x^2)/K + eps), computed with
    rationals: pins the sum of squares (every term, every index), the mean's
    denominator, where eps enters, the square root and the reciprocal."""
    M, K = 24, 512
    x = synthetic.activations(M, K, seed=3, n_out=2)
    x[5] = bf16(np.linspace(-1e-3, 2e-3, K))                    # small magnitudes
    x[6] = bf16(np.where(np.arange(K) % 7 == 0, 1e4, 1e-4))    # wide exponent spread
    gamma = bf16(np.ones(K))
    for eps in (1e-6, 0.25):
        _, rstd = oracle.rmsnorm_bf16(x, gamma, eps)
        xf = f32(x).astype(np.float64)
        for m in range(M):
            ss = sum(Fraction(float(v)) ** 2 for v in xf[m])
            A = ss / K + Fraction(float(np.float32(eps)))
            want, margin = fp32_inv_sqrt(A)
            if margin < Fraction(1, 2 ** 40):
                continue                              # within fp64 evaluation error of a tie
            assert rstd[m] == want, (m, eps, rstd[m], want)


def test_rmsnorm_output_from_library_products():
    """y = bf16(fp32(fp32(x * rstd) * gamma)) with numpy's IEEE fp32 products
    and torch's bf16 cast, elementwise (a shifted or transposed gamma index,
    or a missing product, fails)."""
    M, K = 16, 1024
    x = synthetic.activations(M, K, seed=4, n_out=3)
    gamma = bf16(np.random.default_rng(7).uniform(-2, 2, K).astype(np.float32))
    y, rstd = oracle.rmsnorm_bf16(x, gamma, 1e-5)
    t = (f32(x) * rstd[:, None]).astype(np.float32)
    u = (t * f32(gamma)[None, :]).astype(np.float32)
    assert np.array_equal(y, torch_bf16_bits(u))


def test_rmsnorm_unit_mean_square():
    """With gamma = 1 and eps = 0 the output has mean square 1 up to the bf16
    rounding of each element (relative error <= 2^-8 each)."""
    M, K = 32, 4096
    x = synthetic.activations(M, K, seed=5, n_out=4)
    y, _ = oracle.rmsnorm_bf16(x, bf16(np.ones(K)), 0.0)
    ms = np.mean(f32(y).astype(np.float64) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) <= 2.0 ** -7), ms


def test_rmsnorm_closed_forms():
    """Rows of +-2^e: the mean square is 4^e, rstd = 2^-e exactly, y = +-gamma.
    eps = 0: scaling x by a power of two leaves y unchanged bit for bit.
    An all-zero row with eps > 0 gives signed-zero outputs."""
    K = 256
    gamma = bf16(np.random.default_rng(1).normal(0, 1, K).astype(np.float32))
    signs = np.where(np.random.default_rng(2).random(K) < 0.5, -1.0, 1.0)
    for e in (-20, -3, 0, 5, 30):
        x = bf16((signs * 2.0 ** e)[None, :])
        y, rstd = oracle.rmsnorm_bf16(x, gamma, 0.0)
        assert rstd[0] == np.float32(2.0 ** -e)
        want = np.where(signs < 0, gamma ^ np.uint16(0x8000), gamma)
        assert np.array_equal(y[0], want)
    x = synthetic.activations(8, K, seed=6, n_out=1)
    y0, r0 = oracle.rmsnorm_bf16(x, gamma, 0.0)
    for j in (-12, -1, 3, 40):
        xs = bf16(f32(x) * np.float32(2.0 ** j))
        assert np.array_equal(f32(xs), f32(x) * np.float32(2.0 ** j))   # exact scaling
        yj, rj = oracle.rmsnorm_bf16(xs, gamma, 0.0)
        assert np.array_equal(yj, y0)
        assert np.array_equal(rj, r0 * np.float32(2.0 ** -j))
    z = np.zeros((2, K), np.uint16)
    z[1, ::3] = 0x8000                                          # -0 entries
    y, rstd = oracle.rmsnorm_bf16(z, gamma, 1e-6)
    assert np.all((y & 0x7FFF) == 0)
    q, s, _ = oracle.rmsnorm_quant(z, gamma, 1e-6)
    assert np.all(s == 0) and np.all((q & 0x7F) == 0)


def test_rmsnorm_quant_is_quant_of_output():
    """The fused result is quant_act of the BF16 RMSNorm output, and every
    non-zero group reaches code magnitude 448."""
    M, K = 8, 3584
    x = synthetic.activations(M, K, seed=8, n_out=4)
    gamma = bf16(np.random.default_rng(3).uniform(0.5, 1.5, K).astype(np.float32))
    q, s, r = oracle.rmsnorm_quant(x, gamma, 1e-6)
    y, r2 = oracle.rmsnorm_bf16(x, gamma, 1e-6)
    q2, s2 = oracle.quant_act(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(r, r2)
    mags = (q & 0x7F).reshape(M, K // G, G).max(axis=2)
    assert np.all(mags == 0x7E)


# ------------------------------------------------------------------- SwiGLU

def exact_swiglu_bf16(gv: float, uv: float):
    """bf16 of g*u/(1+exp(-g)) from 60-digit decimal arithmetic, and the
    value's relative distance to the nearest bf16 rounding midpoint."""
    getcontext().prec = 60
    g, u = Decimal(gv), Decimal(uv)
    v = g * u / (1 + (-g).exp())
    q = Fraction(v)
    return round_fraction(q, 8, -126), midpoint_distance(q, 8, -126)


def swiglu_cases():
    g = np.random.default_rng(11)
    gate = np.concatenate([
        g.normal(0, 1, 4000), g.normal(0, 1, 500) * 50, g.uniform(-20, 20, 500),
        np.array([0.0, -0.0, 1.0, -1.0, 128.0, -128.0, 88.0, -88.0, 700.0, -700.0, 1e-30, -1e-30]),
    ]).astype(np.float32)
    up = np.concatenate([
        g.normal(0, 1, 4000), g.normal(0, 1, 500), g.normal(0, 3, 500),
        np.array([1.0, 1.0, -2.0, 3.0, 1.0, 1.0, -1.0, 1.0, 2.0, 1.0, 1.0, 1.0]),
    ]).astype(np.float32)
    n = gate.size - gate.size % G
    return bf16(gate[:n]).reshape(-1, G), bf16(up[:n]).reshape(-1, G)


def test_swiglu_matches_high_precision():
    """Every element equals bf16 (nearest even) of the exact silu(g)*u from
    60-digit decimal arithmetic, except where that value is within 2^-40 of a
    rounding midpoint; those must be flagged as near ties."""
    gb, ub = swiglu_cases()
    h, near = oracle.swiglu_bf16(gb, ub)
    gf, uf = f32(gb).ravel(), f32(ub).ravel()
    hf = f32(h).ravel()
    checked = 0
    for i in range(gf.size):
        want, dist = exact_swiglu_bf16(float(gf[i]), float(uf[i]))
        if dist <= Fraction(1, 2 ** 40):
            continue
        assert not near.ravel()[i]
        assert Fraction(float(hf[i])) == want, (i, gf[i], uf[i], hf[i], float(want))
        checked += 1
    assert checked > 0.99 * gf.size


def test_swiglu_library_silu():
    """Against torch's float64 silu times u, rounded to fp32 then bf16 by
    library casts; the double rounding only differs from one rounding when the
    fp32 value is exactly a bf16 midpoint, and such elements are skipped."""
    M, F = 64, 1024
    gb = synthetic.activations(M, F, seed=9, n_out=3)
    ub = synthetic.activations(M, F, seed=10, n_out=0)
    h, near = oracle.swiglu_bf16(gb, ub)
    gt = torch.from_numpy(f32(gb).astype(np.float64))
    v = (torch.nn.functional.silu(gt) * torch.from_numpy(f32(ub).astype(np.float64))).numpy()
    v32 = v.astype(np.float32)
    ok = (v32.view(np.uint32) & 0xFFFF) != 0x8000
    assert np.array_equal(h[ok & ~near], torch_bf16_bits(v32)[ok & ~near])
    assert near.sum() == 0


def test_swiglu_special_values():
    """silu(0) = 0 with the sign of g*u; large positive g passes g*u through;
    large negative g underflows to a zero signed opposite to u."""
    gb = bf16(np.array([[0.0, -0.0, 0.0, 128.0, 256.0, -128.0, -1000.0, -1000.0] * 16]))
    ub = bf16(np.array([[3.0, 3.0, -3.0, 1.5, -0.375, 2.0, 5.0, -5.0] * 16]))
    h, _ = oracle.swiglu_bf16(gb, ub)
    row = h[0, :8]
    assert list(row) == [0x0000, 0x8000, 0x8000, bf16(192.0)[()], bf16(-96.0)[()], 0x8000, 0x8000, 0x0000]


def test_swiglu_quant_is_quant_of_output():
    gb = synthetic.activations(16, 2048, seed=12, n_out=2)
    ub = synthetic.activations(16, 2048, seed=13, n_out=0)
    q, s, near = oracle.swiglu_quant(gb, ub)
    h, near2 = oracle.swiglu_bf16(gb, ub)
    q2, s2 = oracle.quant_act(h)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(near, near2)


# --------------------------------------------------------- SwiGLU backward

def exact_swiglu_bwd(gv: float, uv: float, dv: float):
    """(d_gate, d_up) of h = silu(g) u from 60-digit decimal arithmetic, each
    as (bf16 value, relative distance to the nearest bf16 midpoint)."""
    getcontext().prec = 60
    g, u, d = Decimal(gv), Decimal(uv), Decimal(dv)
    s = 1 / (1 + (-g).exp())
    d_up = Fraction(d * g * s)
    d_gate = Fraction(d * u * s * (1 + g * (1 - s)))
    return [(round_fraction(q, 8, -126), midpoint_distance(q, 8, -126)) for q in (d_gate, d_up)]


def test_swiglu_bwd_matches_high_precision():
    """Both gradients equal bf16 of the exact derivative from 60-digit decimal
    arithmetic wherever that value is not within 2^-40 of a midpoint (pins
    sigmoid, its derivative 1 + g (1 - s), which factor each output takes,
    and the [d_gate | d_up] layout)."""
    gb, ub = swiglu_cases()
    rng = np.random.default_rng(21)
    db = bf16(rng.normal(0, 1e-3, gb.shape).astype(np.float32) * np.where(rng.random(gb.shape) < 0.1, 1e3, 1.0))
    out, near = oracle.swiglu_bwd_bf16(gb, ub, db)
    R, F = gb.shape
    gf, uf, dfl = f32(gb), f32(ub), f32(db)
    of = f32(out)
    checked = 0
    for r in range(R):
        for c in range(F):
            for j, (want, dist) in enumerate(exact_swiglu_bwd(float(gf[r, c]), float(uf[r, c]), float(dfl[r, c]))):
                col = c + j * F
                if dist <= Fraction(1, 2 ** 40):
                    continue
                assert not near[r, col]
                assert Fraction(float(of[r, col])) == want, (r, c, j, gf[r, c], uf[r, c], dfl[r, c], of[r, col])
                checked += 1
    assert checked > 0.99 * 2 * gf.size


def test_swiglu_bwd_library_autograd():
    """Against torch autograd of silu(g) * u in float64, rounded to fp32 then
    bf16 by library casts (elements whose fp32 value is exactly a bf16 midpoint
    are skipped: there the double rounding may differ)."""
    M, F = 32, 1024
    gb = synthetic.activations(M, F, seed=14, n_out=2)
    ub = synthetic.activations(M, F, seed=15, n_out=0)
    db = synthetic.grad_out(M, F, seed=16)
    out, near = oracle.swiglu_bwd_bf16(gb, ub, db)
    g = torch.from_numpy(f32(gb).astype(np.float64)).requires_grad_(True)
    u = torch.from_numpy(f32(ub).astype(np.float64)).requires_grad_(True)
    h = torch.nn.functional.silu(g) * u
    h.backward(torch.from_numpy(f32(db).astype(np.float64)))
    want = np.concatenate([g.grad.numpy(), u.grad.numpy()], axis=1).astype(np.float32)
    ok = ((want.view(np.uint32) & 0xFFFF) != 0x8000) & ~near
    assert np.array_equal(out[ok], torch_bf16_bits(want)[ok])
    assert ok.mean() > 0.999


def test_swiglu_bwd_special_values():
    """g = 0: d_up = 0 and d_gate = dh u / 2 exactly; large positive g:
    d_up = dh g and d_gate = dh u; large negative g: both vanish."""
    F = 128
    gb = bf16(np.array([[0.0] * 32 + [128.0] * 32 + [-1000.0] * 32 + [0.0] * 32]))
    ub = bf16(np.full((1, F), 3.0))
    db = bf16(np.full((1, F), -0.5))
    out, _ = oracle.swiglu_bwd_bf16(gb, ub, db)
    dg, du = f32(out[0, :F]), f32(out[0, F:])
    assert np.all(dg[:32] == -0.75) and np.all(du[:32] == 0.0)
    assert np.all(dg[32:64] == -1.5) and np.all(du[32:64] == -64.0)
    assert np.all(dg[64:96] == 0.0) and np.all(du[64:96] == 0.0)


# -------------------------------------------------------- RMSNorm backward

def test_rmsnorm_bwd_matches_exact_rationals():
    """dx and dgamma against exact rational evaluation of the textbook
    gradients with the forward's rstd: dx bit-exact wherever the fp64
    evaluation error cannot reach a bf16 midpoint, dgamma equal to the fp32
    rounding of the exact sum (pins the r^3 term, its sign, the 1/K, gamma's
    place and the accumulation over tokens)."""
    M, K = 6, 256
    x = synthetic.activations(M, K, seed=31, n_out=2)
    gamma = synthetic.norm_weights(K, seed=31)
    dy = synthetic.grad_out(M, K, seed=31, sigma=1.0)
    _, rstd = oracle.rmsnorm_bf16(x, gamma, 1e-6)
    dx, dg = oracle.rmsnorm_bwd(x, gamma, rstd, dy)
    xf, gf, df = f32(x), f32(gamma), f32(dy)
    checked = 0
    for m in range(M):
        r = Fraction(float(rstd[m]))
        gi = [Fraction(float(gf[k])) * Fraction(float(df[m, k])) for k in range(K)]
        xs = [Fraction(float(xf[m, k])) for k in range(K)]
        c = sum(g * xv for g, xv in zip(gi, xs))
        kk = r * r * r * c / K
        for k in range(K):
            a, b = r * gi[k], xs[k] * kk
            exact = a - b
            want = round_fraction(exact, 8, -126)
            if exact != 0 and abs(exact - (want if want != 0 else exact)) >= 0:
                margin = midpoint_distance(exact, 8, -126) * abs(exact) if exact != 0 else Fraction(1)
                if margin <= (abs(a) + abs(b)) * Fraction(1, 2 ** 48):
                    continue
            assert Fraction(float(f32(dx[m, k]))) == want, (m, k)
            checked += 1
    assert checked > 0.99 * M * K
    for k in range(0, K, 7):
        total = sum(Fraction(float(df[t, k])) * Fraction(float(xf[t, k])) * Fraction(float(rstd[t]))
                    for t in range(M))
        assert np.float32(dg[k]) == np.float32(float(total)), k


def test_rmsnorm_bwd_library_autograd():
    """Against torch autograd of x * rsqrt(mean(x^2) + eps) * gamma in float64
    (its own r, not the saved fp32 rstd): dx within one bf16 rounding plus
    2^-20 of the two terms' magnitude, dgamma within 2^-20 of the sum of the
    terms' magnitudes (the saved rstd is the fp32 rounding of torch's r); over
    more than one block of 128 tokens."""
    M, K, eps = 300, 512, 1e-6
    x = synthetic.activations(M, K, seed=32, n_out=2)
    gamma = synthetic.norm_weights(K, seed=32)
    dy = synthetic.grad_out(M, K, seed=32, sigma=1.0)
    _, rstd = oracle.rmsnorm_bf16(x, gamma, eps)
    dx, dg = oracle.rmsnorm_bwd(x, gamma, rstd, dy)
    xt = torch.from_numpy(f32(x).astype(np.float64)).requires_grad_(True)
    gt = torch.from_numpy(f32(gamma).astype(np.float64)).requires_grad_(True)
    y = xt * torch.rsqrt((xt * xt).mean(dim=1, keepdim=True) + eps) * gt
    y.backward(torch.from_numpy(f32(dy).astype(np.float64)))
    want = xt.grad.numpy()
    r = rstd.astype(np.float64)[:, None]
    g = f32(gamma).astype(np.float64)[None, :] * f32(dy).astype(np.float64)
    scale = np.abs(r * g) + np.abs(f32(x) * r ** 3 * (g * f32(x)).sum(axis=1, keepdims=True) / K)
    err = np.abs(f32(dx).astype(np.float64) - want)
    assert np.all(err <= 2.0 ** -8 * np.abs(want) + 2.0 ** -20 * scale)
    mag = (np.abs(f32(dy).astype(np.float64) * f32(x)) * rstd.astype(np.float64)[:, None]).sum(axis=0)
    assert np.all(np.abs(dg.astype(np.float64) - gt.grad.numpy()) <= 2.0 ** -20 * mag)


def test_rmsnorm_bwd_invariants():
    """y is invariant to scaling x (eps = 0), so dx is orthogonal to x up to
    rounding; dy = 0 gives zero gradients."""
    M, K = 8, 1024
    x = synthetic.activations(M, K, seed=33, n_out=2)
    gamma = synthetic.norm_weights(K, seed=33)
    dy = synthetic.grad_out(M, K, seed=33, sigma=1.0)
    _, rstd = oracle.rmsnorm_bf16(x, gamma, 0.0)
    dx, _ = oracle.rmsnorm_bwd(x, gamma, rstd, dy)
    xd = f32(x).astype(np.float64)
    dxd = f32(dx).astype(np.float64)
    dot = np.abs((xd * dxd).sum(axis=1))
    assert np.all(dot <= 2.0 ** -6 * (np.abs(xd * dxd)).sum(axis=1))
    dx0, dg0 = oracle.rmsnorm_bwd(x, gamma, rstd, np.zeros_like(dy))
    assert np.all((dx0 & 0x7FFF) == 0) and np.all(dg0 == 0)
