"""Error of the fp32 hardware functions the SwiGLU kernels evaluate with, on
every argument those kernels can pass to them.

The SwiGLU forward and backward kernels evaluate the logistic function in
fp32 as rcp(1 + exp2(g * c)), c = fl32(-log2 e), and re-evaluate in fp64 every
result whose fp32 value lies within its error bound of a BF16 rounding
midpoint.  That bound assumes v_exp_f32 within 2 ulp and v_rcp_f32 within
1 ulp of the exact function; these tests measure both exhaustively:
  - v_exp_f32 on every fp32 x with |x| <= 92.5 (for |g| < 64, the only case
    the fp32 route handles, |g * c| < 92.34);
  - v_rcp_f32 on every fp32 d in [1, 2^93) (d = fl(1 + e) with
    e = exp2(g * c) < 2^92.34).
The reference is the function in fp64 (torch on the device), the error is in
ulps of the fp32 result (spacing at the reference's binade).  The test that
decides the re-evaluation is checked against its definition on every low half
of the fp32 bits, and the division-free group scale and reciprocal of the
quantizers against correct rounding on every argument in their ranges."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


def bits_range(lo, hi):
    """float32 tensors holding every bit pattern in [lo, hi), chunk by chunk."""
    for start in range(lo, hi, CHUNK):
        end = min(start + CHUNK, hi)
        yield torch.arange(start, end, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.float32)


def max_ulp_error(got, ref):
    """max |got - ref| in ulps of fp32 at ref's binade (ref > 0, normal)."""
    _, e = torch.frexp(ref)                      # ref = m 2^e, m in [0.5, 1)
    ulp = torch.ldexp(torch.ones_like(ref), (e - 24).to(torch.int32))
    return ((got.double() - ref).abs() / ulp).max().item()


def test_probe_known_values():
    x = torch.tensor([0.0, 1.0, -1.0, 3.0, -10.0], device=DEV)
    assert fl.fp8lin_math_probe(x, 0).tolist() == [1.0, 2.0, 0.5, 8.0, 2.0 ** -10]
    d = torch.tensor([1.0, 2.0, 4.0, 0.5], device=DEV)
    assert fl.fp8lin_math_probe(d, 1).tolist() == [1.0, 0.5, 0.25, 2.0]


def test_exp2_within_2_ulp_on_the_kernels_arguments():
    top = int(torch.tensor([92.5]).view(torch.int32).item())          # 0x42B90000
    worst = 0.0
    for sign in (0, 1):
        say("v_exp_f32 exhaustive, sign", sign)
        for x in bits_range(0, top + 1):
            if sign:
                x = -x
            got = fl.fp8lin_math_probe(x, 0)
            ref = torch.exp2(x.double())
            worst = max(worst, max_ulp_error(got, ref))
    say("v_exp_f32 max error %.4f ulp" % worst)
    assert worst <= 2.0


def test_rcp_within_1_ulp_on_the_kernels_arguments():
    lo = int(torch.tensor([1.0]).view(torch.int32).item())            # 0x3F800000
    hi = int(torch.tensor([2.0 ** 93]).view(torch.int32).item())      # 0x6E000000
    worst = 0.0
    say("v_rcp_f32 exhaustive on [1, 2^93)")
    for d in bits_range(lo, hi):
        got = fl.fp8lin_math_probe(d, 1)
        ref = 1.0 / d.double()
        worst = max(worst, max_ulp_error(got, ref))
    say("v_rcp_f32 max error %.4f ulp" % worst)
    assert worst <= 1.0


# the fp32 high halves the flag test is checked under: ordinary values of both
# signs, the edges of [2^-100, 2^101), zeros and subnormals, the largest
# finite values, infinities and NaNs
HIGH_HALVES = [0x3F80, 0xBF80, 0x4B00, 0x3380, 0x0D80, 0x0D7F, 0x8D80, 0x7200, 0x71FF, 0xF1FF,
               0x0000, 0x8000, 0x0040, 0x7F7F, 0x7F80, 0xFF80, 0x7FC0]
LIMS = [0.0, 1.0, 11.5, 12.0, 140.0, 32767.0, 32768.0, 65536.0, float("inf")]


def test_reevaluation_flag_matches_its_definition():
    """The SwiGLU kernels' test for an fp64 re-evaluation flags exactly the
    values with a BF16 rounding midpoint within lim ulps (|low 16 bits -
    0x8000| <= lim) or a magnitude outside [2^-100, 2^101) (NaN included), on
    every low half under each high half above and each bound."""
    low = np.arange(1 << 16, dtype=np.uint32)
    dist = np.abs(low.astype(np.int64) - 0x8000)
    for hi in HIGH_HALVES:
        bits = (np.uint32(hi) << np.uint32(16)) | low
        v = bits.view(np.float32)
        with np.errstate(invalid="ignore"):
            a = np.abs(v.astype(np.float64))
            outside = ~((a >= 2.0 ** -100) & (a < 2.0 ** 101))
        vd = torch.from_numpy(v.copy()).to(DEV)
        for lim in LIMS:
            want = (dist <= lim) | outside
            got = fl.fp8lin_flag_probe(vd, lim).cpu().numpy() != 0
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, "high %#06x lim %g: bits %#010x flagged %s, expected %s" % (
                hi, lim, bits[bad[0]], got[bad[0]], want[bad[0]])
    say("re-evaluation flag: %d high halves x %d bounds, every low half" % (len(HIGH_HALVES), len(LIMS)))


def _correctly_rounded(y, resid, scale):
    """y (float32, normal, positive) is the round-to-nearest-even of the exact
    quotient q when |resid| (the exact residual scale * (q - y), fp64) is
    below scale times half the gap to y's neighbour on q's side, or equal to
    it with y's last bit even.  The gap is ulp(y) above y, and below y too
    except at a power of two, where the floats below are twice as dense."""
    _, e = torch.frexp(y.double())
    half = scale * torch.ldexp(torch.full_like(resid, 0.5), (e - 24).to(torch.int32))
    bits = y.view(torch.int32)
    pow2 = (bits & 0x7FFFFF) == 0
    lim = torch.where((resid < 0) & pow2, half / 2, half)
    even = (bits & 1) == 0
    return (resid.abs() < lim) | ((resid.abs() == lim) & even)


def test_div448_correctly_rounded_on_its_range():
    """The quantizers' group scale without a division: fp32(a / 448) on every
    fp32 a in [2^-100, 2^128) (448 y is exact in fp64, so a - 448 y is the
    exact residual)."""
    lo = int(torch.tensor([2.0 ** -100]).view(torch.int32).item())     # 0x0D800000
    hi = 0x7F800000                                                       # +inf, excluded
    say("div448_rn exhaustive on [2^-100, 2^128)")
    for a in bits_range(lo, hi):
        y = fl.fp8lin_math_probe(a, 2)
        ok = _correctly_rounded(y, a.double() - 448.0 * y.double(), 448.0)
        assert bool(ok.all()), "a = %r: got %r" % (a[~ok][0].item(), y[~ok][0].item())


def test_rcp_rn_correctly_rounded_on_its_range():
    """The quantizers' group reciprocal without a division: fp32(1 / s) on
    every fp32 s in [2^-92, 2^120) (s y is exact in fp64, so 1 - s y is the
    exact residual, s times the quotient's)."""
    lo = int(torch.tensor([2.0 ** -92]).view(torch.int32).item())      # 0x11800000
    hi = int(torch.tensor([2.0 ** 120]).view(torch.int32).item())      # 0x7B800000
    say("rcp_rn exhaustive on [2^-92, 2^120)")
    for s in bits_range(lo, hi):
        y = fl.fp8lin_math_probe(s, 3)
        sd = s.double()
        ok = _correctly_rounded(y, 1.0 - sd * y.double(), sd)
        assert bool(ok.all()), "s = %r: got %r" % (s[~ok][0].item(), y[~ok][0].item())
