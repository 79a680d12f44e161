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
ulps of the fp32 result (spacing at the reference's binade)."""
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
