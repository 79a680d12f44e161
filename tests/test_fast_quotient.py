"""The GPU quantizers' quotient route against IEEE division, on the CPU.

The quantizers compute fl32(x / s) as q0 = fl32(x r), res = fma(-q0, s, x),
q1 = fma(res, r, q0) with r = fl32(1 / s) once per group (Markstein's
correction), for scales s >= 2^-92, and by IEEE division below that.  The
definition of a code is E4M3(fl32(x / s)).  These tests emulate the route in C
(tests/csrc/fast_quotient.c, no FMA contraction, the C library's correctly
rounded fmaf) and check that it gives the definition's code on every pair of
bf16 values x <= amax (both signs) and on random fp32 pairs of the kind the
FP8-source requantizer produces (arbitrary fp32 values and maxima): equal
quotients wherever the quotient is at least 2^-11 in magnitude, and a value
that encodes to a zero of the right sign below that.  A route without the
correction step fails the same check."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fq(tmp_path_factory):
    src = os.path.join(ROOT, "tests", "csrc", "fast_quotient.c")
    out = str(tmp_path_factory.mktemp("fq") / "libfq.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                           "-shared", "-o", out, src, "-lm"])
    L = ctypes.CDLL(out)
    i64p, u32p = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint32)
    L.fq_check_bf16.argtypes = [i64p, i64p, u32p, u32p]
    L.fq_check_bf16.restype = ctypes.c_int64
    L.fq_check_random.argtypes = [ctypes.c_uint64, ctypes.c_int64, u32p, u32p]
    L.fq_check_random.restype = ctypes.c_int64
    L.fq_route.argtypes = [ctypes.c_float, ctypes.c_float]
    L.fq_route.restype = ctypes.c_float
    L.fq_product_only.argtypes = [ctypes.c_float, ctypes.c_float]
    L.fq_product_only.restype = ctypes.c_float
    L.fq_is_fast.argtypes = [ctypes.c_float]
    L.fq_is_fast.restype = ctypes.c_int
    return L


def test_route_equals_division_on_every_bf16_pair(fq):
    pairs, fast, bx, ba = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_uint32(), ctypes.c_uint32()
    bad = fq.fq_check_bf16(ctypes.byref(pairs), ctypes.byref(fast), ctypes.byref(bx), ctypes.byref(ba))
    # every (x, amax) with 0 <= x <= amax over the 32639 positive finite bf16 values, two signs
    assert pairs.value == sum(a + 1 for a in range(1, 0x7F80)) * 2
    assert fast.value > 0.95 * pairs.value          # amax below 448 * 2^-92 takes IEEE division
    assert bad == 0, "first mismatch: x bf16 0x%04x, amax bf16 0x%04x" % (bx.value, ba.value)


def test_route_equals_division_on_random_fp32_pairs(fq):
    bx, ba = ctypes.c_uint32(), ctypes.c_uint32()
    bad = fq.fq_check_random(20251203, 60_000_000, ctypes.byref(bx), ctypes.byref(ba))
    assert bad == 0, "first mismatch: x 0x%08x, amax 0x%08x" % (bx.value, ba.value)


def test_switch_to_division_at_2_pow_minus_92(fq):
    """The fast route covers scales from 2^-92 up: amax = 448 * 2^-92 takes it,
    the next smaller fp32 does not."""
    a = np.float32(448.0) * np.float32(2.0 ** -92)
    assert fq.fq_is_fast(a) == 1
    assert fq.fq_is_fast(np.nextafter(a, np.float32(0))) == 0


def test_correction_step_matters(fq):
    """Without the correction (q0 = fl32(x r) alone) the quotient differs from
    IEEE division on some inputs where the code would change: the check above
    is sensitive to the step it proves."""
    r = np.random.default_rng(7)
    amax = (r.random(20000).astype(np.float32) * 1000 + 1).astype(np.float32)
    x = (amax * r.random(20000).astype(np.float32)).astype(np.float32)
    diff = 0
    for xi, ai in zip(x, amax):
        q = np.float32(xi) / (np.float32(ai) / np.float32(448))
        if abs(q) >= 2.0 ** -11:
            assert np.float32(fq.fq_route(float(xi), float(ai))) == q
            diff += np.float32(fq.fq_product_only(float(xi), float(ai))) != q
    assert diff > 100
