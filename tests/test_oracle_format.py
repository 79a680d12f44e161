"""Pins of the oracle's E4M3 decoder, encoder and bf16 rounding.

Each check compares the oracle with something other than itself: an
independent library decoder (torch.float8_e4m3fn), hand-derived values from
the format definition (tests/golden/e4m3_encode_cases.txt), structural facts of
the format, and an exhaustive brute-force nearest-value search.
"""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_encode_cases.txt")


def torch_decode_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_library_decoder():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = torch_decode_table()
    nan_ours = np.isnan(ours)
    assert list(np.nonzero(nan_ours)[0]) == [0x7F, 0xFF]
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])


def test_decode_structure():
    v = oracle.e4m3_decode(np.arange(256))
    finite = v[~np.isnan(v)]
    assert finite.size == 254
    pos = v[:0x7F]
    # strictly increasing magnitudes over codes 0x00..0x7E, max 448
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    # sign symmetry: code | 0x80 negates (and -0 for 0x80)
    assert np.array_equal(v[0x80:0xFF], -pos)
    assert math.copysign(1.0, v[0x80]) == -1.0
    # spacing: 2^-9 across the subnormals and the first normal binade, then it
    # doubles every 8 codes (3 mantissa bits per binade)
    d = np.diff(pos)
    assert np.all(d[:16] == 2.0 ** -9)
    for ef in range(2, 16):
        assert np.all(d[8 * ef: 8 * ef + 8] == 2.0 ** (ef - 10)), ef
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9


def _golden_cases():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        val, code = line.split()[:2]
        out.append((float(val), int(code, 16)))
    return out


@pytest.mark.parametrize("val,code", _golden_cases())
def test_encode_golden(val, code):
    assert oracle.e4m3_encode_scalar(np.float32(val)) == code


def test_encode_matches_library_cast_in_range():
    """torch's float -> float8_e4m3fn cast rounds to nearest even; on |v| <= 448
    (where its overflow behaviour does not enter) it must agree bit for bit."""
    g = np.random.default_rng(1234)
    parts = [
        g.standard_normal(1 << 18).astype(np.float32) * np.float32(100),
        (g.random(1 << 18).astype(np.float32) * np.float32(448)),
        (g.random(1 << 16).astype(np.float32) * np.float32(2 ** -5)),
    ]
    # all E4M3 midpoints and their fp32 neighbours
    mags = torch_decode_table()[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    parts += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))]
    v = np.concatenate(parts).astype(np.float32)
    v = np.concatenate([v, -v])
    v = v[np.abs(v) <= 448]
    L = oracle.lib()
    fn = ctypes.cast(L.oracle_e4m3_encode, ctypes.c_void_p).value
    enc_t = ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_float)(fn)
    ours = np.empty(v.size, np.uint8)
    helper = _encode_many_helper()
    helper(v, ours, enc_t)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


_HELPER = {}


def _encode_many_helper():
    if "f" not in _HELPER:
        import subprocess
        import tempfile
        d = tempfile.mkdtemp()
        so = os.path.join(d, "libbrute.so")
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-o", so,
                               os.path.join(os.path.dirname(__file__), "csrc", "brute_e4m3.c"),
                               "-lm"])
        lib = ctypes.CDLL(so)
        lib.encode_many.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]

        def run(v, out, fn):
            lib.encode_many(v.ctypes.data, v.size, ctypes.cast(fn, ctypes.c_void_p), out.ctypes.data)
        _HELPER["f"] = run
    return _HELPER["f"]


def test_encode_exhaustive_against_brute_force(brute_lib):
    """Every finite fp32 bit pattern (2^32 minus NaN/Inf): the oracle's
    encoder equals a nearest-value search over the library-decoded table with
    ties to the even code."""
    tab = np.ascontiguousarray(torch_decode_table()[:0x7F], dtype=np.float64)
    brute_lib.set_table(tab.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    L = oracle.lib()
    fn = ctypes.cast(L.oracle_e4m3_encode, ctypes.c_void_p)
    brute_lib.count_mismatches.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_uint32)]
    brute_lib.count_mismatches.restype = ctypes.c_int64
    first = ctypes.c_uint32(0)
    bad = brute_lib.count_mismatches(0, 1 << 32, fn, ctypes.byref(first))
    assert bad == 0, "first mismatching fp32 bits: 0x%08x" % first.value


def test_encode_sign_symmetry_and_no_nan():
    g = np.random.default_rng(7)
    v = np.concatenate([g.standard_normal(4096).astype(np.float32) * np.float32(10.0 ** k)
                        for k in range(-12, 40, 4)])
    for x in v[:: 7]:
        c = oracle.e4m3_encode_scalar(x)
        assert c not in (0x7F, 0xFF)
        assert oracle.e4m3_encode_scalar(-x) == c ^ 0x80


def test_f64_to_bf16_matches_library():
    """fp64 -> bf16 RNE against torch's float -> bfloat16 cast on values that
    are exact in fp32 (so torch's conversion is a single rounding too)."""
    g = np.random.default_rng(3)
    v = g.standard_normal(20000).astype(np.float32) * np.float32(1000)
    u = v.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)   # exact midpoints
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, 1.0, 3e-39, -5e-40])])
    ours = oracle.f64_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
