"""Why the GEMMs multiply FP8 codes on the fp16 matrix core: the forward
product computed by one plain kernel on each FP8 MFMA instruction of gfx950
(fp8lin_gemm_fwd_mfma_probe forms 0-3) and on the fp16 instruction the
library uses (form 4, the control), compared with the fp64 oracle.

Jet-RL technical summary, "Quantization scheme": the forward, DGrad and WGrad
GEMMs run on FP8 codes with one scale per 128-wide group; the accuracy bound
of the layer is max |C - C_ref| / (|C_ref| + 0.01 rms(C_ref)) <= 1e-2 on the
BF16 outputs.  The tests pin (a) the probe kernel itself (every form is exact
where every product fits the instructions' summation window), (b) the FP8
instructions' truncated summation on a two-element case, and (c) the accuracy
metric of every form on sampled rows of the workloads' data.  The metric of
each form and workload is printed and, when FP8LIN_PROBE_OUT names a file,
written there as JSON."""
import json
import os

import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, f32_to_dev, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
G = 128
FORMS = sorted(fl.MFMA_PROBE_FORMS)
FP8_FORMS = [0, 1, 2, 3]
CONTROL = 4


def probe(xq, sx, wq, sw, form):
    y = fl.fp8lin_gemm_fwd_mfma_probe(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw), form)
    return host(y).astype(np.float64)


def to_bf16_f64(y_f32):
    """fp32 -> bf16 (round to nearest even) -> float64, as the GEMMs store."""
    u = np.ascontiguousarray(y_f32, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


E4M3_448, E4M3_ONE = 0x7E, 0x38
E4M3_15_OVER_256 = 0x17          # (8 + 7) * 2^(2 - 10) = 0.05859375


def test_every_form_exact_when_products_fit():
    """Codes with exponent field 7 or 8 (values 1 .. 3.75): every product is a
    multiple of 2^-6 below 15, every group sum and the fp32 total are exact, so
    every form must return the oracle's value exactly.  This checks the probe
    kernel's operand and output layouts, rows past M included."""
    M, N, K = 45, 256, 1024
    r = synthetic.rng(5, 90)
    def codes(shape):
        e = r.integers(7, 9, size=shape)
        f = r.integers(0, 8, size=shape)
        s = r.integers(0, 2, size=shape)
        return ((s << 7) | (e << 3) | f).astype(np.uint8)
    xq, wq = codes((M, K)), codes((N, K))
    sx = np.ones((M, K // G), np.float32)
    sw = np.ones((N // G, K // G), np.float32)
    ref = oracle.gemm_fwd(xq, sx, wq, sw)
    for form in FORMS:
        say("mfma probe exact", form)
        y = probe(xq, sx, wq, sw, form)
        assert np.array_equal(y, ref), (form, np.argwhere(y != ref)[:3])


def test_fp8_forms_truncate_two_element_sum():
    """448 + 0.05859375 in adjacent k slots of one group: the exact sum is
    448.05859375 (exact in fp32).  The FP8 instructions drop the bits of the
    smaller product below 2^-5 (13 bits under the larger product's leading
    bit) and return 448.03125; the fp16 instruction returns the exact sum."""
    M, N, K = 1, 128, 128
    xq = np.zeros((M, K), np.uint8)
    wq = np.zeros((N, K), np.uint8)
    xq[0, 0], xq[0, 1] = E4M3_448, E4M3_15_OVER_256
    wq[0, 0], wq[0, 1] = E4M3_ONE, E4M3_ONE
    sx = np.ones((M, 1), np.float32)
    sw = np.ones((1, 1), np.float32)
    exact = 448.05859375
    assert oracle.gemm_fwd(xq, sx, wq, sw)[0, 0] == exact
    got = {}
    for form in FORMS:
        say("mfma probe two-element", form)
        got[form] = probe(xq, sx, wq, sw, form)[0, 0]
    print("two-element sum 448 + 0.05859375 per form:", got)
    assert got[CONTROL] == exact
    for form in FP8_FORMS:
        assert got[form] == 448.03125, (form, got[form])


def _sample_rows(M, n, seed):
    r = synthetic.rng(seed, 91)
    rows = np.sort(r.choice(M, size=min(n, M), replace=False))
    rows[-1] = M - 1
    return np.unique(rows)


# (name, M, N, K, outlier columns, sampled rows); the workloads' shapes and data
CASES = [
    ("tiny 128x1024x1024", 128, 1024, 1024, 4, 128),
    ("decode 8B up-proj 64x14336x4096", 64, 14336, 4096, synthetic.n_outliers(4096), 64),
    ("prefill 7B 8192x18944x3584", 8192, 18944, 3584, synthetic.n_outliers(3584), 96),
    ("large 32B 16384x27648x5120", 16384, 27648, 5120, synthetic.n_outliers(5120), 96),
    ("large 32B, no outlier channels", 16384, 27648, 5120, 0, 96),
]


@pytest.fixture(scope="module")
def metrics():
    out = {}
    yield out
    path = os.environ.get("FP8LIN_PROBE_OUT")
    if path:
        with open(path, "w") as f:
            json.dump(out, f, indent=1)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_workload_metric_per_form(case, metrics):
    name, M, N, K, n_out, nrows = case
    rows = _sample_rows(M, nrows, seed=M + N)
    x = synthetic.activations(M, K, seed=0, n_out=n_out)[rows] if n_out else \
        synthetic.gaussian_bf16((M, K), 1.0, 0, synthetic.TID_X)[rows]
    w = synthetic.weights(N, K, seed=0)
    xq, sx = oracle.quant_act(x)
    wq, sw = oracle.quant_weight(w)
    del w
    ref = oracle.gemm_fwd(xq, sx, wq, sw)
    rms = float(np.sqrt(np.mean(ref * ref)))
    res = {}
    outs = {}
    for form in FORMS:
        say("mfma probe metric", name, form)
        y = probe(xq, sx, wq, sw, form)
        outs[form] = y
        res[fl.MFMA_PROBE_FORMS[form]] = oracle.gemm_metric(to_bf16_f64(y), ref, rms)
    say("library fp8_gemm_fwd", name)
    yl = fl.fp8_gemm_fwd(u8_to_dev(xq), f32_to_dev(sx), u8_to_dev(wq), f32_to_dev(sw))
    yl = host(yl).astype(np.uint32) << np.uint32(16)
    res["library fp8_gemm_fwd"] = oracle.gemm_metric(yl.view(np.float32).astype(np.float64), ref, rms)
    metrics[name] = {"rows": int(len(rows)), "metric": res}
    print(name, json.dumps(res))
    assert res[fl.MFMA_PROBE_FORMS[CONTROL]] <= 1e-2
    assert res["library fp8_gemm_fwd"] <= 1e-2
    # the FP8 instructions' sums agree closely but not always bit for bit (on
    # one machine they were identical on these data, on another a few
    # elements in a million differed by an fp32 ulp); each is judged alone
    for form in FP8_FORMS:
        fp8 = res[fl.MFMA_PROBE_FORMS[form]]
        if n_out:
            # with the outlier channels every FP8 form misses the accuracy bound
            assert fp8 > 1e-2, (name, form, fp8)
        else:
            # without them it meets it: the outlier channels are what breaks FP8
            assert fp8 <= 1e-2, (name, form, fp8)
