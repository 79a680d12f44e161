"""The allocation-free split-K decode GEMM (fp8_gemm_fwd_packed_splitk_noalloc)
against the entry point that takes a caller workspace, through the C ABI:
bit-identical outputs on two calls in a row, the second on a smaller input
(so the shared static scratch holds the first call's partial sums when the
second starts), both within the accuracy metric of the fp64 oracle."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_act_amd as fl
import oracle
import synthetic
from gpu_util import DEV, bf16_bits_to_f64, f32_to_dev, host, say, u8_to_dev

pytestmark = pytest.mark.gpu
G = 128


def _case(M, N, K, seed):
    xq = synthetic.random_codes((M, K), seed, 71)
    sx = synthetic.random_scales((M, K // G), seed, 171)
    wq = synthetic.random_codes((N, K), seed, 72)
    sw = synthetic.random_scales((N // G, K // G), seed, 172)
    return xq, sx, wq, sw


def test_noalloc_matches_workspace_entry_two_calls():
    # first: the 8B MLP down projection at 64 tokens (4 splits, the whole
    # 4 MiB scratch); second: a smaller shape with more splits (8)
    shapes = [(64, 4096, 14336), (17, 2048, 4096)]
    for i, (M, N, K) in enumerate(shapes):
        need = fl.fp8_gemm_fwd_packed_splitk_workspace(M, N, K)
        assert 0 < need <= fl.SPLITK_SCRATCH_BYTES, (M, N, K, need)
        xq, sx, wq, sw = _case(M, N, K, seed=1000 + i)
        xd, sxd, swd = u8_to_dev(xq), f32_to_dev(sx), f32_to_dev(sw)
        wp = fl.fp8_weight_pack(u8_to_dev(wq))
        y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        y_ws = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        say("splitk noalloc call", i, M, N, K)
        fl.fp8_gemm_fwd_packed_splitk_noalloc(xd, sxd, wp, swd, out=y_na)
        fl.fp8_gemm_fwd_packed_splitk(xd, sxd, wp, swd, workspace=ws, out=y_ws)
        a, b = host(y_na), host(y_ws)
        assert np.array_equal(a, b), "call %d (%d x %d x %d): noalloc differs from the workspace entry" % (
            i, M, N, K)
        err = oracle.gemm_metric(bf16_bits_to_f64(a), oracle.gemm_fwd(xq, sx, wq, sw))
        assert err <= 1e-2, "call %d: metric %.3e" % (i, err)


def test_noalloc_repeat_same_bits():
    """Repeated calls on one stream leave no state that changes the result."""
    M, N, K = 33, 1024, 2048
    xq, sx, wq, sw = _case(M, N, K, seed=7)
    xd, sxd, swd = u8_to_dev(xq), f32_to_dev(sx), f32_to_dev(sw)
    wp = fl.fp8_weight_pack(u8_to_dev(wq))
    say("splitk noalloc repeat", M, N, K)
    y1 = host(fl.fp8_gemm_fwd_packed_splitk_noalloc(xd, sxd, wp, swd))
    y2 = host(fl.fp8_gemm_fwd_packed_splitk_noalloc(xd, sxd, wp, swd))
    assert np.array_equal(y1, y2)
    assert np.array_equal(y1, host(fl.fp8_gemm_fwd_packed_splitk(xd, sxd, wp, swd)))


def test_noalloc_rejects_beyond_scratch():
    M, N, K = 64, 6144, 4096
    assert fl.fp8_gemm_fwd_packed_splitk_workspace(M, N, K) > fl.SPLITK_SCRATCH_BYTES
    xd = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    sxd = torch.zeros((M, K // G), dtype=torch.float32, device=DEV)
    wp = torch.zeros((N, K), dtype=torch.uint8, device=DEV)
    swd = torch.zeros((N // G, K // G), dtype=torch.float32, device=DEV)
    with pytest.raises(fl.Fp8LinError, match="FP8LIN_ERR_SCRATCH"):
        fl.fp8_gemm_fwd_packed_splitk_noalloc(xd, sxd, wp, swd)
