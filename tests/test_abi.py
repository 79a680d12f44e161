"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before touching a
device.  Pointers here are fake addresses: validation never dereferences them,
and no call reaches a kernel launch (a valid call without a gfx950 device
returns FP8LIN_ERR_DEVICE)."""
import ctypes
import os
import re

import pytest
import torch

import fp8_block_scaled_act_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")

OK, NULL, SHAPE, ALIGN, ALIAS, DEVICE, HIP, ARG, SCRATCH = range(9)
HAS_GPU = torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:fp8lin_status|int64_t|int|const char\*)\s+(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from fp8_block_scaled_act_amd import _build
    if not os.path.exists(fl.LIB_PATH):
        _build.build()
    return fl.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11, names
    for n in ["fp8_quant_act", "fp8_quant_weight", "fp8_quant_transpose", "fp8_gemm_fwd",
              "fp8_linear_fwd", "fp8_weight_transpose", "fp8_weight_pack", "fp8_gemm_fwd_packed", "fp8_gemm_dgrad",
              "fp8_gemm_dgrad_t", "fp8_gemm_wgrad", "fp8_rmsnorm_quant", "fp8_swiglu_quant",
              "fp8_mlp_fwd", "fp8_swiglu_bwd", "fp8_gemm_fwd_unified", "fp8_gemm_fwd_packed_splitk",
              "fp8_gemm_fwd_packed_splitk_workspace", "fp8_swiglu_bwd_quant", "fp8_rmsnorm_bwd",
              "fp8_rmsnorm_bwd_workspace", "fp8_gemm_fwd_packed_splitk_noalloc", "fp8lin_status_string",
              "fp8lin_last_hip_error"]:
        assert n in names
    for n in names:
        assert hasattr(L, n), n
    assert L.fp8lin_version() == 1


def test_status_strings(L):
    for s in range(9):
        t = L.fp8lin_status_string(s).decode()
        assert t.startswith("FP8LIN_")
    assert "unknown" in L.fp8lin_status_string(99).decode()


def test_product_path_does_not_touch_oracle():
    """The binding and the library never reference the CPU oracle."""
    pkg = os.path.join(ROOT, "fp8_block_scaled_act_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                for pat in (r"\bimport\s+oracle", r"\bfrom\s+oracle", r"liboracle", r"\boracle_\w+\s*\(",
                            r"oracle[/\\]"):
                    assert not re.search(pat, src), (f, pat)


# fake, 16-byte aligned, non-overlapping device addresses; only used where no
# GPU is visible, so that a validation regression can never launch on them
A, B, C, D, E, F = (0x10000000 * (i + 1) for i in range(6))
s0 = ctypes.c_void_p(0)
fake_ptrs = pytest.mark.skipif(HAS_GPU, reason="fake device addresses are only passed where no GPU exists")


@fake_ptrs
def test_quant_act_validation(L):
    assert L.fp8_quant_act(A, 4, 100, B, C, s0) == SHAPE            # K not multiple of 128
    assert L.fp8_quant_act(A, -1, 128, B, C, s0) == SHAPE
    assert L.fp8_quant_act(None, 4, 128, B, C, s0) == NULL
    assert L.fp8_quant_act(A, 4, 128, None, C, s0) == NULL
    assert L.fp8_quant_act(A + 8, 4, 128, B, C, s0) == ALIGN
    assert L.fp8_quant_act(A, 4, 128, A + 512, C, s0) == ALIAS      # codes overlap input
    assert L.fp8_quant_act(A, 4, 128, B, B + 256, s0) == ALIAS      # scales overlap codes
    assert L.fp8_quant_act(A, 2 ** 62, 2 ** 20, B, C, s0) == SHAPE  # byte count overflows
    # empty: OK without any device and with NULL pointers
    assert L.fp8_quant_act(None, 0, 256, None, None, s0) == OK
    assert L.fp8_quant_act(None, 5, 0, None, None, s0) == OK


@fake_ptrs
def test_quant_weight_validation(L):
    assert L.fp8_quant_weight(A, 128, 100, B, C, s0) == SHAPE
    assert L.fp8_quant_weight(A, 100, 128, B, C, s0) == SHAPE
    assert L.fp8_quant_weight(A, 128 * 70000, 128, B, C, s0) == SHAPE   # grid limit
    assert L.fp8_quant_weight(A, 128, 128, None, C, s0) == NULL
    assert L.fp8_quant_weight(A, 128, 128, B, A, s0) == ALIAS
    assert L.fp8_quant_weight(None, 0, 0, None, None, s0) == OK


@fake_ptrs
def test_quant_transpose_validation(L):
    assert L.fp8_quant_transpose(7, A, None, 128, 128, B, C, None, None, s0) == ARG
    assert L.fp8_quant_transpose(0, A, D, 128, 128, B, C, None, None, s0) == ARG      # bf16 + scales
    assert L.fp8_quant_transpose(1, A, D, 128, 128, B, C, E, F, s0) == ARG           # fp8 + dual
    assert L.fp8_quant_transpose(1, A, None, 128, 128, B, C, None, None, s0) == ARG   # fp8 w/o scales
    assert L.fp8_quant_transpose(0, A, None, 100, 128, B, C, None, None, s0) == SHAPE
    assert L.fp8_quant_transpose(1, A, D, 128, 100, B, C, None, None, s0) == SHAPE    # fp8: C % 128
    assert L.fp8_quant_transpose(0, A, None, 128, 100, B, C, E, F, s0) == SHAPE       # dual: C % 128
    assert L.fp8_quant_transpose(0, A, None, 128, 128, B, C, E, None, s0) == NULL     # half a dual
    assert L.fp8_quant_transpose(0, A, None, 128, 128, B, C, B, F, s0) == ALIAS
    assert L.fp8_quant_transpose(0, A, None, 128, 77, B + 4, C, None, None, s0) == ALIGN
    assert L.fp8_quant_transpose(0, None, None, 0, 77, None, None, None, None, s0) == OK


@fake_ptrs
def test_gemm_validation(L):
    assert L.fp8_gemm_fwd(A, B, C, D, 4, 100, 128, E, s0) == SHAPE
    assert L.fp8_gemm_fwd(A, B, C, D, 4, 128, 100, E, s0) == SHAPE
    assert L.fp8_gemm_fwd(A, B, None, D, 4, 128, 128, E, s0) == NULL
    assert L.fp8_gemm_fwd(A, B, C, D, 4, 128, 128, C, s0) == ALIAS
    assert L.fp8_gemm_fwd(A, B, C, D + 4, 4, 128, 128, E, s0) == ALIGN
    assert L.fp8_gemm_fwd(None, None, None, None, 0, 128, 128, None, s0) == OK
    assert L.fp8_gemm_dgrad(A, B, C, D, 4, 100, 128, E, s0) == SHAPE
    assert L.fp8_gemm_dgrad(A, B, C, D, 4, 128, 100, E, s0) == SHAPE
    assert L.fp8_gemm_dgrad(None, None, None, None, 0, 128, 128, None, s0) == OK
    assert L.fp8_gemm_dgrad_t(A, B, C, D, 4, 100, 128, E, s0) == SHAPE
    assert L.fp8_gemm_dgrad_t(A, B, C, D, 4, 128, 128, C, s0) == ALIAS
    assert L.fp8_gemm_dgrad_t(None, None, None, None, 0, 128, 128, None, s0) == OK
    assert L.fp8_gemm_wgrad(A, B, C, D, 5, 7, 100, E, s0) == SHAPE                 # T % 128
    assert L.fp8_gemm_wgrad(A, B, C, D, 5, 7, 128, A, s0) == ALIAS
    assert L.fp8_gemm_wgrad(None, None, None, None, 5, 0, 128, None, s0) == OK


@fake_ptrs
def test_linear_fwd_validation(L):
    # x, wq, sw, M, N, K, xq, sx, y
    assert L.fp8_linear_fwd(A, B, C, 4, 100, 128, D, E, F, s0) == SHAPE
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 100, D, E, F, s0) == SHAPE
    assert L.fp8_linear_fwd(A, B, C, -1, 128, 128, D, E, F, s0) == SHAPE
    assert L.fp8_linear_fwd(A, None, C, 4, 128, 128, D, E, F, s0) == NULL
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 128, None, E, F, s0) == NULL
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 128, D, E, F + 8, s0) == ALIGN
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 128, A + 256, E, F, s0) == ALIAS   # xq over x
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 128, D, E, B, s0) == ALIAS         # y over wq
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 128, D, D + 256, F, s0) == ALIAS   # sx over xq
    assert L.fp8_linear_fwd(None, None, None, 0, 128, 128, None, None, None, s0) == OK
    # N == 0 still quantizes x, so the weights may be NULL but x may not
    assert L.fp8_linear_fwd(None, None, None, 4, 0, 128, D, E, None, s0) == NULL
    assert L.fp8_linear_fwd(A, None, None, 4, 0, 128, D, E, None, s0) == DEVICE
    assert L.fp8_linear_fwd(A, B, C, 4, 128, 128, D, E, F, s0) == DEVICE


@fake_ptrs
def test_weight_transpose_validation(L):
    assert L.fp8_weight_transpose(A, B, 100, 128, C, D, s0) == SHAPE
    assert L.fp8_weight_transpose(A, B, 128, 100, C, D, s0) == SHAPE
    assert L.fp8_weight_transpose(A, B, 128 * 70000, 128, C, D, s0) == SHAPE   # grid limit
    assert L.fp8_weight_transpose(A, None, 128, 128, C, D, s0) == NULL
    assert L.fp8_weight_transpose(A, B, 128, 128, A, D, s0) == ALIAS
    assert L.fp8_weight_transpose(A, B, 128, 128, C + 4, D, s0) == ALIGN
    assert L.fp8_weight_transpose(None, None, 0, 128, None, None, s0) == OK
    assert L.fp8_weight_transpose(A, B, 128, 128, C, D, s0) == DEVICE


@fake_ptrs
def test_packed_decode_validation(L):
    assert L.fp8_weight_pack(A, 128, 128, B, s0) == SHAPE               # K % 256
    assert L.fp8_weight_pack(A, 64, 256, B, s0) == SHAPE                # N % 128
    assert L.fp8_weight_pack(A, 128, 256, A, s0) == ALIAS
    assert L.fp8_weight_pack(None, 0, 256, None, s0) == OK
    assert L.fp8_weight_pack(A, 128, 256, B, s0) == DEVICE
    # xq, sx, wqp, sw, M, N, K, y
    assert L.fp8_gemm_fwd_packed(A, B, C, D, 65, 128, 256, E, s0) == SHAPE    # M > 64
    assert L.fp8_gemm_fwd_packed(A, B, C, D, 4, 128, 384, E, s0) == SHAPE     # K % 256
    assert L.fp8_gemm_fwd_packed(A, B, C, D, 4, 128, 16640, E, s0) == SHAPE   # K > 16384
    assert L.fp8_gemm_fwd_packed(A, B, C, D, 4, 128, 256, C, s0) == ALIAS
    assert L.fp8_gemm_fwd_packed(None, None, None, None, 0, 128, 256, None, s0) == OK
    assert L.fp8_gemm_fwd_packed(A, B, C, D, 4, 128, 256, E, s0) == DEVICE


@fake_ptrs
def test_rmsnorm_quant_validation(L):
    # x, gamma, M, K, eps, xq, sx, rstd
    assert L.fp8_rmsnorm_quant(A, B, 4, 100, 1e-6, C, D, E, s0) == SHAPE       # K % 128
    assert L.fp8_rmsnorm_quant(A, B, 4, 16512, 1e-6, C, D, E, s0) == SHAPE     # K > 16384
    assert L.fp8_rmsnorm_quant(A, B, -1, 128, 1e-6, C, D, E, s0) == SHAPE
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, -1.0, C, D, E, s0) == ARG
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, float("nan"), C, D, E, s0) == ARG
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, float("inf"), C, D, E, s0) == ARG
    assert L.fp8_rmsnorm_quant(A, None, 4, 128, 1e-6, C, D, E, s0) == NULL     # gamma
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, 1e-6, None, D, E, s0) == NULL
    assert L.fp8_rmsnorm_quant(A, B + 2, 4, 128, 1e-6, C, D, E, s0) == ALIGN
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, 1e-6, C, D, A + 16, s0) == ALIAS   # rstd over x
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, 1e-6, B, D, E, s0) == ALIAS        # xq over gamma
    assert L.fp8_rmsnorm_quant(None, None, 0, 128, 1e-6, None, None, None, s0) == OK
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, 1e-6, C, D, None, s0) == DEVICE   # rstd optional
    assert L.fp8_rmsnorm_quant(A, B, 4, 128, 0.0, C, D, E, s0) == DEVICE


@fake_ptrs
def test_swiglu_quant_validation(L):
    # gate, up, ld, M, F, hq, sh
    assert L.fp8_swiglu_quant(A, B, 256, 4, 100, C, D, s0) == SHAPE           # F % 128
    assert L.fp8_swiglu_quant(A, B, 128, 4, 256, C, D, s0) == SHAPE           # ld < F
    assert L.fp8_swiglu_quant(A, B, 2 ** 40, 2 ** 40, 128, C, D, s0) == SHAPE   # groups >= 2^32
    assert L.fp8_swiglu_quant(A, B, 260, 4, 256, C, D, s0) == ALIGN           # rows not 16-byte aligned
    assert L.fp8_swiglu_quant(None, B, 256, 4, 256, C, D, s0) == NULL
    assert L.fp8_swiglu_quant(A, B, 256, 4, 256, A + 1024, D, s0) == ALIAS    # hq inside gate's rows
    assert L.fp8_swiglu_quant(A, A + 256, 512, 4, 256, C, D, s0) == DEVICE    # halves of one tensor
    assert L.fp8_swiglu_quant(None, None, 256, 0, 256, None, None, s0) == OK
    assert L.fp8_swiglu_quant(A, B, 256, 4, 256, C, D, s0) == DEVICE


def test_splitk_workspace_query(L):
    assert L.fp8_gemm_fwd_packed_splitk_workspace(65, 4096, 4096) == -1          # M > 64
    assert L.fp8_gemm_fwd_packed_splitk_workspace(64, 4096, 384) == -1           # K % 256
    assert L.fp8_gemm_fwd_packed_splitk_workspace(64, 14336, 4096) == 0          # enough columns: no split
    assert L.fp8_gemm_fwd_packed_splitk_workspace(64, 4096, 14336) == 4 * 64 * 4096 * 4
    assert L.fp8_gemm_fwd_packed_splitk_workspace(0, 4096, 14336) == 0


@fake_ptrs
def test_splitk_validation(L):
    need = L.fp8_gemm_fwd_packed_splitk_workspace(64, 4096, 4096)
    assert need > 0
    assert L.fp8_gemm_fwd_packed_splitk(A, B, C, D, 64, 4096, 4096, E, F, need - 1, s0) == ARG
    assert L.fp8_gemm_fwd_packed_splitk(A, B, C, D, 65, 4096, 4096, E, F, need, s0) == SHAPE
    assert L.fp8_gemm_fwd_packed_splitk(A, B, C, D, 64, 4096, 4096, E, C, need, s0) == ALIAS     # ws over wqp
    assert L.fp8_gemm_fwd_packed_splitk(A, B, C, D, 64, 4096, 4096, E, F + 4, need, s0) == ALIGN
    assert L.fp8_gemm_fwd_packed_splitk(A, B, C, D, 64, 14336, 4096, E, None, 0, s0) == DEVICE    # no split
    assert L.fp8_gemm_fwd_packed_splitk(A, B, C, D, 64, 4096, 4096, E, F, need, s0) == DEVICE


def test_splitk_noalloc_scratch_limit(L):
    """The allocation-free split-K call holds its partial sums in a static
    device array of FP8LIN_SPLITK_SCRATCH_BYTES; shapes that need more are
    rejected on the host with FP8LIN_ERR_SCRATCH (checked before the device)."""
    limit = fl.SPLITK_SCRATCH_BYTES
    assert "FP8LIN_SPLITK_SCRATCH_BYTES (4 << 20)" in open(HEADER).read()
    # the 8B down projection at 64 tokens needs exactly the whole array
    assert L.fp8_gemm_fwd_packed_splitk_workspace(64, 4096, 14336) == limit
    big = L.fp8_gemm_fwd_packed_splitk_workspace(64, 6144, 4096)
    assert big > limit
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(A, B, C, D, 64, 6144, 4096, E, s0) == SCRATCH
    assert "FP8LIN_ERR_SCRATCH" in L.fp8lin_status_string(SCRATCH).decode()
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(A, B, C, D, 65, 4096, 4096, E, s0) == SHAPE


@fake_ptrs
def test_mfma_probe_validation(L):
    f = L.fp8lin_gemm_fwd_mfma_probe
    assert f(A, B, C, D, 16, 256, 256, E, 5, s0) == ARG                # no such form
    assert f(A, B, C, D, 16, 256, 256, E, -1, s0) == ARG
    assert f(A, B, C, D, 16, 200, 256, E, 0, s0) == SHAPE              # N % 128
    assert f(A, B, C, D, 16, 256, 0, E, 0, s0) == SHAPE                # K == 0
    assert f(A, B, C, D, 0, 256, 256, E, 0, s0) == OK                  # nothing to do
    assert f(A, B, C, D, 16, 256, 256, C, 0, s0) == ALIAS
    assert f(A, B, C, D, 16, 256, 256, E, 0, s0) == DEVICE


@fake_ptrs
def test_splitk_noalloc_validation(L):
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(A, B, C, D, 64, 4096, 4096, C, s0) == ALIAS     # y over wqp
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(A, B, C, D + 4, 64, 4096, 4096, E, s0) == ALIGN
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(None, B, C, D, 64, 4096, 4096, E, s0) == NULL
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(A, B, C, D, 0, 4096, 4096, E, s0) == OK          # nothing to do
    assert L.fp8_gemm_fwd_packed_splitk_noalloc(A, B, C, D, 64, 4096, 14336, E, s0) == DEVICE


@fake_ptrs
def test_gemm_fwd_unified_validation(L):
    assert L.fp8_gemm_fwd_unified(A, B, C, D, 4, 100, 128, E, s0) == SHAPE
    assert L.fp8_gemm_fwd_unified(A, B, C, D, 4, 128, 100, E, s0) == SHAPE
    assert L.fp8_gemm_fwd_unified(A, B, None, D, 4, 128, 128, E, s0) == NULL
    assert L.fp8_gemm_fwd_unified(A, B, C, D, 4, 128, 128, C, s0) == ALIAS
    assert L.fp8_gemm_fwd_unified(A, B, C, D, 4, 128, 128, E + 2, s0) == ALIGN
    assert L.fp8_gemm_fwd_unified(None, None, None, None, 0, 128, 128, None, s0) == OK
    assert L.fp8_gemm_fwd_unified(A, B, C, D, 4, 128, 128, E, s0) == DEVICE


@fake_ptrs
def test_swiglu_bwd_validation(L):
    # gate, up, ld, dh, M, F, dgu
    assert L.fp8_swiglu_bwd(A, B, 256, C, 4, 100, D, s0) == SHAPE          # F % 128
    assert L.fp8_swiglu_bwd(A, B, 128, C, 4, 256, D, s0) == SHAPE          # ld < F
    assert L.fp8_swiglu_bwd(A, B, 260, C, 4, 256, D, s0) == ALIGN
    assert L.fp8_swiglu_bwd(A, B, 256, None, 4, 256, D, s0) == NULL
    assert L.fp8_swiglu_bwd(A, B, 256, C, 4, 256, C + 64, s0) == ALIAS     # dgu over dh
    assert L.fp8_swiglu_bwd(A, A + 256, 512, C, 4, 256, D, s0) == DEVICE   # halves of one tensor
    assert L.fp8_swiglu_bwd(None, None, 256, None, 0, 256, None, s0) == OK


@fake_ptrs
def test_swiglu_bwd_quant_validation(L):
    # gate, up, ld, dh, T, F, dguq, sdgu, dguTq, sdguT
    assert L.fp8_swiglu_bwd_quant(A, B, 256, C, 100, 256, D, E, F, A + 2 ** 26, s0) == SHAPE     # T % 128
    assert L.fp8_swiglu_bwd_quant(A, B, 256, C, 128, 200, D, E, F, A + 2 ** 26, s0) == SHAPE     # F % 128
    assert L.fp8_swiglu_bwd_quant(A, B, 260, C, 128, 256, D, E, F, A + 2 ** 26, s0) == ALIGN
    assert L.fp8_swiglu_bwd_quant(A, B, 256, None, 128, 256, D, E, F, A + 2 ** 26, s0) == NULL
    assert L.fp8_swiglu_bwd_quant(A, B, 256, C, 128, 256, D, E, D + 64, A + 2 ** 26, s0) == ALIAS
    assert L.fp8_swiglu_bwd_quant(None, None, 256, None, 0, 256, None, None, None, None, s0) == OK
    assert L.fp8_swiglu_bwd_quant(A, B, 256, C, 128, 256, D, E, F, A + 2 ** 26, s0) == DEVICE


@fake_ptrs
def test_rmsnorm_bwd_validation(L):
    # x, gamma, rstd, dy, M, K, dx, dgamma, ws, ws_bytes
    need = L.fp8_rmsnorm_bwd_workspace(300, 256)
    assert need == 3 * 256 * 8
    assert L.fp8_rmsnorm_bwd_workspace(4, 100) == -1
    P = [0x10000000 * (i + 1) for i in range(10)]
    x, g, r, dy, dx, dg, ws = P[:7]
    assert L.fp8_rmsnorm_bwd(x, g, r, dy, 300, 100, dx, dg, ws, need, s0) == SHAPE
    assert L.fp8_rmsnorm_bwd(x, g, r, dy, 300, 256, dx, dg, ws, need - 8, s0) == ARG
    assert L.fp8_rmsnorm_bwd(x, g, r, dy, 300, 256, dx, None, None, 0, s0) == DEVICE   # no dgamma: no workspace
    assert L.fp8_rmsnorm_bwd(x, g, None, dy, 300, 256, dx, dg, ws, need, s0) == NULL
    assert L.fp8_rmsnorm_bwd(x, g, r, dy, 300, 256, x + 64, dg, ws, need, s0) == ALIAS
    assert L.fp8_rmsnorm_bwd(x, g, r, dy, 300, 256, dx, dg, ws + 4, need, s0) == ALIGN
    assert L.fp8_rmsnorm_bwd(None, None, None, None, 0, 256, None, None, None, 0, s0) == OK
    assert L.fp8_rmsnorm_bwd(x, g, r, dy, 300, 256, dx, dg, ws, need, s0) == DEVICE


@fake_ptrs
def test_mlp_fwd_validation(L):
    P = [0x10000000 * (i + 1) for i in range(14)]
    x, g, wgu, sgu, wd, sd, xq, sx, r, gu, hq, sh, y = P[:13]

    def call(T, K, F, eps=1e-6, **kw):
        a = dict(x=x, g=g, wgu=wgu, sgu=sgu, wd=wd, sd=sd, xq=xq, sx=sx, r=r, gu=gu, hq=hq, sh=sh, y=y)
        a.update(kw)
        return L.fp8_mlp_fwd(a["x"], a["g"], eps, a["wgu"], a["sgu"], a["wd"], a["sd"], T, K, F, a["xq"],
                             a["sx"], a["r"], a["gu"], a["hq"], a["sh"], a["y"], s0)
    assert call(4, 100, 128) == SHAPE
    assert call(4, 128, 100) == SHAPE
    assert call(4, 16512, 128) == SHAPE
    assert call(-1, 128, 128) == SHAPE
    assert call(4, 128, 128, eps=-1.0) == ARG
    assert call(4, 128, 128, wd=None) == NULL
    assert call(4, 128, 128, gu=None) == NULL
    assert call(4, 128, 128, hq=hq + 4) == ALIGN
    assert call(4, 128, 128, y=wgu) == ALIAS
    assert call(4, 128, 128, gu=xq + 128) == ALIAS
    assert call(0, 128, 128, x=None, g=None, wgu=None, sgu=None, wd=None, sd=None, xq=None, sx=None, r=None,
                gu=None, hq=None, sh=None, y=None) == OK
    assert call(4, 128, 128, r=None) == DEVICE
    assert call(4, 128, 128) == DEVICE


@fake_ptrs
def test_diagnostics_validation(L):
    assert L.fp8lin_encode_e4m3(A, 16, B, 3, s0) == ARG
    assert L.fp8lin_decode_e4m3(A, -1, B, 0, s0) == SHAPE
    assert L.fp8lin_encode_e4m3(None, 0, None, 0, s0) == OK
    # math probe: in, n, out, fn
    assert L.fp8lin_math_probe(A, -1, B, 0, s0) == SHAPE
    assert L.fp8lin_math_probe(A, 16, B, 4, s0) == ARG
    assert L.fp8lin_math_probe(A, 16, B, -1, s0) == ARG
    assert L.fp8lin_math_probe(None, 16, B, 0, s0) == NULL
    assert L.fp8lin_math_probe(A, 16, A, 1, s0) == ALIAS
    assert L.fp8lin_math_probe(None, 0, None, 1, s0) == OK
    assert L.fp8lin_math_probe(A, 16, B, 1, s0) == DEVICE
    # re-evaluation test probe: v, n, lim, out
    assert L.fp8lin_flag_probe(A, -1, 12.0, B, s0) == SHAPE
    assert L.fp8lin_flag_probe(None, 16, 12.0, B, s0) == NULL
    assert L.fp8lin_flag_probe(A, 16, 12.0, None, s0) == NULL
    assert L.fp8lin_flag_probe(A, 16, 12.0, A, s0) == ALIAS
    assert L.fp8lin_flag_probe(None, 0, 12.0, None, s0) == OK
    assert L.fp8lin_flag_probe(A, 16, 12.0, B, s0) == DEVICE


@fake_ptrs
def test_valid_call_without_gpu_reports_device_error(L):
    assert L.fp8_quant_act(A, 4, 128, B, C, s0) == DEVICE
    assert L.fp8_gemm_fwd(A, B, C, D, 4, 128, 128, E, s0) == DEVICE


def test_binding_raises_on_error(L):
    with pytest.raises(fl.Fp8LinError, match="FP8LIN_ERR_SHAPE"):
        fl._check(SHAPE, "x")


@fake_ptrs
def test_mxfp4_quant_weight_validation(L):
    # w, N, K, codes, scales
    assert L.fp8_mxfp4_quant_weight(A, 4, 100, B, C, s0) == SHAPE          # K % 32
    assert L.fp8_mxfp4_quant_weight(A, -1, 64, B, C, s0) == SHAPE
    assert L.fp8_mxfp4_quant_weight(A, 2 ** 62, 2 ** 20, B, C, s0) == SHAPE  # byte count overflows
    assert L.fp8_mxfp4_quant_weight(A, 4, 64, None, C, s0) == NULL
    assert L.fp8_mxfp4_quant_weight(A, 4, 64, B, C + 4, s0) == ALIGN
    assert L.fp8_mxfp4_quant_weight(A, 4, 64, A + 64, C, s0) == ALIAS     # codes over w
    assert L.fp8_mxfp4_quant_weight(None, 0, 64, None, None, s0) == OK
    assert L.fp8_mxfp4_quant_weight(A, 4, 96, B, C, s0) == DEVICE          # K % 128 != 0 is fine here


@fake_ptrs
def test_gemm_fwd_w4_validation(L):
    # xq, sx, codes, scales, M, N, K, y
    assert L.fp8_gemm_fwd_w4(A, B, C, D, 4, 100, 96, E, s0) == SHAPE      # K % 128
    assert L.fp8_gemm_fwd_w4(A, B, C, D, 4, 100, 16384 + 128, E, s0) == SHAPE   # K limit
    assert L.fp8_gemm_fwd_w4(A, B, C, D, 64 * 65536, 100, 128, E, s0) == SHAPE  # grid limit
    assert L.fp8_gemm_fwd_w4(A, B, None, D, 4, 100, 128, E, s0) == NULL
    assert L.fp8_gemm_fwd_w4(A, B, C, D + 4, 4, 100, 128, E, s0) == ALIGN
    assert L.fp8_gemm_fwd_w4(A, B, C, D, 4, 100, 128, C, s0) == ALIAS
    assert L.fp8_gemm_fwd_w4(None, None, None, None, 0, 100, 128, None, s0) == OK
    assert L.fp8_gemm_fwd_w4(A, B, C, D, 4, 100, 128, E, s0) == DEVICE    # any N


def test_binding_rejects_bad_workspaces():
    """Caller workspaces are checked like any other operand before the C call:
    wrong dtype -> TypeError, host memory or a non-contiguous view ->
    ValueError (zero-sized operands, so no device memory is needed here)."""
    bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
    x = torch.empty((0, 0), dtype=bf)
    args = (x, torch.empty((0,), dtype=bf), torch.empty((0,), dtype=f32), torch.empty((0, 0), dtype=bf))
    with pytest.raises(TypeError, match="workspace must be torch.float64"):
        fl.fp8_rmsnorm_bwd(*args, workspace=torch.empty((16,), dtype=f32))
    with pytest.raises(ValueError, match="workspace must be on the GPU"):
        fl.fp8_rmsnorm_bwd(*args, workspace=torch.empty((16,), dtype=torch.float64))
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        fl.fp8_rmsnorm_bwd(*args, workspace=torch.empty((16, 2), dtype=torch.float64)[:, 0])
    g = (torch.empty((0, 0), dtype=u8), torch.empty((0, 0), dtype=f32), torch.empty((128, 0), dtype=u8),
         torch.empty((1, 0), dtype=f32))
    with pytest.raises(TypeError, match="workspace must be torch.float32"):
        fl.fp8_gemm_fwd_packed_splitk(*g, workspace=torch.empty((16,), dtype=torch.float64))
    with pytest.raises(ValueError, match="workspace must be on the GPU"):
        fl.fp8_gemm_fwd_packed_splitk(*g, workspace=torch.empty((16,), dtype=f32))
