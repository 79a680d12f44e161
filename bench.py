#!/usr/bin/env python3
"""Throughput of the FP8 block-scaled quantized linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the layer's hot path over one batch of synthetic
inputs already resident in HBM:
  large    (default) 32B-shaped forward: 1x128 quantization of X [16384,5120],
           128x128 quantization of W [27648,5120] and the block-scaled GEMM,
           all three inside the timed step; the decode step's kernels below
           are timed beside it (under "kernels_decode")
  decode   8B-shaped MLP up-proj rollout step: 1x128 quantization of
           X [64,4096] + block-scaled GEMM against W [14336,4096] quantized
           128x128 (and put in the decode layout, fp8_weight_pack) beforehand,
           as rollout does between optimizer steps; 10 weight copies are
           rotated so the weights come from HBM, not MALL
  prefill  7B-shaped forward: quantize X [8192,3584] and W [18944,3584], GEMM
  backward 8B-shaped backward: dual transpose-quant of dY [8192,14336],
           transpose-requant of the saved FP8 X [8192,4096], DGrad (as the NT
           GEMM on the transposed FP8 weight, made once with the weight
           quantization) and WGrad
  tiny     X [128,1024], W [1024,1024] (correctness-sized)
The step is captured once in a HIP graph and replayed; K steps are timed
between device synchronisations.  value = GEMM TFLOP/s of the whole step.

Also reported, per kernel: the average launch duration from HIP events around
graph replays of that kernel alone on the same stream, with its algorithmic
bytes or flops and its fraction of the roofline (GEMMs against the dense FP8
MFMA peak, the metric's unit; the fp16 fraction beside it, since the codes are
multiplied on the fp16 matrix core); `roofline` for the dominant kernel;
`cpu_baseline`: the CPU oracle timed per stage on a bounded sample of the
same workload on this host, extrapolated to the full step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA (the unit the GEMMs run on)
MALL_BYTES = 256 << 20
G = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_block_scaled_act_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ bytes

def act_quant_bytes(rows, cols):
    return rows * cols * 2 + rows * cols + rows * (cols // G) * 4


def w4_gemm_bytes(M, N, K):
    """Algorithmic bytes of the 4-bit GEMM: FP8 X and its scales, E2M1 codes
    (half a byte each) and E8M0 scales (one byte per 32), BF16 Y."""
    return M * K + M * (K // G) * 4 + N * K // 2 + N * (K // 32) + M * N * 2


def weight_quant_bytes(rows, cols):
    return rows * cols * 2 + rows * cols + (rows // G) * (cols // G) * 4


def gemm_bytes(M, N, K, b_scale_elems):
    return M * K + M * (K // G) * 4 + N * K + b_scale_elems * 4 + 2 * M * N


# --------------------------------------------------------------- workloads

class Step:
    """Kernels of one step: list of (name, launch(i), kind, algorithmic units)."""

    def __init__(self):
        self.kernels = []
        self.rotate = 1
        self.gemm_flop = 0
        self.step_bytes = 0        # producers: algorithmic bytes of the step
        self.config = {}

    def add(self, name, fn, kind, units):
        self.kernels.append((name, fn, kind, units))

    def run(self, i):
        for _, fn, _, _ in self.kernels:
            fn(i)


def build_step(name, torch, fl, synthetic):
    dev = "cuda"
    wl = synthetic.WORKLOADS[name]
    st = Step()

    def bf16(bits):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def empty(shape, dtype):
        return torch.empty(shape, dtype=dtype, device=dev)

    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    if wl.kind == "forward":
        M, N, K = wl.M, wl.N, wl.K
        x = bf16(synthetic.activations(M, K, seed=0, n_out=wl.n_out))
        w = bf16(synthetic.weights(N, K, seed=0))
        xq, sx = empty((M, K), u8), empty((M, K // G), f32)
        y = empty((M, N), bf)
        if name == "decode":
            wbytes = N * K
            st.rotate = max(8, -(-2 * MALL_BYTES // wbytes))
            wqs = []
            for r in range(st.rotate):
                wq, sw = fl.fp8_quant_weight(w)
                wqs.append((fl.fp8_weight_pack(wq), sw))   # decode layout, made with the quantization
                del wq
            torch.cuda.synchronize()
            del w
            st.add("quant_act", lambda i: fl.fp8_quant_act(x, out=(xq, sx)), "hbm", act_quant_bytes(M, K))
            st.add("gemm_fwd", lambda i: fl.fp8_gemm_fwd_packed(xq, sx, wqs[i % st.rotate][0], wqs[i % st.rotate][1],
                                                                 out=y),
                   "hbm", gemm_bytes(M, N, K, (N // G) * (K // G)))
            st.dominant = "gemm_fwd"
        elif name == "w4_decode":
            wbytes = N * K // 2 + N * K // 32
            st.rotate = max(8, -(-2 * MALL_BYTES // wbytes))
            w4s = [fl.fp8_mxfp4_quant_weight(w) for _ in range(st.rotate)]
            torch.cuda.synchronize()
            del w
            st.add("quant_act", lambda i: fl.fp8_quant_act(x, out=(xq, sx)), "hbm", act_quant_bytes(M, K))
            st.add("gemm_w4", lambda i: fl.fp8_gemm_fwd_w4(xq, sx, w4s[i % st.rotate][0], w4s[i % st.rotate][1],
                                                            out=y),
                   "hbm", w4_gemm_bytes(M, N, K))
            st.dominant = "gemm_w4"
        elif name == "decode_unified":
            st.rotate = max(8, -(-2 * MALL_BYTES // (N * K)))
            wqs = [fl.fp8_quant_weight(w) for _ in range(st.rotate)]
            torch.cuda.synchronize()
            del w
            st.add("quant_act", lambda i: fl.fp8_quant_act(x, out=(xq, sx)), "hbm", act_quant_bytes(M, K))
            st.add("gemm_fwd", lambda i: fl.fp8_gemm_fwd_unified(xq, sx, wqs[i % st.rotate][0],
                                                                  wqs[i % st.rotate][1], out=y),
                   "hbm", gemm_bytes(M, N, K, (N // G) * (K // G)))
            st.dominant = "gemm_fwd"
        else:
            wq, sw = empty((N, K), u8), empty((N // G, K // G), f32)
            st.add("quant_act", lambda i: fl.fp8_quant_act(x, out=(xq, sx)), "hbm", act_quant_bytes(M, K))
            st.add("quant_weight", lambda i: fl.fp8_quant_weight(w, out=(wq, sw)), "hbm", weight_quant_bytes(N, K))
            st.add("gemm_fwd", lambda i: fl.fp8_gemm_fwd(xq, sx, wq, sw, out=y), "mfma", 2 * M * N * K)
            st.dominant = "gemm_fwd"
        st.gemm_flop = 2 * M * N * K
        st.config = {"workload": wl.doc, "M": M, "N": N, "K": K, "outlier_columns": wl.n_out,
                     "weight_copies_rotated": st.rotate}
        if name == "decode":
            st.config["weight_layout"] = "decode layout (fp8_weight_pack), made with the weight quantization"
        if name == "w4_decode":
            st.config["weight_format"] = "MXFP4 (E2M1 codes, E8M0 scale per 32 along K), quantized once"
    elif wl.kind == "mlp":
        T, F, K = wl.M, wl.N, wl.K
        x = bf16(synthetic.activations(T, K, seed=0, n_out=wl.n_out))
        gamma = bf16(synthetic.norm_weights(K, seed=0))
        wgu_b = bf16(synthetic.weights(2 * F, K, seed=0))
        wd_b = bf16(synthetic.weights(K, F, seed=1))
        decode = T <= 64
        per_copy = 3 * F * K
        st.rotate = max(3, -(-2 * MALL_BYTES // per_copy)) if decode else 1
        ws = []
        for r in range(st.rotate):
            wgu, sgu = fl.fp8_quant_weight(wgu_b)
            wd, sd = fl.fp8_quant_weight(wd_b)
            if decode:                              # decode layout, made with the weight quantization
                wgu, wd = fl.fp8_weight_pack(wgu), fl.fp8_weight_pack(wd)
            ws.append((wgu, sgu, wd, sd))
        torch.cuda.synchronize()
        del wgu_b, wd_b
        xq, sx, rstd = empty((T, K), u8), empty((T, K // G), f32), empty((T,), f32)
        gu = empty((T, 2 * F), bf)
        hq, sh = empty((T, F), u8), empty((T, F // G), f32)
        y = empty((T, K), bf)
        kind = "hbm" if decode else "mfma"
        if decode:                                  # split over K where the weight has few columns
            wsp = torch.empty((max(max(fl.fp8_gemm_fwd_packed_splitk_workspace(T, n, k)
                                       for n, k in ((2 * F, K), (K, F))) // 4, 1),), dtype=f32, device=dev)
            gemm = lambda a, sa, b, sb, out: fl.fp8_gemm_fwd_packed_splitk(a, sa, b, sb, workspace=wsp, out=out)
        else:
            gemm = fl.fp8_gemm_fwd
        st.add("rmsnorm_quant", lambda i: fl.fp8_rmsnorm_quant(x, gamma, 1e-6, out=(xq, sx, rstd)), "hbm",
               act_quant_bytes(T, K) + 4 * T + 2 * K)
        st.add("gemm_gate_up", lambda i: gemm(xq, sx, ws[i % st.rotate][0], ws[i % st.rotate][1], out=gu), kind,
               gemm_bytes(T, 2 * F, K, (2 * F // G) * (K // G)) if decode else 2 * T * 2 * F * K)
        st.add("swiglu_quant", lambda i: fl.fp8_swiglu_quant(gu[:, :F], gu[:, F:], out=(hq, sh)), "hbm",
               2 * T * F * 2 + T * F + T * (F // G) * 4)
        st.add("gemm_down", lambda i: gemm(hq, sh, ws[i % st.rotate][2], ws[i % st.rotate][3], out=y), kind,
               gemm_bytes(T, K, F, (K // G) * (F // G)) if decode else 2 * T * K * F)
        st.dominant = "gemm_gate_up"
        st.gemm_flop = 6 * T * K * F
        st.config = {"workload": wl.doc, "T": T, "K": K, "F": F, "eps": 1e-6, "outlier_columns": wl.n_out,
                     "weight_copies_rotated": st.rotate,
                     "same_kernels_as": "fp8_mlp_fwd (one call; bit-identical outputs)"}
    elif wl.kind == "mlp_train":
        T, F, K = wl.M, wl.N, wl.K
        x = bf16(synthetic.activations(T, K, seed=0, n_out=wl.n_out))
        gamma = bf16(synthetic.norm_weights(K, seed=0))
        dy = bf16(synthetic.grad_out(T, K, seed=0))
        wgu_b = bf16(synthetic.weights(2 * F, K, seed=0))     # BF16 master weights
        wd_b = bf16(synthetic.weights(K, F, seed=1))
        wgu, sgu = empty((2 * F, K), u8), empty((2 * F // G, K // G), f32)
        wd, sd = empty((K, F), u8), empty((K // G, F // G), f32)
        wguT, sguT = empty((K, 2 * F), u8), empty((K // G, 2 * F // G), f32)
        wdT, sdT = empty((F, K), u8), empty((F // G, K // G), f32)
        torch.cuda.synchronize()
        xq, sx, rstd = empty((T, K), u8), empty((T, K // G), f32), empty((T,), f32)
        gu, hq, sh, y = empty((T, 2 * F), bf), empty((T, F), u8), empty((T, F // G), f32), empty((T, K), bf)
        dyTq, sdyT, dyq, sdy = empty((K, T), u8), empty((K, T // G), f32), empty((T, K), u8), empty((T, K // G), f32)
        hTq, shT = empty((F, T), u8), empty((F, T // G), f32)
        dwd, dh = empty((K, F), bf), empty((T, F), bf)
        dguTq, sdguT = empty((2 * F, T), u8), empty((2 * F, T // G), f32)
        dguq, sdgu = empty((T, 2 * F), u8), empty((T, 2 * F // G), f32)
        xTq, sxT = empty((K, T), u8), empty((K, T // G), f32)
        dwgu, dxn = empty((2 * F, K), bf), empty((T, K), bf)
        dual = lambda r, c: r * c * 2 + 2 * r * c + (c * (r // G) + r * (c // G)) * 4
        requant = lambda r, c: 2 * r * c + (r * (c // G) + c * (r // G)) * 4
        # per optimizer step: the weights re-quantized from the BF16 masters, with
        # the transposed copies DGrad reads
        st.add("quant_weight_gate_up", lambda i: fl.fp8_quant_weight(wgu_b, out=(wgu, sgu)), "hbm",
               weight_quant_bytes(2 * F, K))
        st.add("quant_weight_down", lambda i: fl.fp8_quant_weight(wd_b, out=(wd, sd)), "hbm",
               weight_quant_bytes(K, F))
        st.add("weight_transpose_gate_up", lambda i: fl.fp8_weight_transpose(wgu, sgu, out=(wguT, sguT)), "hbm",
               2 * 2 * F * K + 2 * (2 * F // G) * (K // G) * 4)
        st.add("weight_transpose_down", lambda i: fl.fp8_weight_transpose(wd, sd, out=(wdT, sdT)), "hbm",
               2 * K * F + 2 * (K // G) * (F // G) * 4)
        st.add("rmsnorm_quant", lambda i: fl.fp8_rmsnorm_quant(x, gamma, 1e-6, out=(xq, sx, rstd)), "hbm",
               act_quant_bytes(T, K) + 4 * T + 2 * K)
        st.add("gemm_gate_up", lambda i: fl.fp8_gemm_fwd(xq, sx, wgu, sgu, out=gu), "mfma", 4 * T * F * K)
        st.add("swiglu_quant", lambda i: fl.fp8_swiglu_quant(gu[:, :F], gu[:, F:], out=(hq, sh)), "hbm",
               2 * T * F * 2 + T * F + T * (F // G) * 4)
        st.add("gemm_down", lambda i: fl.fp8_gemm_fwd(hq, sh, wd, sd, out=y), "mfma", 2 * T * K * F)
        st.add("quant_transpose_dual_dY", lambda i: fl.fp8_quant_transpose(dy, dual=True, out=(dyTq, sdyT, dyq, sdy)),
               "hbm", dual(T, K))
        st.add("quant_transpose_fp8_H", lambda i: fl.fp8_quant_transpose(hq, sh, out=(hTq, shT, None, None)), "hbm",
               requant(T, F))
        st.add("gemm_wgrad_down", lambda i: fl.fp8_gemm_wgrad(dyTq, sdyT, hTq, shT, out=dwd), "mfma", 2 * T * K * F)
        st.add("gemm_dgrad_down", lambda i: fl.fp8_gemm_dgrad_t(dyq, sdy, wdT, sdT, out=dh), "mfma", 2 * T * K * F)
        st.add("swiglu_bwd_quant",
               lambda i: fl.fp8_swiglu_bwd_quant(gu[:, :F], gu[:, F:], dh, out=(dguTq, sdguT, dguq, sdgu)), "hbm",
               3 * T * F * 2 + 2 * (2 * T * F) + (2 * F * (T // G) + T * (2 * F // G)) * 4)
        st.add("quant_transpose_fp8_X", lambda i: fl.fp8_quant_transpose(xq, sx, out=(xTq, sxT, None, None)), "hbm",
               requant(T, K))
        st.add("gemm_wgrad_gate_up", lambda i: fl.fp8_gemm_wgrad(dguTq, sdguT, xTq, sxT, out=dwgu), "mfma",
               4 * T * F * K)
        st.add("gemm_dgrad_gate_up", lambda i: fl.fp8_gemm_dgrad_t(dguq, sdgu, wguT, sguT, out=dxn), "mfma",
               4 * T * F * K)
        dxb, dgam = empty((T, K), bf), empty((K,), f32)
        wsn = torch.empty((fl.fp8_rmsnorm_bwd_workspace(T, K) // 8,), dtype=torch.float64, device=dev)
        st.add("rmsnorm_bwd", lambda i: fl.fp8_rmsnorm_bwd(x, gamma, rstd, dxn, workspace=wsn, out=(dxb, dgam)),
               "hbm", 3 * T * K * 2 + 4 * T + 2 * K + 4 * K)
        st.dominant = None
        st.gemm_flop = 18 * T * K * F
        st.config = {"workload": wl.doc, "T": T, "K": K, "F": F, "eps": 1e-6, "outlier_columns": wl.n_out,
                     "same_kernels_as": "fp8_mlp_fwd + fp8_mlp_bwd (with the RMSNorm backward)",
                     "weights": "re-quantized from BF16 masters inside the step (fp8_quant_weight), with "
                                "the transposed FP8 copies DGrad reads (fp8_weight_transpose)"}
    elif wl.kind == "producers":
        T, F, K = wl.M, wl.N, wl.K
        x = bf16(synthetic.activations(T, K, seed=0, n_out=wl.n_out))
        gamma = bf16(synthetic.norm_weights(K, seed=0))
        gu = bf16(synthetic.activations(T, 2 * F, seed=1, n_out=synthetic.n_outliers(2 * F)))
        gate, up = gu[:, :F], gu[:, F:]
        xq, sx, rstd = empty((T, K), u8), empty((T, K // G), f32), empty((T,), f32)
        hq, sh = empty((T, F), u8), empty((T, F // G), f32)
        st.add("rmsnorm_quant", lambda i: fl.fp8_rmsnorm_quant(x, gamma, 1e-6, out=(xq, sx, rstd)), "hbm",
               act_quant_bytes(T, K) + 4 * T + 2 * K)
        st.add("swiglu_quant", lambda i: fl.fp8_swiglu_quant(gate, up, out=(hq, sh)), "hbm",
               2 * T * F * 2 + T * F + T * (F // G) * 4)
        st.dominant = "swiglu_quant"
        st.step_bytes = sum(k[3] for k in st.kernels)
        st.config = {"workload": wl.doc, "T": T, "K": K, "F": F, "eps": 1e-6,
                     "outlier_columns": wl.n_out}
    else:
        T, N, K = wl.M, wl.N, wl.K
        dy = bf16(synthetic.grad_out(T, N, seed=0))
        x = bf16(synthetic.activations(T, K, seed=0, n_out=wl.n_out))
        w = bf16(synthetic.weights(N, K, seed=0))
        wq, sw = fl.fp8_quant_weight(w)              # forward's weight quantization
        wqT, swT = fl.fp8_weight_transpose(wq, sw)    # its transposed copy, made alongside for DGrad
        xq, sx = fl.fp8_quant_act(x)                  # saved FP8 activations of the forward
        torch.cuda.synchronize()
        del w, x
        dyTq, sdyT = empty((N, T), u8), empty((N, T // G), f32)
        dyq, sdy = empty((T, N), u8), empty((T, N // G), f32)
        xTq, sxT = empty((K, T), u8), empty((K, T // G), f32)
        dx, dw = empty((T, K), bf), empty((N, K), bf)
        st.add("quant_transpose_dual_dY",
               lambda i: fl.fp8_quant_transpose(dy, dual=True, out=(dyTq, sdyT, dyq, sdy)), "hbm",
               T * N * 2 + 2 * T * N + (N * (T // G) + T * (N // G)) * 4)
        st.add("quant_transpose_fp8_X", lambda i: fl.fp8_quant_transpose(xq, sx, out=(xTq, sxT, None, None)),
               "hbm", T * K + T * (K // G) * 4 + T * K + K * (T // G) * 4)
        # DGrad dX = dY W on the transposed weight (same sums as fp8_gemm_dgrad)
        st.add("gemm_dgrad", lambda i: fl.fp8_gemm_dgrad_t(dyq, sdy, wqT, swT, out=dx), "mfma", 2 * T * N * K)
        st.add("gemm_wgrad", lambda i: fl.fp8_gemm_wgrad(dyTq, sdyT, xTq, sxT, out=dw), "mfma", 2 * T * N * K)
        st.gemm_flop = 4 * T * N * K
        st.dominant = None
        st.config = {"workload": wl.doc, "T": T, "N": N, "K": K, "outlier_columns": wl.n_out,
                     "dgrad_weight": "transposed FP8 copy (fp8_weight_transpose), made with the weight "
                                     "quantization outside the step"}
    return st


# ------------------------------------------------------------------ timing

def capture(torch, fns, count):
    """HIP graph of fns(i) for i in range(count) on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(count):
            for f in fns:
                f(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            for f in fns:
                f(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps):
    """Average ms per replay, HIP events on the replaying stream."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_kernels(torch, st, reps):
    """Per kernel of a step: graph replays of that kernel alone (R launches per
    replay over the rotated buffers), HIP events on the replaying stream."""
    R = st.rotate
    kernels = {}
    for name, fn, kind, units in st.kernels:
        gk = capture(torch, [fn], R)
        ms = time_graph(torch, gk, reps) / R
        if kind == "hbm":
            ach, unit, peak = units / (ms * 1e-3) / 1e9, "GB/s", HBM_PEAK_GBS
        else:
            ach, unit, peak = units / (ms * 1e-3) / 1e12, "TFLOP/s", FP8_PEAK_TFLOPS
        kernels[name] = {"us": round(ms * 1e3, 2), "achieved": round(ach, 1), "unit": unit,
                         "frac": round(ach / peak, 4), "algorithmic": units}
        if kind == "mfma":
            kernels[name]["frac_of_fp16_peak"] = round(ach / F16_PEAK_TFLOPS, 4)
        log("[bench]  %-26s %9.2f us  %9.1f %s" % (name, ms * 1e3, ach, unit))
        del gk
    return kernels


# ------------------------------------------------------------ cpu baseline

def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"nproc": avail, "cpu_model": model}


def timed(fn, min_seconds, max_reps=1000):
    """Repeat fn until min_seconds have passed; seconds per repetition."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            return dt / reps, reps


def cpu_baseline_forward_stages(name, synthetic, budget=12.0):
    """The oracle per stage of the forward step (activation quantization,
    weight quantization, GEMM), each on a bounded sample of the workload and
    extrapolated linearly in rows to the full step."""
    import oracle
    wl = synthetic.WORKLOADS[name]
    M, N, K = wl.M, wl.N, wl.K
    ra = min(M, 1024)
    rw = min(N, 1024)
    rg = min(M, 16)
    x = synthetic.activations(M, K, seed=0, n_out=wl.n_out)[:max(ra, rg)]
    w = synthetic.weights(N, K, seed=0)
    wq, sw = oracle.quant_weight(w)                # the GEMM's operand (outside the timing)
    wpart = w[:rw]
    xq, sx = oracle.quant_act(x[:rg])
    t_act, n_act = timed(lambda: oracle.quant_act(x[:ra]), 0.15 * budget)
    t_wq, n_wq = timed(lambda: oracle.quant_weight(wpart), 0.15 * budget)
    t_gemm, n_gemm = timed(lambda: oracle.gemm_fwd(xq, sx, wq, sw), 0.7 * budget)
    full_act = t_act * M / ra
    full_wq = t_wq * N / rw
    full_gemm = t_gemm * M / rg
    total = full_act + full_wq + full_gemm
    stages = {
        "quant_act": {"sample": "%d of %d rows" % (ra, M), "reps": n_act, "ms_sample": round(t_act * 1e3, 3),
                      "ms_full": round(full_act * 1e3, 1),
                      "GB/s": round(act_quant_bytes(ra, K) / t_act / 1e9, 3)},
        "quant_weight": {"sample": "%d of %d rows" % (rw, N), "reps": n_wq, "ms_sample": round(t_wq * 1e3, 3),
                         "ms_full": round(full_wq * 1e3, 1),
                         "GB/s": round(weight_quant_bytes(rw, K) / t_wq / 1e9, 3)},
        "gemm_fwd": {"sample": "%d of %d rows x all %d columns, fp64" % (rg, M, N), "reps": n_gemm,
                     "ms_sample": round(t_gemm * 1e3, 3), "ms_full": round(full_gemm * 1e3, 1),
                     "GFLOP/s": round(2 * rg * N * K / t_gemm / 1e9, 2)},
    }
    info = host_info()
    return {"value": 2 * M * N * K / total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "nproc": info["nproc"], "cpu_model": info["cpu_model"],
            "sample": "each stage timed on a sample of the step's inputs (see stages) and extrapolated "
                      "linearly in rows to the full step; value = the step's GEMM flop / the extrapolated "
                      "step time (%.1f s)" % total,
            "ms_per_step_extrapolated": round(total * 1e3, 1), "stages": stages,
            "seconds": round(n_act * t_act + n_wq * t_wq + n_gemm * t_gemm, 2)}


def cpu_baseline(name, synthetic, min_seconds=10.0, max_reps=200):
    """The oracle, as it stands, on a bounded sample of the workload: the
    sampled step is repeated until at least min_seconds of CPU time."""
    import numpy as np
    import oracle
    wl = synthetic.WORKLOADS[name]
    if name in ("large", "prefill", "tiny"):
        return cpu_baseline_forward_stages(name, synthetic)
    if wl.kind == "forward":
        M, N, K = wl.M, wl.N, wl.K
        rows = min(M, 64)
        x = synthetic.activations(M, K, seed=0, n_out=wl.n_out)[:rows]
        w = synthetic.weights(N, K, seed=0)
        if name == "w4_decode":
            w4, s4 = oracle.mxfp4_quant(w)

            def work():
                xq, sx = oracle.quant_act(x)
                oracle.gemm_fwd_w4(xq, sx, w4, s4)
        else:
            wq, sw = oracle.quant_weight(w)

            def work():
                xq, sx = oracle.quant_act(x)
                oracle.gemm_fwd(xq, sx, wq, sw)
        what = ("%d of %d rows of X per repetition: oracle 1x128 quantization + fp64 GEMM against "
                "the full %sW (W quantized once, outside the timing)" % (rows, M,
                                                                         "MXFP4 " if name == "w4_decode" else ""))
    elif wl.kind in ("mlp", "mlp_train"):
        T, F, K = wl.M, wl.N, wl.K
        rows = min(T, 8)
        x = synthetic.activations(T, K, seed=0, n_out=wl.n_out)[:rows]
        gamma = synthetic.norm_weights(K, seed=0)
        owgu, osgu = oracle.quant_weight(synthetic.weights(2 * F, K, seed=0))
        owd, osd = oracle.quant_weight(synthetic.weights(K, F, seed=1))

        def work():
            xq, sx, _ = oracle.rmsnorm_quant(x, gamma, 1e-6)
            gu = oracle.f64_to_bf16(oracle.gemm_fwd(xq, sx, owgu, osgu))
            hq, sh, _ = oracle.swiglu_quant(np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]))
            oracle.gemm_fwd(hq, sh, owd, osd)
        flop = 6 * rows * K * F
        reps, t0 = 0, time.perf_counter()
        while True:
            work()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or reps >= max_reps:
                break
        return {"value": flop * reps / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": "%d of %d token rows per repetition through the oracle block: RMSNorm + quantization, "
                          "fp64 gate/up GEMM, bf16 rounding, SwiGLU + quantization, fp64 down GEMM (weights "
                          "quantized once, outside the timing); %d repetitions%s" % (
                              rows, T, reps, "; forward only: its oracle GEMM rate stands for the training step's"
                              if wl.kind == "mlp_train" else ""),
                "seconds": round(dt, 2)}
    elif wl.kind == "producers":
        T, F, K = wl.M, wl.N, wl.K
        rows = 1024
        max_reps = 10 ** 6
        x = synthetic.activations(T, K, seed=0, n_out=wl.n_out)[:rows]
        gamma = synthetic.norm_weights(K, seed=0)
        gu = synthetic.activations(T, 2 * F, seed=1, n_out=synthetic.n_outliers(2 * F))[:rows]
        gate, up = np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:])
        del gu

        def work():
            oracle.rmsnorm_quant(x, gamma, 1e-6)
            oracle.swiglu_quant(gate, up)
        nbytes = act_quant_bytes(rows, K) + 4 * rows + 2 * K + 2 * rows * F * 2 + rows * F + rows * (F // G) * 4
        reps, t0 = 0, time.perf_counter()
        while True:
            work()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or reps >= max_reps:
                break
        return {"value": nbytes * reps / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": "%d of %d token rows per repetition: oracle RMSNorm + 1x128 quantization of X rows and "
                          "SwiGLU + 1x128 quantization of gate/up rows; %d repetitions" % (rows, T, reps),
                "seconds": round(dt, 2)}
    else:
        T, N, K = wl.M, wl.N, wl.K
        rows = 8
        dy = synthetic.grad_out(T, N, seed=0)[:rows]
        w = synthetic.weights(N, K, seed=0)
        wq, sw = oracle.quant_weight(w)

        def work():
            dyq, sdy = oracle.quant_act(dy)
            oracle.gemm_dgrad(dyq, sdy, wq, sw)
        what = ("DGrad for %d of %d token rows per repetition: oracle 1x128 quantization of the dY "
                "rows + fp64 GEMM against the full W" % (rows, T))
    flop = 2 * rows * N * K
    reps = 0
    t0 = time.perf_counter()
    while True:
        work()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    return {"value": flop * reps / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%s; %d repetitions" % (what, reps), "seconds": round(dt, 2)}


# --------------------------------------------------------------- profiling
#
# rocprofv3 counter passes need plain (non-graph) dispatches, and the HBM
# counters are calibrated against a copy of known size:
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d D1 -o run -- python3 bench.py --workload W --profile-eager
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d D2 -o run -- python3 bench.py --workload W --profile-eager
#   python3 bench.py --workload W --ingest-pmc D1/run_counter_collection.csv D2/run_counter_collection.csv
# The ingest step writes profiles/traffic.json (bytes per launch, scaled by
# the copy's calibration factor, with the kernel-source hash it belongs to).

KERNEL_SOURCES = {           # bench kernel name -> the sources its code comes from
    "quant_act": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "quant_weight": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "quant_transpose_dual_dY": ("quant_kernels.hip", "quant_tile.hpp", "fp8lin_device.hpp"),
    "quant_transpose_fp8_X": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "gemm_fwd": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "gemm_dgrad": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "gemm_wgrad": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "gemm_gate_up": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "gemm_wgrad_down": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "quant_weight_gate_up": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "quant_weight_down": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "weight_transpose_gate_up": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "weight_transpose_down": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "gemm_dgrad_down": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "gemm_wgrad_gate_up": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "gemm_dgrad_gate_up": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "quant_transpose_fp8_H": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "quant_transpose_dual_dGU": ("quant_kernels.hip", "fp8lin_device.hpp"),
    "swiglu_bwd": ("producer_kernels.hip", "fp8lin_device.hpp"),
    "rmsnorm_bwd": ("producer_kernels.hip", "fp8lin_device.hpp"),
    "swiglu_bwd_quant": ("producer_kernels.hip", "quant_tile.hpp", "fp8lin_device.hpp"),
    "gemm_down": ("gemm_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
    "rmsnorm_quant": ("producer_kernels.hip", "fp8lin_device.hpp"),
    "swiglu_quant": ("producer_kernels.hip", "fp8lin_device.hpp"),
    "gemm_w4": ("w4_kernels.hip", "decode_stream.hpp", "fp8lin_device.hpp"),
}

CALIB_BYTES = 4 << 30
PROFILE_REPS = 5
KERNEL_SYMBOLS = {           # bench kernel name -> substring of the HIP symbol
    "quant_act": "quant_rowgroup_kernel",
    "quant_weight": "quant_block_kernel",
    "quant_transpose_dual_dY": "quant_transpose_bf16_kernel",
    "quant_transpose_fp8_X": "quant_transpose_fp8_kernel",
    "gemm_fwd": "gemm_",
    "gemm_dgrad": "Mode)0",     # the backward step runs DGrad as the NT GEMM on W^T
    "gemm_wgrad": "Mode)2",
    "gemm_wgrad_down": None,    # kernels run at several shapes in one step: counters cannot tell them apart
    "quant_weight_gate_up": None,
    "quant_weight_down": None,
    "weight_transpose_gate_up": None,
    "weight_transpose_down": None,
    "gemm_dgrad_down": None,
    "gemm_wgrad_gate_up": None,
    "gemm_dgrad_gate_up": None,
    "quant_transpose_fp8_H": None,
    "quant_transpose_dual_dGU": None,
    "swiglu_bwd": "swiglu_bwd_kernel",
    "rmsnorm_bwd": None,        # three kernels (dx, dgamma block sums, dgamma total)
    "swiglu_bwd_quant": "swiglu_bwd_quant_kernel",
    "gemm_gate_up": None,       # same kernel as gemm_down: counters cannot tell them apart
    "gemm_down": None,
    "rmsnorm_quant": "rmsnorm_quant_kernel",
    "swiglu_quant": "swiglu_quant_kernel",
    "gemm_w4": "gemm_w4",
}


# (workload, kernel) pairs whose HIP kernel also runs at another shape in the
# same step under another name: their counters cannot be told apart
AMBIGUOUS_SYMBOLS = {("mlp_train", "quant_transpose_fp8_X")}   # also the H requant


def profile_eager(name, torch, fl, synthetic):
    st = build_step(name, torch, fl, synthetic)
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(PROFILE_REPS):
        dst.copy_(src)
    for kname, fn, _, _ in st.kernels:
        for i in range(PROFILE_REPS):
            fn(i)
    torch.cuda.synchronize()
    log("[bench] profile-eager: %d copies of %d bytes, %d launches of each kernel" %
        (PROFILE_REPS, CALIB_BYTES, PROFILE_REPS))


def ingest_pmc(name, fetch_csv, write_csv, torch, fl, synthetic):
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def avg_kib(table, pred):
        xs = [v for k, vs in table.items() if pred(k) for v in vs]
        return sum(xs) / len(xs) if xs else None

    copy_pred = lambda k: "elementwise" in k or "copy" in k.lower()

    def calib_kib(table):
        # the calibration copies are the largest copy dispatches (input uploads
        # of the step are small copies too)
        xs = sorted((v for k, vs in table.items() if copy_pred(k) for v in vs), reverse=True)[:PROFILE_REPS]
        return sum(xs) / len(xs)
    f_copy, w_copy = calib_kib(fetch), calib_kib(write)
    factor_f = CALIB_BYTES / (f_copy * 1024.0)
    factor_w = CALIB_BYTES / (w_copy * 1024.0)
    st = build_step(name, torch, fl, synthetic)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    for kname, _, kind, units in st.kernels:
        sym = KERNEL_SYMBOLS[kname]
        if sym is None or (name, kname) in AMBIGUOUS_SYMBOLS:
            continue
        pred = lambda k, sym=sym: sym in k and not copy_pred(k)
        f, w = avg_kib(fetch, pred), avg_kib(write, pred)
        if f is None or w is None:
            continue
        b = f * 1024.0 * factor_f + w * 1024.0 * factor_w
        data["%s/%s" % (name, kname)] = {
            "bytes_per_launch": round(b), "fetch_kib_raw": round(f, 1), "write_kib_raw": round(w, 1),
            "calibration": {"copy_bytes": CALIB_BYTES, "fetch_factor": round(factor_f, 4),
                            "write_factor": round(factor_w, 4)},
            "algorithmic_bytes": units if kind == "hbm" else None,
            "source_sha": source_hash(*KERNEL_SOURCES[kname]),
        }
        log("[bench] %s/%s: %.1f MB per launch (fetch %.1f MiB, write %.1f MiB raw)" %
            (name, kname, b / 1e6, f / 1024, w / 1024))
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)


# -------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large", choices=["decode", "w4_decode", "decode_unified", "prefill", "large", "backward", "tiny", "producers", "mlp",
                             "mlp_decode", "mlp_train"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="large: skip timing the decode step's kernels beside it")
    ap.add_argument("--profile-eager", action="store_true",
                    help="run each kernel of the step eagerly (for rocprofv3 counter passes) and exit")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn FETCH_SIZE / WRITE_SIZE counter CSVs into profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the layer would "
              "shard by token rows, 128-aligned, with one all-reduce of the weight gradients); "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_block_scaled_act_amd as fl
    import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.profile_eager:
        profile_eager(args.workload, torch, fl, synthetic)
        return
    if args.ingest_pmc:
        ingest_pmc(args.workload, args.ingest_pmc[0], args.ingest_pmc[1], torch, fl, synthetic)
        return
    log("[bench] workload", args.workload, "- building inputs")
    st = build_step(args.workload, torch, fl, synthetic)
    R = st.rotate
    st_config = st.config
    steps = -(-args.steps // R) * R
    warm = -(-args.warmup // R) * R

    log("[bench] capturing step graph (%d steps per replay)" % R)
    g_step = capture(torch, [lambda i: st.run(i)], R)
    for _ in range(warm // R):
        g_step.replay()
    torch.cuda.synchronize()
    log("[bench] timing %d steps" % steps)
    stream = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps // R + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for j in range(steps // R):
        g_step.replay()
        marks[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    per_replay = sorted(marks[j].elapsed_time(marks[j + 1]) / R for j in range(steps // R))
    ms_per_step_median = per_replay[len(per_replay) // 2]
    if st.gemm_flop:
        value, value_unit = st.gemm_flop / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, value_unit = st.step_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"

    log("[bench] step: %.2f us, %.1f %s" % (ms_per_step * 1e3, value, value_unit))
    log("[bench] per-kernel timing")
    reps = max(4, min(200, steps // R))
    kernels = time_kernels(torch, st, reps)
    dom = st.dominant or max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dom]
    kind = [k for (n, _, k, _) in st.kernels if n == dom][0]
    roofline = {"kernel": dom, "bound": kind, "achieved": dk["achieved"],
                "peak": HBM_PEAK_GBS if kind == "hbm" else FP8_PEAK_TFLOPS, "unit": dk["unit"],
                "frac": dk["frac"], "traffic": None,
                "algorithmic_per_launch": dk["algorithmic"], "avg_launch_us": dk["us"]}
    if kind == "mfma":
        roofline["peak_note"] = ("dense FP8 MFMA peak (the metric's unit); the FP8 codes are multiplied "
                                 "exactly on the fp16 matrix core, whose dense peak is 2500 TFLOP/s")
        roofline["frac_of_fp16_peak"] = dk["frac_of_fp16_peak"]
    traffic_file = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(traffic_file):
        rec = json.load(open(traffic_file)).get("%s/%s" % (args.workload, dom))
        if rec and rec.get("source_sha") == source_hash(*KERNEL_SOURCES[dom]):
            roofline["traffic"] = rec["bytes_per_launch"]

    extra = {}
    if args.workload == "large" and not args.no_extra:
        # the decode step's kernels, timed the same way (its own rotated weights)
        del st, g_step
        torch.cuda.empty_cache()
        log("[bench] decode step kernels (8B up-proj, X[64,4096], W[14336,4096])")
        sd = build_step("decode", torch, fl, synthetic)
        extra = {"workload": sd.config["workload"], "weight_copies_rotated": sd.rotate,
                 "kernels": time_kernels(torch, sd, 200)}
        del sd

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample)")
        cpu = cpu_baseline(args.workload, synthetic)
        log("[bench]  oracle: %.6f %s in %.1f s on %d threads" % (cpu["value"], cpu["unit"], cpu["seconds"],
                                                                 cpu["cores"]))

    line = {
        "metric": "FP8 block-scaled GEMM TFLOP/s (% of FP8 MFMA peak); quant GB/s (% HBM)",
        "value": round(value, 2), "unit": value_unit, "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms_per_step, 5), "ms_per_step_median": round(ms_per_step_median, 5),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": st_config, "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    if R > 1 and (steps != args.steps or warm != args.warmup):
        line["rounding"] = ("steps and warmup rounded up to a multiple of the %d-copy weight rotation "
                            "(asked: %d and %d)" % (R, args.steps, args.warmup))
    if extra:
        line["kernels_decode"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
