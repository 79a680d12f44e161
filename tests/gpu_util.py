"""Helpers shared by the GPU parity tests: host <-> device marshalling."""
import sys

import numpy as np
import torch

DEV = "cuda"


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def first_mismatch(a: np.ndarray, b: np.ndarray):
    idx = np.argwhere(a != b)
    return None if idx.size == 0 else (tuple(idx[0]), a[tuple(idx[0])], b[tuple(idx[0])], len(idx))
