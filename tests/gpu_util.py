"""Helpers shared by the GPU tests: host bits <-> device tensors, error norms."""
import sys

import numpy as np
import torch

import sparse_gemm_02_amd as S

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(bits: np.ndarray) -> torch.Tensor:
    """Raw host bits -> device tensor (uint16 -> bfloat16, uint32 -> float32, uint8 stays)."""
    bits = np.ascontiguousarray(bits)
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    if bits.dtype == np.uint32:
        return torch.from_numpy(bits.view(np.float32)).to(DEV)
    if bits.dtype == np.uint8:
        return torch.from_numpy(bits).to(DEV)
    raise TypeError(bits.dtype)


def dev_meta(meta: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(meta).view(np.int32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> raw host bits (bf16 -> uint16, f32 -> uint32, int32 -> uint32)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=DEV)


def normwise(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 for an all-zero reference matched exactly)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    if scale == 0:
        return float(err)
    return float(err / scale)


def torch_dtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


# tolerances: bf16 outputs with fp32 accumulation, and the fp32 path
TOL = {"bf16": 1e-2, "f32": 1e-5}


class Compressed:
    """Device buffers of a compressed [rows, cols] 2:4 matrix."""

    def __init__(self, rows, cols, dtype):
        nv, nm = S.slope_compressed_sizes(rows, cols)
        self.values = empty((rows, cols // 2), dtype)
        self.meta = torch.empty((rows, (cols // 4 + 7) // 8), dtype=torch.int32, device=DEV)
        assert self.values.numel() == nv and self.meta.numel() == nm


def workspace(T, K, r, N):
    b = S.slope_lowrank_workspace_bytes(T, K, r, N)
    return torch.empty(max(b, 16), dtype=torch.uint8, device=DEV)
