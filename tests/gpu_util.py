"""Helpers shared by the GPU tests: host bits <-> device tensors, error norms."""
import sys

import numpy as np
import torch

import oracle
import sparse_gemm_02_amd as S

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(bits: np.ndarray) -> torch.Tensor:
    """Raw host bits -> device tensor (uint16 -> bfloat16, uint32 -> float32, float16 and uint8 stay)."""
    bits = np.ascontiguousarray(bits)
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    if bits.dtype == np.uint32:
        return torch.from_numpy(bits.view(np.float32)).to(DEV)
    if bits.dtype == np.float16:
        return torch.from_numpy(bits).to(DEV)
    if bits.dtype == np.uint8:
        return torch.from_numpy(bits).to(DEV)
    raise TypeError(bits.dtype)


def dev_meta(meta: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(meta).view(np.int32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> raw host bits (bf16 -> uint16, f32 -> uint32, int32 -> uint32; fp16 stays float16)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    if t.dtype == torch.float16:
        return t.numpy()
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
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]


# tolerances: bf16 outputs with fp32 accumulation, and the fp32 path
TOL = {"bf16": 1e-2, "f16": 1e-2, "f32": 1e-5}


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


def spacing(x, fmt):
    """Distance between neighbouring representable values at |x| (bf16, f16 or fp32)."""
    mant, tiny = {"bf16": (8, -133), "f16": (11, -24), "f32": (24, -149)}[fmt]
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, np.maximum(e - mant, tiny))


def check_adamw_update(p0, g, m0, v0, step, hp, p_gpu, m_gpu, v_gpu):
    """Stored values and moments against the oracle, within the derived bound."""
    fmt = {np.dtype(np.uint16): "bf16", np.dtype(np.float16): "f16"}.get(np.asarray(p0).dtype, "f32")
    p_ref, m_ref, v_ref = oracle.adamw_compressed(p0, g, m0, v0, step, **hp)
    pe, me, ve = oracle.adamw_update(oracle.widen(p0), oracle.widen(g), m0, v0, step, **hp)
    gw = oracle.widen(g)
    b1, b2 = hp["beta1"], hp["beta2"]
    step_size = hp["lr"] / (1 - b1 ** step)
    den = np.sqrt(ve / (1 - b2 ** step)) + hp["eps"]
    m_terms = b1 * np.abs(m0) + (1 - b1) * np.abs(gw)
    v_terms = b2 * v0 + (1 - b2) * gw * gw
    upd = step_size * np.abs(me) / den
    err = 2.0 ** -20 * np.abs(oracle.widen(p0)) + 2.0 ** -18 * (upd + step_size * m_terms / den)
    got, want = oracle.widen(p_gpu), oracle.widen(p_ref)
    bound = spacing(np.maximum(np.abs(got), np.abs(want)), fmt) + err
    bad = np.abs(got - want) > bound
    assert not bad.any(), (np.flatnonzero(bad)[:5], got[bad][:5], want[bad][:5], pe[bad][:5])
    if fmt != "f32":        # the fp32 error is far below a 16-bit spacing: nearly every value rounds alike
        assert (p_gpu == p_ref).mean() >= 0.99
    assert (np.abs(m_gpu.astype(np.float64) - m_ref) <= spacing(m_ref, "f32") + 2.0 ** -20 * m_terms).all()
    assert (np.abs(v_gpu.astype(np.float64) - v_ref) <= spacing(v_ref, "f32") + 2.0 ** -20 * v_terms).all()


def pack_sparse_reference(vals_bits, meta_words, rows, cols):
    """The tile-chunk layout as include/slope.h states it, built with numpy."""
    S_ = -(-cols // 64)
    tiles = -(-rows // 256)
    wpr = meta_words.shape[1]
    out = np.zeros((tiles, S_, 18432), dtype=np.uint8)
    vb = np.zeros((tiles * 256, S_ * 32), dtype=np.uint16)
    vb[:rows, :cols // 2] = vals_bits
    mw = np.zeros((tiles * 256, 2 * S_), dtype=np.uint32)
    mw[:rows, :wpr] = meta_words
    for t in range(tiles):
        for s_ in range(S_):
            blk = vb[256 * t:256 * t + 256, 32 * s_:32 * s_ + 32].reshape(256, 4, 8)   # [row][granule][value]
            a = np.zeros((256, 4, 8), dtype=np.uint16)
            for r in range(256):
                for c in range(4):
                    a[r, c ^ ((r >> 2) & 3)] = blk[r, c]
            out[t, s_, :16384] = a.reshape(-1).view(np.uint8)
            out[t, s_, 16384:] = np.ascontiguousarray(mw[256 * t:256 * t + 256, 2 * s_:2 * s_ + 2]).view(np.uint8).reshape(-1)
    return out.reshape(-1)
