"""Seeded synthetic inputs and layer shapes for the 2:4 sparse linear layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds none of the method's arithmetic: only layer shapes, random
draws, and the rounding of those draws to the storage precision of the inputs.

Shapes follow the workloads the SLoPe pages train and serve (GPT-2-small,
BERT-Large, OPT-13B, OPT-66B; "SLoPe" summary page, Key results and
Experimental setup; explainer page, section 4): each transformer layer has four
linears (QKV, attention output O, FC1, FC2), given as (K -> N) = (in -> out).
The pages publish no datasets or weights that fit this path, so Gaussian
synthetic tensors stand in for them:

    W ~ N(0, 0.02)  [N, K]      X  ~ N(0, 1)  [T, K]      dY ~ N(0, 1)  [T, N]
    L ~ N(0, 0.02)  [K, r]      R  ~ N(0, 0.02)  [r, N]

Recipe (deterministic, parallel): for linear number ``i`` of a workload and
base seed ``s``, ``SeedSequence([s, i]).spawn(5)`` gives one child per tensor in
the order W, X, dY, L, R.  A tensor is drawn in row chunks of ``CHUNK_ROWS``
rows; chunk ``c`` uses ``default_rng(child.spawn(n_chunks)[c])`` and draws
float64 standard normals, scaled by the tensor's sigma, then cast to float32
(round to nearest even) and, for bf16 workloads, rounded to bf16 (round to
nearest even on the float32 bit pattern), for fp16 ones to fp16 (numpy's
conversion, nearest even).  Tensors are returned as raw bit patterns:
``uint16`` for bf16 and ``uint32`` for fp32; fp16 tensors as numpy ``float16``.

Optimizer-step inputs of linear ``i`` (``optimizer_inputs``): a gradient in
the compressed slot order G [N, K/2] ~ N(0, 1) in the workload's precision and
two fp32 moment arrays M ~ N(0, 0.1) and V = Z^2 with Z ~ N(0, 0.1), from the
children of ``SeedSequence([s, i, 1]).spawn(3)``, drawn with the same chunked
recipe.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Linear", "Workload", "WORKLOADS", "SIGMA", "CHUNK_ROWS",
    "f32_to_bf16_bits", "bits_to_float32", "draw", "layer_inputs", "optimizer_inputs",
]

CHUNK_ROWS = 1024
SIGMA = {"W": 0.02, "X": 1.0, "dY": 1.0, "L": 0.02, "R": 0.02}
_ORDER = ("W", "X", "dY", "L", "R")


@dataclass(frozen=True)
class Linear:
    name: str
    K: int  # input features (forward reduction dimension)
    N: int  # output features


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": storage precision of every input
    T: int                # tokens of the training step
    r: int                # adapter rank
    linears: tuple = field(default_factory=tuple)
    decode_T: tuple = ()  # token counts of the inference (decode) shapes


WORKLOADS = {
    "toy_fp32": Workload("toy_fp32", "f32", T=64, r=8,
                         linears=(Linear("linear", 256, 256),)),
    "gpt2_small": Workload("gpt2_small", "bf16", T=8 * 1024, r=16,
                           linears=(Linear("qkv", 768, 2304), Linear("o", 768, 768),
                                    Linear("fc1", 768, 3072), Linear("fc2", 3072, 768))),
    "bert_large": Workload("bert_large", "bf16", T=32 * 512, r=64,
                           linears=(Linear("qkv", 1024, 3072), Linear("o", 1024, 1024),
                                    Linear("ffn1", 1024, 4096), Linear("ffn2", 4096, 1024))),
    "opt_13b": Workload("opt_13b", "bf16", T=4096, r=40, decode_T=(16,),
                        linears=(Linear("qkv", 5120, 15360), Linear("o", 5120, 5120),
                                 Linear("fc1", 5120, 20480), Linear("fc2", 20480, 5120))),
    "opt_66b": Workload("opt_66b", "bf16", T=8192, r=72, decode_T=(1, 64),
                        linears=(Linear("qkv", 9216, 27648), Linear("o", 9216, 9216),
                                 Linear("fc1", 9216, 36864), Linear("fc2", 36864, 9216))),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    NaN inputs keep a quiet-NaN pattern; the generator never produces them.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """View raw bf16 (uint16) or fp32 (uint32) bits as float32 values."""
    if bits.dtype == np.uint16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if bits.dtype == np.uint32:
        return bits.view(np.float32)
    raise TypeError(f"expected uint16 or uint32 bits, got {bits.dtype}")


_STORE = {"bf16": np.uint16, "f16": np.float16, "f32": np.uint32}


def _draw_chunk(seed_seq, rows, cols, sigma, dtype):
    g = np.random.default_rng(seed_seq)
    v = (g.standard_normal((rows, cols)) * sigma).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    if dtype == "f16":
        return v.astype(np.float16)
    return v.view(np.uint32).copy()


def draw(seed_seq: np.random.SeedSequence, shape, sigma: float, dtype: str,
         threads: int | None = None) -> np.ndarray:
    """Draw one tensor of ``shape`` = (rows, cols) following the module recipe."""
    rows, cols = int(shape[0]), int(shape[1])
    n_chunks = max(1, -(-rows // CHUNK_ROWS))
    # the children a fresh seed_seq.spawn(n_chunks) would hand out, built
    # without changing seed_seq (spawn() advances its counter)
    base = tuple(seed_seq.spawn_key)
    kids = [np.random.SeedSequence(seed_seq.entropy, spawn_key=base + (c,),
                                   pool_size=seed_seq.pool_size) for c in range(n_chunks)]
    out = np.empty((rows, cols), dtype=_STORE[dtype])
    spans = [(c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)) for c in range(n_chunks)]

    def work(c):
        a, b = spans[c]
        out[a:b] = _draw_chunk(kids[c], b - a, cols, sigma, dtype)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if n_chunks == 1 or nthreads == 1:
        for c in range(n_chunks):
            work(c)
    else:
        with _cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def layer_inputs(K: int, N: int, T: int, r: int, dtype: str, seed: int = 0,
                 index: int = 0, which=_ORDER, threads: int | None = None) -> dict:
    """Inputs of one linear: raw bits of W [N,K], X [T,K], dY [T,N], L [K,r], R [r,N].

    ``which`` restricts the tensors drawn (the others are not generated); the
    draws of a tensor do not depend on which others are requested.
    """
    if dtype not in _STORE:
        raise ValueError(dtype)
    kids = dict(zip(_ORDER, np.random.SeedSequence([seed, index]).spawn(len(_ORDER))))
    shapes = {"W": (N, K), "X": (T, K), "dY": (T, N), "L": (K, r), "R": (r, N)}
    return {name: draw(kids[name], shapes[name], SIGMA[name], dtype, threads)
            for name in _ORDER if name in which}


def optimizer_inputs(N: int, K: int, dtype: str, seed: int = 0, index: int = 0,
                     threads: int | None = None) -> dict:
    """Gradient (raw bits) and fp32 moments of one compressed [N, K/2] weight.

    Returns {"G": bits [N, K/2], "M": float32 [N, K/2], "V": float32 [N, K/2]}.
    """
    if dtype not in _STORE:
        raise ValueError(dtype)
    kg, km, kv = np.random.SeedSequence([seed, index, 1]).spawn(3)
    shape = (N, K // 2)
    G = draw(kg, shape, 1.0, dtype, threads)
    M = draw(km, shape, 0.1, "f32", threads).view(np.float32)
    Z = draw(kv, shape, 0.1, "f32", threads).view(np.float32)
    return {"G": G, "M": M, "V": Z * Z}

