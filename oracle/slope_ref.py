"""Plain CPU oracle of the SLoPe 2:4 sparse linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the entry module
and the CPU-baseline leg of the benchmark use it.  It shares no code with the
GPU library (no kernels, headers, helpers or tables) and imports nothing from it.

What it computes follows the SLoPe pages ("SLoPe: Double-Pruned Sparse Plus
Lazy Low-Rank Adapter Pretraining of LLMs"):

* the AI summary page (atlas.scime.ai), sections Problem and Approach,
* the technical explainer (gist.science), Technical Summary sections 1
  (Problem Statement), 2.A (Double-Pruned Backward Pass), 2.B (Lazy Low-Rank
  Adapters), 2.C (Optimized CUDA Kernels),
* the OpenReview discussion (paperhub.cn), sections "Impact of Introducing
  Additional Zeros in N:M Pattern", "Memory Footprint Reduction During
  Pretraining and Inference", "Clarification on Inference Speedup and Sparse
  Pre-Training" and "Choice of Optimizer".

Conventions (W is [N, K] = [out, in] as for a linear layer):

    Y  = X . W_s^T            X [T, K], W_s = W (.) M_s, 2:4 groups along K
    dX = dY . W_dp            W_dp^T = prune24(W_s^T): 2:4 groups along N
    dW = (dY^T . X) (.) M_s   kept only at the static forward mask
    Y += (X . L) . R          L [K, r], R [r, N]  (W_dense = W_sparse + L R)
    dX += (dY . R^T) . L^T, dL = X^T . (dY . R^T), dR = (X . L)^T . dY
    AdamW on the compressed values of W_s (moments only for the kept slots),
    then the double prune of the updated W_s

Tensors arrive as raw bit patterns (uint16 = bf16, uint32 = fp32) or as numpy
float16 arrays (fp16), so every selection is made on the exact stored values.  Products and sums are done in
float64 on the exactly widened inputs and returned unrounded.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):

* criterion: magnitude; keep the two largest |w| of every 4 (the pages name
  N:M with N:M = 2:4 but not the score);
* ties: equal magnitudes (including +0 / -0 and x / -x) go to the lower index;
  NaN ranks above every number and NaNs tie with each other;
* a pruned entry becomes +0 (all bits clear);
* stored metadata: per group the two kept positions i0 < i1 as 2-bit fields,
  nibble = i0 | i1 << 2, group g at bits 4*(g%8) of uint32 word g//8 of its row;
* double pruning is deterministic: the current W_s is transposed and pruned
  again with the same rule, every time it is called (no random element).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "prune24", "prune_nm", "compress24", "decompress24", "mask_from_meta",
    "double_prune", "spmm_fwd", "spmm_bwd_dx", "masked_wgrad", "lowrank_add", "lowrank_bwd",
    "round_bf16", "round_f16", "round_f32", "adamw_update", "adamw_compressed", "adamw_double_prune",
    "storage_accounting", "LEGAL_NIBBLES",
    "E4M3_MAX", "decode_e4m3", "round_e4m3", "e4m3_scale", "quantize_e4m3", "spmm_e4m3",
]

# The six ways to keep 2 of 4 positions, as nibbles i0 | i1 << 2 with i0 < i1.
LEGAL_NIBBLES = frozenset(i0 | (i1 << 2) for i0 in range(4) for i1 in range(i0 + 1, 4))


# --------------------------------------------------------------------------- values

def widen(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of raw bf16 (uint16) or fp32 (uint32) bit patterns,
    or of fp16 values (numpy float16 arrays)."""
    bits = np.asarray(bits)
    if bits.dtype == np.uint16:
        f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif bits.dtype == np.uint32:
        f32 = bits.view(np.float32)
    elif bits.dtype == np.float16:
        return bits.astype(np.float64)
    else:
        raise TypeError(f"raw bits must be uint16 (bf16), uint32 (fp32) or float16, got {bits.dtype}")
    return f32.astype(np.float64)


def _ranks_above(mag, nan, i, j):
    """Where element i of each group ranks strictly above element j.

    Larger magnitude ranks higher; NaN ranks above every number; equal
    magnitudes (and two NaNs) are broken toward the lower index.
    """
    mi, mj = mag[..., i], mag[..., j]
    ni, nj = nan[..., i], nan[..., j]
    larger = (ni & ~nj) | (~ni & ~nj & (mi > mj))
    tie = (ni & nj) | (~ni & ~nj & (mi == mj))
    return larger | (tie & (i < j))


# --------------------------------------------------------------------------- prune / compress

def prune24(A: np.ndarray):
    """Magnitude 2:4 pruning along the rows of A (groups of 4 consecutive columns).

    Forward weight W^R: pruned along its rows (the explainer's section 2.A); N:M
    with 2:4 in the summary page's Approach.  Within each group the element j is kept
    iff fewer than two elements rank above it (magnitude, ties to lower index).

    Returns (mask uint8 [rows, cols] with 1 at kept positions,
             A_s: bits of A at kept positions, +0 elsewhere).
    """
    A = np.asarray(A)
    rows, cols = A.shape
    if cols % 4:
        raise ValueError("the pruned dimension must be a multiple of 4")
    v = widen(A).reshape(rows, cols // 4, 4)
    mag, nan = np.abs(v), np.isnan(v)
    keep = np.zeros(v.shape, dtype=bool)
    for j in range(4):
        above = np.zeros(v.shape[:-1], dtype=np.int64)
        for i in range(4):
            if i != j:
                above += _ranks_above(mag, nan, i, j)
        keep[..., j] = above < 2
    mask = keep.reshape(rows, cols).astype(np.uint8)
    A_s = np.where(mask != 0, A, np.zeros((), dtype=A.dtype)).astype(A.dtype)
    return mask, A_s


def prune_nm(A: np.ndarray, n: int, m: int):
    """Magnitude N:M pruning along the rows of A: in every group of m
    consecutive columns the n highest-ranked elements are kept (same ranking as
    prune24: magnitude, NaN above every number, ties to the lower index).

    The explainer's Technical Summary 1 (Problem Statement) introduces N:M
    structured sparsity in general; its "N zeros out of M" is read, as for 2:4,
    as n kept (non-zero) positions out of every m.  prune24 is the case n = 2,
    m = 4.  Element j is kept iff fewer than n elements of its group rank above it.

    Returns (mask uint8 [rows, cols], A_s: bits of A at kept positions, +0 elsewhere).
    """
    A = np.asarray(A)
    rows, cols = A.shape
    if m < 1 or not 1 <= n <= m:
        raise ValueError("need 1 <= n <= m")
    if cols % m:
        raise ValueError("the pruned dimension must be a multiple of m")
    v = widen(A).reshape(rows, cols // m, m)
    mag, nan = np.abs(v), np.isnan(v)
    keep = np.zeros(v.shape, dtype=bool)
    for j in range(m):
        above = np.zeros(v.shape[:-1], dtype=np.int64)
        for i in range(m):
            if i != j:
                above += _ranks_above(mag, nan, i, j)
        keep[..., j] = above < n
    mask = keep.reshape(rows, cols).astype(np.uint8)
    A_s = np.where(mask != 0, A, np.zeros((), dtype=A.dtype)).astype(A.dtype)
    return mask, A_s


def compress24(A: np.ndarray, mask: np.ndarray):
    """Compressed 2:4 form: two values and two 2-bit positions per group of 4.

    Storage of the discussion page's "Memory Footprint" section (two 16-bit
    non-zeros plus their indices per four elements).  For every group the two
    slots are the kept positions in ascending order.  A group with fewer than
    two kept positions is filled with its lowest unkept positions, whose value
    is +0; a group with more than two keeps its two lowest kept positions and is
    counted as invalid.

    Returns (values [rows, cols/2] (same bit type as A),
             meta uint32 [rows, ceil(cols/32)],
             number of invalid groups).
    """
    A = np.asarray(A)
    rows, cols = A.shape
    if cols % 4 or mask.shape != A.shape:
        raise ValueError("bad shapes for compress24")
    groups = cols // 4
    kept = (np.asarray(mask) != 0).reshape(rows, groups, 4)
    invalid = int((kept.sum(axis=-1) > 2).sum())
    # Order positions: kept ones first, each part in ascending position.
    order_key = np.where(kept, 0, 4) + np.arange(4)
    first_two = np.sort(np.argsort(order_key, axis=-1, kind="stable")[..., :2], axis=-1)
    i0, i1 = first_two[..., 0], first_two[..., 1]
    G = A.reshape(rows, groups, 4)
    zero = np.zeros((), dtype=A.dtype)
    v0 = np.where(np.take_along_axis(kept, i0[..., None], -1)[..., 0],
                  np.take_along_axis(G, i0[..., None], -1)[..., 0], zero)
    v1 = np.where(np.take_along_axis(kept, i1[..., None], -1)[..., 0],
                  np.take_along_axis(G, i1[..., None], -1)[..., 0], zero)
    values = np.stack([v0, v1], axis=-1).reshape(rows, groups * 2).astype(A.dtype)

    nib = (i0 | (i1 << 2)).astype(np.uint64)
    words = -(-groups // 8)
    padded = np.zeros((rows, words * 8), dtype=np.uint64)
    padded[:, :groups] = nib
    shifts = (4 * np.arange(8, dtype=np.uint64))
    meta = (padded.reshape(rows, words, 8) << shifts).sum(axis=-1).astype(np.uint32)
    return values, meta, invalid


def _positions(meta: np.ndarray, cols: int):
    rows = meta.shape[0]
    groups = cols // 4
    if meta.shape[1] != -(-groups // 8):
        raise ValueError("metadata has the wrong number of words per row")
    g = np.arange(groups)
    nib = (meta[:, g // 8].astype(np.uint64) >> (4 * (g % 8)).astype(np.uint64)) & np.uint64(0xF)
    nib = nib.astype(np.int64)
    bad = ~np.isin(nib, sorted(LEGAL_NIBBLES))
    if bad.any():
        raise ValueError("metadata holds a nibble that is not a pair i0 < i1")
    return nib & 3, nib >> 2, rows, groups


def decompress24(values: np.ndarray, meta: np.ndarray, cols: int) -> np.ndarray:
    """Inverse of compress24: dense [rows, cols] bits, +0 at unkept positions."""
    i0, i1, rows, groups = _positions(meta, cols)
    values = np.asarray(values).reshape(rows, groups, 2)
    dense = np.zeros((rows, groups, 4), dtype=values.dtype)
    np.put_along_axis(dense, i0[..., None], values[..., 0:1], -1)
    np.put_along_axis(dense, i1[..., None], values[..., 1:2], -1)
    return dense.reshape(rows, cols)


def mask_from_meta(meta: np.ndarray, cols: int) -> np.ndarray:
    """Dense 0/1 mask [rows, cols] of the positions named by the metadata."""
    i0, i1, rows, groups = _positions(meta, cols)
    m = np.zeros((rows, groups, 4), dtype=np.uint8)
    np.put_along_axis(m, i0[..., None], 1, -1)
    np.put_along_axis(m, i1[..., None], 1, -1)
    return m.reshape(rows, cols)


def double_prune(values_s: np.ndarray, meta_s: np.ndarray, N: int, K: int):
    """Double-pruned backward weight W^{R,C}.

    Explainer section 2.A and Key Contributions: the already 2:4-sparse W_s is
    transposed and pruned 2:4 a second time, so the backward operand is N:M
    sparse along its new rows (the output dimension N).  The discussion page
    keeps the result as a second compressed copy next to the weight.

    Returns (values_dpT [K, N/2], meta_dpT [K, ceil(N/32)], mask_dpT [K, N]).
    """
    W_s = decompress24(values_s, meta_s, K)
    if W_s.shape != (N, K):
        raise ValueError("compressed weight does not match N x K")
    W_sT = np.ascontiguousarray(W_s.T)
    mask_dpT, _ = prune24(W_sT)
    values_dpT, meta_dpT, _ = compress24(W_sT, mask_dpT)
    return values_dpT, meta_dpT, mask_dpT


# --------------------------------------------------------------------------- products

def spmm_fwd(X, values_s, meta_s, K, L=None, R=None) -> np.ndarray:
    """Y = X . W_s^T (+ (X . L) . R when both adapter factors are given).

    Forward pass with the row-wise pruned weight (explainer 2.A) and the
    unmerged low-rank term W_dense = W_sparse + L R (explainer 2.B; discussion
    page, "SLoPe inference computation": adapters stay unmerged).
    """
    W_s = widen(decompress24(values_s, meta_s, K))
    x = widen(X)
    Y = x @ W_s.T
    if L is not None and R is not None and np.asarray(L).shape[1] > 0:
        Y = Y + (x @ widen(L)) @ widen(R)
    return Y


def spmm_bwd_dx(dY, values_dpT, meta_dpT, N) -> np.ndarray:
    """dX = dY . W_dp, with W_dp the transpose of the double-pruned W_dp^T [K, N]."""
    W_dpT = widen(decompress24(values_dpT, meta_dpT, N))
    return widen(dY) @ W_dpT.T


def masked_wgrad(dY, X, meta_s, K, dW_values_in=None, dW_dense_in=None):
    """Weight gradient kept at the static mask: dW = (dY^T . X) (.) M_s.

    The discussion page counts two 16-bit gradient values per four weights
    and, for fine-tuning, updates only the weights that are not pruned; the
    values are laid out in W_s's compressed slot order.  With ``dW_*_in`` given the result
    is added to them (gradient accumulation).

    Returns (dW_values [N, K/2] float64, dW_dense [N, K] float64).
    """
    G = widen(dY).T @ widen(X)
    N = G.shape[0]
    i0, i1, rows, groups = _positions(meta_s, K)
    if rows != N:
        raise ValueError("metadata rows must equal N")
    Gg = G.reshape(N, groups, 4)
    vals = np.stack([np.take_along_axis(Gg, i0[..., None], -1)[..., 0],
                     np.take_along_axis(Gg, i1[..., None], -1)[..., 0]], axis=-1).reshape(N, K // 2)
    dense = G * mask_from_meta(meta_s, K)
    if dW_values_in is not None:
        vals = vals + widen(dW_values_in)
    if dW_dense_in is not None:
        dense = dense + widen(dW_dense_in)
    return vals, dense


def lowrank_add(X, L, R, Y_in=None):
    """Adapter term: XL = X . L, Y = Y_in + XL . R (explainer 2.B); Y_in is raw bits.

    Returns (XL [T, r] float64, Y [T, N] float64).
    """
    XL = widen(X) @ widen(L)
    Y = XL @ widen(R)
    if Y_in is not None:
        Y = Y + widen(Y_in)
    return XL, Y


def lowrank_bwd(X, dY, L, R):
    """Gradients of the adapter term Y += (X . L) . R (explainer 2.B) for an
    output gradient dY: the term is bilinear, so with G = dY . R^T [T, r]

        dX += G . L^T        [T, K]
        dL  = X^T . G        [K, r]
        dR  = (X . L)^T . dY [r, N]

    Returns (dX_term, dL, dR) as float64 (not rounded).
    """
    Xw, dYw, Lw, Rw = widen(X), widen(dY), widen(L), widen(R)
    G = dYw @ Rw.T
    return G @ Lw.T, Xw.T @ G, (Xw @ Lw).T @ dYw


# --------------------------------------------------------------------------- optimizer

def round_bf16(x) -> np.ndarray:
    """bf16 bit patterns (uint16) nearest to float64 values, ties to even.

    Rounds once, straight from float64 (no intermediate fp32 rounding): the
    value is scaled so that the bf16 quantum of its binade (2**(e-8) for
    2**(e-1) <= |x| < 2**e, never below the subnormal quantum 2**-133) becomes
    1, rounded half-to-even, and scaled back; past the largest finite bf16 it
    becomes an infinity, NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_f16(x) -> np.ndarray:
    """fp16 values nearest to float64 values, ties to even (one rounding,
    straight from float64; past the largest finite fp16 an infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


def round_f32(x) -> np.ndarray:
    """fp32 values nearest to float64 values, ties to even (IEEE conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32)


def adamw_update(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    """One AdamW step in float64: Adam moments with bias correction and weight
    decay decoupled from the gradient (Loshchilov and Hutter, "Decoupled
    Weight Decay Regularization", Algorithm 2), in the common library form
    where the learning rate scales both terms:

        m <- beta1 m + (1 - beta1) g
        v <- beta2 v + (1 - beta2) g^2
        p <- p - lr * weight_decay * p - lr * m_hat / (sqrt(v_hat) + eps)
        m_hat = m / (1 - beta1^step), v_hat = v / (1 - beta2^step)

    step counts updates from 1.  Returns (p, m, v) as float64, unrounded.
    """
    p, g, m, v = (np.asarray(a, dtype=np.float64) for a in (p, g, m, v))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * weight_decay * p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def adamw_compressed(values, grads, m, v, step, **hp):
    """AdamW on the stored non-zeros of a 2:4 weight.

    The discussion page trains SLoPe with AdamW ("Choice of Optimizer") and
    counts the optimizer state as two 32-bit moments for each of the two
    non-zeros of every four weights ("Memory Footprint Reduction During
    Pretraining and Inference"): the update runs on the compressed values, the
    pruned positions have no state and stay zero, the mask does not move.

    values: the compressed values (uint16 bf16 bits, float16, or uint32 fp32
    bits); grads: the gradient in the same slot order (any of those formats);
    m, v: float32 moments of the same shape.  The step is computed in float64
    and stored once: values rounded to their own format, moments to fp32.
    Returns (values bits, m float32, v float32).
    """
    values = np.asarray(values)
    p, m1, v1 = adamw_update(widen(values), widen(grads), np.asarray(m, np.float32),
                             np.asarray(v, np.float32), step, **hp)
    if values.dtype == np.uint16:
        out = round_bf16(p)
    elif values.dtype == np.float16:
        out = round_f16(p)
    else:
        out = round_f32(p).view(np.uint32)
    return out, round_f32(m1), round_f32(v1)


def adamw_double_prune(values_s, meta_s, dW_values, m, v, N, K, step, **hp):
    """The weight update of one SLoPe training step: AdamW on the compressed
    values of W_s (static mask, metadata unchanged), then the double-pruned
    transposed copy of the updated weight for the next backward pass
    (explainer 2.A: the column mask follows the current weights).

    Returns (values_s bits, m, v, values_dpT, meta_dpT, mask_dpT).
    """
    vals, m1, v1 = adamw_compressed(values_s, dW_values, m, v, step, **hp)
    return (vals, m1, v1) + tuple(double_prune(vals, meta_s, N, K))


# --------------------------------------------------------------------------- accounting

def storage_accounting(value_bits=16, index_bits=3, mask_bits=8, moment_bits=32):
    """Per-four-element storage of the 2:4 layer relative to dense.

    Discussion page, "Memory Footprint Reduction During Pretraining and
    Inference": inference keeps two non-zero values plus their indices per four
    weights; training keeps the weight, its double-pruned transposed copy (each
    values plus indices), a binary mask of one byte per weight, the gradient at
    the two non-zeros and two optimizer moments at the two non-zeros, against a
    dense weight, gradient and two moments.

    Returns (inference ratio, training ratio) as exact fractions of floats.
    """
    sparse_weight = 2 * value_bits + index_bits
    inference = sparse_weight / (4 * value_bits)
    sparse_train = (sparse_weight            # weight
                    + sparse_weight          # transposed copy for the backward pass
                    + 4 * mask_bits          # binary mask
                    + 2 * value_bits         # gradient at the non-zeros
                    + 2 * 2 * moment_bits)   # two optimizer moments at the non-zeros
    dense_train = 4 * value_bits + 4 * value_bits + 2 * 4 * moment_bits
    return inference, sparse_train / dense_train


# --------------------------------------------------------------------------- 8-bit (e4m3) variant

# The explainer's Technical Summary 1 (Problem Statement) names N:M sparsity
# in general and the discussion page ("Memory Footprint Reduction During
# Pretraining and Inference") counts 16-bit values; neither gives an 8-bit
# format or a scaling rule.  The 8-bit variant here is a reading taken for them:
# the OCP FP8 E4M3 format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
# bits, subnormals, no infinities, the all-ones codes 0x7F / 0xFF are NaN,
# largest finite value 448), one scale per tensor chosen from its largest
# magnitude, products accumulated in float32 and the two scales divided out
# at the end.

E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """Exact float64 values of E4M3 codes (uint8), from the format definition:
    exponent field e and mantissa field m give (1 + m/8) * 2^(e - 7) for
    e >= 1 and (m/8) * 2^-6 for e == 0; codes 0x7F and 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def round_e4m3(x) -> np.ndarray:
    """E4M3 codes (uint8) nearest to float64 values, ties to the even code
    (even mantissa), saturating: magnitudes beyond 448 give +-448 (a reading
    taken here; a conversion to the largest finite value, since the format has no
    infinity).  NaN gives 0x7F; the sign of zero is kept.

    Written as a nearest-value search over the 127 finite non-negative codes."""
    x = np.asarray(x, dtype=np.float64)
    table = decode_e4m3(np.arange(0x7F, dtype=np.uint8))          # 0x00 .. 0x7E, increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = np.abs(a - table[lo]), np.abs(table[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = pick.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_scale(bits) -> np.float32:
    """Per-tensor scale of the 8-bit variant: 448 / amax as one float32
    division (round to nearest), amax the largest magnitude of the stored
    16-bit values (exact); 1 when amax is 0 or not finite."""
    a = np.abs(widen(bits))
    amax = float(np.max(a)) if a.size else 0.0
    if not (amax > 0.0) or not np.isfinite(amax):
        return np.float32(1.0)
    return np.float32(np.float32(E4M3_MAX) / np.float32(amax))


def quantize_e4m3(bits, scale) -> np.ndarray:
    """E4M3 codes of stored 16-bit values times a float32 scale: the product is
    rounded to float32 once (the kernel's precision, which decides the code),
    then to E4M3 with round_e4m3."""
    prod = widen(bits).astype(np.float32) * np.float32(scale)
    return round_e4m3(prod.astype(np.float64))


def spmm_e4m3(Xq, x_scale, values_q, meta_q, K, w_scale) -> np.ndarray:
    """The 2:4 product on E4M3 operands: Y = (Xq . W_q^T) / (x_scale * w_scale)
    with W_q the decompressed E4M3 weight (values_q [N, K/2] codes, meta_q the
    same 2:4 metadata as the 16-bit weight).  Exact float64 products and sums,
    returned unrounded; it serves the forward (X, W_s) and dX (dY, W_dp^T)."""
    Xd = decode_e4m3(Xq)
    Wd = decode_e4m3(decompress24(np.asarray(values_q, dtype=np.uint8), meta_q, K))   # code 0 (+0) elsewhere
    return (Xd @ Wd.T) / (float(x_scale) * float(w_scale))
