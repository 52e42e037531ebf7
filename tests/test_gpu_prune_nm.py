"""GPU parity of the general N:M magnitude prune (slope_prune_nm) with the oracle.

Masks and pruned weights are integer work: bit-exact.  Inputs mix Gaussian
values with ties, signed zeros, denormals, infinities and NaN; shapes include
ragged row counts, and one case runs at the OPT-66B FC1 weight size (checked
on sampled rows).  The last test feeds a 2:8 pruned weight through the 2:4
compression and the sparse forward.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import f32_to_bf16_bits, layer_inputs

from gpu_util import TOL, dev, dev_meta, empty, host, host_f64, normwise, say, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()


SPECIALS = {
    "bf16": np.array([0x7F80, 0xFF80, 0x7FC0, 0x7FC1, 0x0001, 0x8003, 0x7F7F], dtype=np.uint16),
    "f16": np.array([0x7C00, 0xFC00, 0x7E00, 0x7E01, 0x0001, 0x8003, 0x7BFF], dtype=np.uint16),
    "f32": np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x7FC00001, 0x00000001, 0x80000005, 0x7F7FFFFF],
                    dtype=np.uint32),
}


def _special_matrix(rows, cols, dt, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32) * 0.02
    pick = rng.integers(0, 10, size=(rows, cols))
    v[pick == 0] = 0.0
    v[pick == 1] = -0.0
    v[pick == 2] = np.round(v[pick == 2] * 100) / 100
    v[pick == 3] = -v[pick == 3]
    if dt == "bf16":
        bits = f32_to_bf16_bits(v)
    elif dt == "f16":
        bits = v.astype(np.float16).view(np.uint16)
    else:
        bits = v.view(np.uint32).copy()
    flat = bits.reshape(-1)
    idx = rng.choice(flat.size, size=max(1, flat.size // 50), replace=False)
    flat[idx] = SPECIALS[dt][rng.integers(0, len(SPECIALS[dt]), size=idx.size)]
    return bits.view(np.float16) if dt == "f16" else bits


def _raw(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a


NM = [(1, 4), (3, 4), (2, 4), (1, 8), (2, 8), (4, 8), (2, 16), (5, 16), (2, 32), (16, 32)]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("rows", [1, 37, 256])
def test_prune_nm_bit_exact(dt, n, m, rows):
    cols = 4 * m + (96 if m <= 8 else 0)
    say(f"prune_nm {dt} {n}:{m} {rows}x{cols}")
    W = _special_matrix(rows, cols, dt, 1000 * n + 10 * m + rows)
    mask_ref, Ws_ref = oracle.prune_nm(W, n, m)
    Wd = dev(W)
    mask = torch.full((rows, cols), 7, dtype=torch.uint8, device="cuda")
    Ws = empty((rows, cols), torch_dtype(dt))
    S.slope_prune_nm(Wd, n, m, mask, Ws)
    mask2 = torch.full((rows, cols), 7, dtype=torch.uint8, device="cuda")
    S.slope_prune_nm(Wd, n, m, mask2)                      # W_s is optional
    torch.cuda.synchronize()
    assert (host(mask) == mask_ref).all()
    assert (_raw(host(Ws)) == _raw(Ws_ref)).all()
    assert (host(mask2) == mask_ref).all()


def test_prune_nm_empty():
    mask = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    S.slope_prune_nm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), 2, 8, mask)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n,m", [(2, 8), (1, 4)])
def test_prune_nm_full_size_sampled_rows(n, m):
    """The OPT-66B FC1 weight (36864 x 9216, bf16) pruned in one launch; 64
    sampled rows compared with the oracle bit for bit, every group's count checked."""
    N, K = 36864, 9216
    say(f"prune_nm full size {n}:{m} {N}x{K}")
    Wh_all = layer_inputs(K, N, 1, 1, "bf16", seed=5, which=("W",), threads=16)["W"]
    W = dev(Wh_all)
    mask = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    Ws = torch.empty_like(W)
    S.slope_prune_nm(W, n, m, mask, Ws)
    torch.cuda.synchronize()
    counts = mask.view(N, K // m, m).sum(-1, dtype=torch.int32)
    assert bool((counts == n).all())
    rows = np.random.default_rng(6).choice(N, size=64, replace=False)
    rows.sort()
    idx = torch.from_numpy(rows).cuda()
    mask_ref, Ws_ref = oracle.prune_nm(Wh_all[rows], n, m)
    assert (mask.index_select(0, idx).cpu().numpy() == mask_ref).all()
    assert (Ws.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16) == Ws_ref).all()


@pytest.mark.parametrize("n,m", [(2, 8), (1, 4), (2, 16)])
def test_prune_nm_feeds_24_products(n, m):
    """A weight pruned n:m (n <= 2) goes through the 2:4 compression with no
    invalid group, and the sparse forward computes X . W_nm^T."""
    T, N, K = 96, 256, 512
    say(f"prune_nm -> compress24 -> spmm_fwd {n}:{m} T={T} N={N} K={K}")
    d = layer_inputs(K, N, T, 1, "bf16", seed=n + m, which=("W", "X"))
    W, X = d["W"], d["X"]
    mask_ref, Ws_ref = oracle.prune_nm(W, n, m)
    vals_ref, meta_ref, invalid_ref = oracle.compress24(Ws_ref, mask_ref)
    assert invalid_ref == 0
    mask = empty((N, K), torch.uint8)
    Ws = empty((N, K), torch.bfloat16)
    S.slope_prune_nm(dev(W), n, m, mask, Ws)
    vals = empty((N, K // 2), torch.bfloat16)
    meta = torch.empty((N, (K + 31) // 32), dtype=torch.int32, device="cuda")
    invalid = torch.zeros(1, dtype=torch.int32, device="cuda")
    S.slope_compress24(Ws, mask, vals, meta, invalid)
    Y = empty((T, N), torch.float32)
    S.slope_spmm_fwd(dev(X), vals, meta, N, Y)
    torch.cuda.synchronize()
    assert int(invalid.item()) == 0
    assert (host(vals) == vals_ref).all()
    assert (host(meta).view(np.uint32) == meta_ref).all()
    ref = oracle.spmm_fwd(X, vals_ref, meta_ref, K)
    err = normwise(host_f64(Y), ref)
    assert err <= 2e-5 * max(1.0, np.sqrt(K / 256)), err
    # the kept weights are exactly those of the dense masked product
    dense = oracle.widen(Ws_ref)
    assert normwise(host_f64(Y), oracle.widen(X) @ dense.T) <= TOL["f32"] * 10
