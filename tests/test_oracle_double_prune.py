"""Pins of the oracle's double pruning (the backward weight W^{R,C}).

Explainer, Technical Summary 2.A and Key Contributions: the already 2:4-sparse
weight is transposed and pruned 2:4 again along its new rows.  Pins: the N:M
invariants in both orientations, the subset relation, the identity on weights
whose columns already satisfy 2:4, a brute-force column enumerator on small
inputs, and the kept density of i.i.d. weights (a closed form derived below).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits


def _setup(N, K, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W = f32_to_bf16_bits(v) if dtype == "bf16" else v.view(np.uint32).copy()
    mask_s, W_s = oracle.prune24(W)
    values_s, meta_s, _ = oracle.compress24(W, mask_s)
    return W, mask_s, W_s, values_s, meta_s


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,K", [(8, 8), (64, 32), (36, 100), (128, 256)])
def test_invariants(N, K, dtype):
    W, mask_s, W_s, values_s, meta_s = _setup(N, K, N * K, dtype)
    values_dpT, meta_dpT, mask_dpT = oracle.double_prune(values_s, meta_s, N, K)
    assert values_dpT.shape == (K, N // 2) and meta_dpT.shape == (K, -(-N // 32))
    W_dpT = oracle.decompress24(values_dpT, meta_dpT, N)
    # at most two non-zeros in every group of both orientations
    assert ((oracle.widen(W_s).reshape(N, K // 4, 4) != 0).sum(-1) <= 2).all()
    assert ((oracle.widen(W_dpT).reshape(K, N // 4, 4) != 0).sum(-1) <= 2).all()
    # every kept group has exactly two slots, and the mask matches the metadata
    assert (mask_dpT.reshape(K, N // 4, 4).sum(-1) == 2).all()
    assert (oracle.mask_from_meta(meta_dpT, N) == mask_dpT).all()
    # nz(W_dp) is a subset of nz(W_s), with identical values there
    W_dp = W_dpT.T
    nz = oracle.widen(W_dp) != 0
    assert (oracle.widen(W_s)[nz] != 0).all()
    assert (W_dp[nz] == W_s[nz]).all()
    # the values it keeps are the bits of W_s^T at the kept positions
    assert (W_dpT[mask_dpT == 1] == W_s.T[mask_dpT == 1]).all()


def _col_enumerator(col4):
    s = [(1, 0.0) if math.isnan(x) else (0, abs(x)) for x in col4]
    for a, b in itertools.combinations(range(4), 2):
        rest = [j for j in range(4) if j not in (a, b)]
        if min(s[a], s[b]) >= max(s[j] for j in rest):
            return {a, b}


def test_brute_force_columns():
    W, mask_s, W_s, values_s, meta_s = _setup(16, 24, 11)
    _, _, mask_dpT = oracle.double_prune(values_s, meta_s, 16, 24)
    ws = oracle.widen(W_s)
    for k in range(24):
        for g in range(4):
            kept = set(np.flatnonzero(mask_dpT[k, 4 * g:4 * g + 4]).tolist())
            assert kept == _col_enumerator(ws[4 * g:4 * g + 4, k]), (k, g)


def test_identity_when_columns_already_2_4():
    # a banded pattern with two non-zeros in every row group and every column group
    N = K = 16
    rng = np.random.default_rng(5)
    dense = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        for g in range(K // 4):
            for j in ((n % 4), (n + 1) % 4):
                dense[n, 4 * g + j] = rng.uniform(0.5, 1.5)
    W = f32_to_bf16_bits(dense)
    mask_s, W_s = oracle.prune24(W)
    assert (W_s == W).all()
    values_s, meta_s, _ = oracle.compress24(W, mask_s)
    values_dpT, meta_dpT, _ = oracle.double_prune(values_s, meta_s, N, K)
    assert (oracle.decompress24(values_dpT, meta_dpT, N).T == W_s).all()


def test_density_closed_form():
    """Density of W_dp for i.i.d. continuous W.

    Each row group of W_s keeps 2 of 4, so an entry of W_s is non-zero with
    probability 1/2, independently across rows; a column group therefore holds
    k ~ Binomial(4, 1/2) non-zeros and keeps min(k, 2):
    E[min(k,2)] = (0*1 + 1*4 + 2*6 + 2*4 + 2*1) / 16 = 26/16, so the density of
    W_dp is 26/64 = 13/32 = 0.40625 and 31.25% of column groups lose one or more.
    """
    N = K = 256
    W, mask_s, W_s, values_s, meta_s = _setup(N, K, 0)
    values_dpT, meta_dpT, _ = oracle.double_prune(values_s, meta_s, N, K)
    W_dpT = oracle.widen(oracle.decompress24(values_dpT, meta_dpT, N))
    density = (W_dpT != 0).mean()
    assert abs(density - 13 / 32) < 0.01
    col_nz = (oracle.widen(W_s).T.reshape(K, N // 4, 4) != 0).sum(-1)
    assert abs((col_nz > 2).mean() - 5 / 16) < 0.02


def test_is_deterministic_and_tracks_the_current_weight():
    W, mask_s, W_s, values_s, meta_s = _setup(32, 32, 9)
    a = oracle.double_prune(values_s, meta_s, 32, 32)
    b = oracle.double_prune(values_s.copy(), meta_s.copy(), 32, 32)
    assert all((x == y).all() for x, y in zip(a, b))
    # change the values under the same static mask: the column mask may move
    values2 = values_s.copy()
    values2[:, 0::2], values2[:, 1::2] = values_s[:, 1::2], values_s[:, 0::2]
    c = oracle.double_prune(values2, meta_s, 32, 32)
    assert not (c[2] == a[2]).all()
