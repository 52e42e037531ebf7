"""Pins of the oracle's general N:M magnitude pruning.

The explainer (Technical Summary 1, Problem Statement) introduces N:M
structured sparsity in general; the method itself fixes 2:4.  The oracle keeps
the n highest-ranked of every m consecutive elements (magnitude, NaN above
every number, ties to the lower index).  Its rank-count formulation is checked
against two independent ones: a subset enumerator (small m) and a stable sort
(large m); the 2:4 case must agree with prune24, which is pinned exhaustively.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits


def _score(x: float):
    return (1, 0.0) if math.isnan(x) else (0, abs(x))


def subset_enumerator(group, n):
    """First index subset (lexicographic) of size n whose kept scores all reach the dropped ones."""
    m = len(group)
    s = [_score(float(v)) for v in group]
    for sub in itertools.combinations(range(m), n):
        rest = [j for j in range(m) if j not in sub]
        if not rest or min(s[a] for a in sub) >= max(s[j] for j in rest):
            return sub
    raise AssertionError("no valid subset")


def sort_select(group, n):
    """The n first positions of a stable sort by descending score."""
    s = [_score(float(v)) for v in group]
    order = sorted(range(len(group)), key=lambda j: (-s[j][0], -s[j][1], j))
    return tuple(sorted(order[:n]))


def _bits(vals, dtype):
    f = np.asarray(vals, dtype=np.float32)
    if dtype == "f16":
        return f.astype(np.float16)
    return f32_to_bf16_bits(f) if dtype == "bf16" else f.view(np.uint32).copy()


ALPHABET = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, float("inf"), float("nan")]


@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (1, 8), (2, 8), (4, 8), (7, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_against_subset_enumerator(n, m, dtype):
    rng = np.random.default_rng(100 * n + m)
    groups = rng.choice(np.array(ALPHABET), size=(1500, m))
    bits = _bits(groups, dtype)
    mask, A_s = oracle.prune_nm(bits, n, m)
    for g in range(groups.shape[0]):
        expect = np.zeros(m, dtype=np.uint8)
        expect[list(subset_enumerator(groups[g], n))] = 1
        assert (mask[g] == expect).all(), (groups[g], mask[g], expect)
        assert (A_s[g][expect == 1].view(np.uint8) == bits[g][expect == 1].view(np.uint8)).all()
        assert (A_s[g][expect == 0].view(np.uint8) == 0).all()


@pytest.mark.parametrize("n,m", [(5, 16), (8, 16), (2, 32), (16, 32)])
def test_large_groups_against_stable_sort(n, m):
    rng = np.random.default_rng(7 * n + m)
    groups = rng.choice(np.array(ALPHABET), size=(300, m))
    mask, _ = oracle.prune_nm(_bits(groups, "f32"), n, m)
    for g in range(groups.shape[0]):
        expect = np.zeros(m, dtype=np.uint8)
        expect[list(sort_select(groups[g], n))] = 1
        assert (mask[g] == expect).all(), (groups[g], mask[g], expect)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_two_of_four_is_prune24(dtype):
    rng = np.random.default_rng(3)
    vals = rng.choice(np.array([0.0, -0.0, 0.5, -0.5, 1.5, -2.0, 3.0]), size=(64, 96))
    vals[::7] = rng.standard_normal((10, 96))
    bits = _bits(vals, dtype)
    m24, s24 = oracle.prune24(bits)
    mnm, snm = oracle.prune_nm(bits, 2, 4)
    assert (m24 == mnm).all()
    assert (s24.view(np.uint8) == snm.view(np.uint8)).all()


@pytest.mark.parametrize("n,m", [(1, 4), (2, 8), (3, 8), (4, 16), (7, 32)])
def test_invariants(n, m):
    rng = np.random.default_rng(n * m)
    A = f32_to_bf16_bits(rng.standard_normal((48, 4 * m)).astype(np.float32))
    mask, A_s = oracle.prune_nm(A, n, m)
    g = mask.reshape(48, -1, m)
    assert (g.sum(-1) == n).all()                               # exactly n kept per group
    mag = np.abs(oracle.widen(A)).reshape(48, -1, m)
    kept_min = np.where(g == 1, mag, np.inf).min(-1)
    dropped_max = np.where(g == 0, mag, -np.inf).max(-1)
    assert (kept_min >= dropped_max).all()                      # every kept magnitude reaches every dropped one
    mask2, A_s2 = oracle.prune_nm(A_s, n, m)                    # idempotent (no zeros in A)
    assert (mask2 == mask).all() and (A_s2 == A_s).all()
    assert mask.sum() == A.size * n // m


def test_keep_all_is_identity():
    A = f32_to_bf16_bits(np.random.default_rng(1).standard_normal((8, 32)).astype(np.float32))
    mask, A_s = oracle.prune_nm(A, 8, 8)
    assert (mask == 1).all() and (A_s == A).all()


@pytest.mark.parametrize("n,m", [(1, 4), (1, 8), (2, 8), (2, 16), (2, 32)])
def test_at_most_two_per_aligned_four_runs_on_24_format(n, m):
    """n <= 2 with m a multiple of 4 keeps at most two of every aligned four, so the
    2:4 compressed format holds the pruned weight exactly."""
    rng = np.random.default_rng(11 + n + m)
    A = f32_to_bf16_bits(rng.standard_normal((32, 2 * m)).astype(np.float32))
    mask, A_s = oracle.prune_nm(A, n, m)
    assert (mask.reshape(32, -1, 4).sum(-1) <= 2).all()
    values, meta, invalid = oracle.compress24(A_s, mask)
    assert invalid == 0
    assert (oracle.decompress24(values, meta, A.shape[1]) == A_s).all()


def test_rejects_bad_arguments():
    A = np.zeros((2, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.prune_nm(A, 0, 4)
    with pytest.raises(ValueError):
        oracle.prune_nm(A, 5, 4)
    with pytest.raises(ValueError):
        oracle.prune_nm(np.zeros((2, 12), dtype=np.uint16), 2, 8)
