"""Pins of the oracle's 2:4 magnitude pruning against brute force and invariants.

The pages fix 2:4 (N:M) pruning of the weight along its rows for the forward pass
(summary page, Approach; explainer, Technical Summary 2.A).  The selection rule
itself (largest two magnitudes, ties to the lower index) is the reading the
oracle takes; these tests check the oracle's rank formulation against a second,
independent formulation that enumerates the six index pairs.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits


def _score(x: float):
    # NaN above every number, otherwise the magnitude.
    return (1, 0.0) if math.isnan(x) else (0, abs(x))


def pair_enumerator(group):
    """First index pair (lexicographic) whose kept scores all reach the dropped ones."""
    s = [_score(float(v)) for v in group]
    for a, b in itertools.combinations(range(4), 2):
        rest = [j for j in range(4) if j not in (a, b)]
        if min(s[a], s[b]) >= max(s[j] for j in rest):
            return (a, b)
    raise AssertionError("no valid pair")


def _all_groups(alphabet):
    return np.array(list(itertools.product(alphabet, repeat=4)))


def _bits(vals, dtype):
    f = np.asarray(vals, dtype=np.float32)
    if dtype == "f16":
        return f.astype(np.float16)
    return f32_to_bf16_bits(f) if dtype == "bf16" else f.view(np.uint32).copy()


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_exhaustive_small_alphabet_with_ties(dtype):
    # +0, -0 and +-1, +-2, +-3: 8^4 = 4096 groups, ties and signed zeros everywhere.
    alphabet = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0]
    groups = _all_groups(alphabet)
    bits = _bits(groups, dtype).reshape(-1, 4)
    mask, A_s = oracle.prune24(bits)
    for g in range(groups.shape[0]):
        a, b = pair_enumerator(groups[g])
        expect = np.zeros(4, dtype=np.uint8)
        expect[[a, b]] = 1
        assert (mask[g] == expect).all(), (groups[g], mask[g], (a, b))
        assert (A_s[g][expect == 1] == bits[g][expect == 1]).all()
        assert (A_s[g][expect == 0] == 0).all()


def test_exhaustive_special_values_f32():
    # denormals, infinities, NaN and the largest finite value
    tiny = np.float32(1e-45)          # smallest fp32 denormal
    alphabet = [0.0, tiny, -2 * tiny, np.inf, -np.inf, np.nan, 1.0, -np.float32(3.4e38)]
    groups = _all_groups(alphabet).astype(np.float32)
    bits = groups.view(np.uint32).reshape(-1, 4)
    mask, _ = oracle.prune24(bits)
    for g in range(groups.shape[0]):
        a, b = pair_enumerator(groups[g])
        assert set(np.flatnonzero(mask[g])) == {a, b}, groups[g]


def test_exhaustive_special_values_bf16():
    # bf16 denormal patterns 0x0001 and 0x8002, inf, NaN, 1, -max
    pats = [0x0000, 0x0001, 0x8002, 0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xFF7F]
    groups = _all_groups(pats).astype(np.uint16)
    mask, _ = oracle.prune24(groups)
    vals = oracle.widen(groups)
    for g in range(groups.shape[0]):
        a, b = pair_enumerator(vals[g])
        assert set(np.flatnonzero(mask[g])) == {a, b}


def test_exhaustive_special_values_f16():
    # fp16 subnormals 0x0001 and 0x8002, inf, -inf, NaN, 1, -max (65504)
    pats = [0x0000, 0x0001, 0x8002, 0x7C00, 0xFC00, 0x7E00, 0x3C00, 0xFBFF]
    groups = _all_groups(pats).astype(np.uint16).view(np.float16)
    mask, _ = oracle.prune24(groups)
    vals = oracle.widen(groups)
    assert vals[1, 3] == 2.0 ** -24 and np.isnan(vals[5 * 8 ** 3, 0]) and vals[7 * 8 ** 3, 0] == -65504.0
    for g in range(groups.shape[0]):
        a, b = pair_enumerator(vals[g])
        assert set(np.flatnonzero(mask[g])) == {a, b}


def test_nan_payloads_tie_and_go_to_lower_index():
    g = np.array([[0x7FC1, 0x7FFF, 0x7FC0, 0x3F80]], dtype=np.uint16)
    mask, _ = oracle.prune24(g)
    assert mask.tolist() == [[1, 1, 0, 0]]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_invariants_random(dtype):
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    bits = _bits(v, dtype)
    mask, A_s = oracle.prune24(bits)
    m = mask.reshape(64, 32, 4)
    assert (m.sum(-1) == 2).all()                       # exactly two kept per group
    mag = np.abs(oracle.widen(bits)).reshape(64, 32, 4)
    kept_min = np.where(m == 1, mag, np.inf).min(-1)
    drop_max = np.where(m == 0, mag, -np.inf).max(-1)
    assert (kept_min >= drop_max).all()                 # kept magnitudes dominate
    mask2, A_s2 = oracle.prune24(A_s)                    # idempotent on W_s
    assert (mask2 == mask).all() and (A_s2 == A_s).all()


def test_precision_independence():
    # bf16 values widened exactly to fp32 must give the same selection
    rng = np.random.default_rng(3)
    b = f32_to_bf16_bits((rng.standard_normal((32, 64)) * 0.02).astype(np.float32))
    as_f32 = (b.astype(np.uint32) << np.uint32(16))
    assert (oracle.prune24(b)[0] == oracle.prune24(as_f32)[0]).all()


def test_row_wise_groups_not_column_wise():
    # groups are 4 consecutive entries of a row: a column of large values must not
    # be kept as a whole.
    A = np.array([[9, 1, 2, 3, 0, 0, 0, 5],
                  [9, 4, 1, 1, 7, 6, 0, 0]], dtype=np.float32).view(np.uint32)
    mask, _ = oracle.prune24(A)
    assert mask.tolist() == [[1, 0, 0, 1, 1, 0, 0, 1],
                             [1, 1, 0, 0, 1, 1, 0, 0]]


def test_rejects_bad_width():
    with pytest.raises(ValueError):
        oracle.prune24(np.zeros((2, 6), dtype=np.uint16))
