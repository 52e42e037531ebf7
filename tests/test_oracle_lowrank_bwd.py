"""Pins of the oracle's adapter backward (dX term, dL, dR).

The adapter term Y += (X . L) . R (explainer, Technical Summary 2.B: W_dense =
W_sparse + L R) is linear in each of X, L and R, so its gradients are pinned
against the oracle's own forward adapter (lowrank_add, pinned elsewhere) by
finite differences: for integer-valued inputs a unit step changes
sum(dY * Y) by exactly the derivative.  Special cases (a zero factor) and
identity inputs that expose the orientation of each output complete the pins.
"""
import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits


def _ints(rng, *shape, dt="f32"):
    a = rng.integers(-3, 4, size=shape).astype(np.float32)
    return f32_to_bf16_bits(a) if dt == "bf16" else a.view(np.uint32)


def _bump(bits, idx):
    """Bits of the same array with element idx increased by exactly 1."""
    if bits.dtype == np.uint32:
        v = bits.view(np.float32).copy()
        v[idx] += 1.0
        return v.view(np.uint32)
    v = oracle.widen(bits).astype(np.float32)
    v[idx] += 1.0
    return f32_to_bf16_bits(v)


def _loss(X, L, R, dY):
    _, Y = oracle.lowrank_add(X, L, R)
    return float((oracle.widen(dY) * Y).sum())


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gradients_by_finite_differences(dt):
    T, K, r, N = 5, 7, 3, 6
    rng = np.random.default_rng(3)
    X, L, R, dY = _ints(rng, T, K, dt=dt), _ints(rng, K, r, dt=dt), _ints(rng, r, N, dt=dt), _ints(rng, T, N, dt=dt)
    dX, dL, dR = oracle.lowrank_bwd(X, dY, L, R)
    assert dX.shape == (T, K) and dL.shape == (K, r) and dR.shape == (r, N)
    base = _loss(X, L, R, dY)
    for t in range(T):
        for k in range(K):
            assert _loss(_bump(X, (t, k)), L, R, dY) - base == dX[t, k]
    for k in range(K):
        for j in range(r):
            assert _loss(X, _bump(L, (k, j)), R, dY) - base == dL[k, j]
    for j in range(r):
        for n in range(N):
            assert _loss(X, L, _bump(R, (j, n)), dY) - base == dR[j, n]


def test_zero_factors():
    T, K, r, N = 4, 8, 2, 5
    rng = np.random.default_rng(4)
    X, L, R, dY = _ints(rng, T, K), _ints(rng, K, r), _ints(rng, r, N), _ints(rng, T, N)
    zL, zR = np.zeros_like(L), np.zeros_like(R)
    dX, dL, dR = oracle.lowrank_bwd(X, dY, L, zR)
    assert not dX.any() and not dL.any() and dR.any()       # R = 0: nothing flows back through R
    dX, dL, dR = oracle.lowrank_bwd(X, dY, zL, R)
    assert not dX.any() and dL.any() and not dR.any()       # L = 0: X . L = 0


def test_identity_inputs_pin_orientation():
    # X = I (T = K) and L = I (K = r): dR = (X L)^T dY = dY
    n = 4
    rng = np.random.default_rng(5)
    eye = np.eye(n, dtype=np.float32).view(np.uint32)
    R, dY = _ints(rng, n, 6), _ints(rng, n, 6)
    _, dL, dR = oracle.lowrank_bwd(eye, dY, eye, R)
    assert np.array_equal(dR, oracle.widen(dY))
    # with R = I as well (r = N): dL = X^T dY R^T = dY, and the dX term is dY L^T = dY
    dYs = _ints(rng, n, n)
    dX, dL, _ = oracle.lowrank_bwd(eye, dYs, eye, eye)
    assert np.array_equal(dL, oracle.widen(dYs))
    assert np.array_equal(dX, oracle.widen(dYs))
