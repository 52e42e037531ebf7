"""Pins of the oracle's products: forward, double-pruned dX, masked dW, adapter.

Definitions (explainer, Technical Summary 2.A and 2.B; discussion page,
"Memory Footprint" and "SLoPe downstream finetuning"):
Y = X . W_s^T, dX = dY . W_dp, dW = (dY^T . X) kept at the static mask,
Y += (X . L) . R with W_dense = W_sparse + L R.

Pins: brute-force triple loops on tiny inputs, identity inputs that expose the
orientation, gradients by finite differences of the forward map (linear, so the
difference quotient is exact up to rounding), integer-valued inputs whose
products are exact, and the dense-equivalent form of the adapter.
"""
import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits


def _bf16(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _layer(T, N, K, r, seed, ints=False):
    rng = np.random.default_rng(seed)
    if ints:
        mk = lambda *s: _bf16(rng.integers(-3, 4, size=s))
    else:
        mk = lambda *s: _bf16(rng.standard_normal(s))
    W, X, dY, L, R = mk(N, K), mk(T, K), mk(T, N), mk(K, r), mk(r, N)
    mask_s, W_s = oracle.prune24(W)
    values_s, meta_s, _ = oracle.compress24(W, mask_s)
    values_dpT, meta_dpT, mask_dpT = oracle.double_prune(values_s, meta_s, N, K)
    return dict(W=W, X=X, dY=dY, L=L, R=R, mask_s=mask_s, W_s=W_s, values_s=values_s,
                meta_s=meta_s, values_dpT=values_dpT, meta_dpT=meta_dpT, mask_dpT=mask_dpT)


def _loops_fwd(x, w_s):
    T, K = len(x), len(x[0])
    N = len(w_s)
    y = [[0.0] * N for _ in range(T)]
    for t in range(T):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(x[t][k]) * float(w_s[n][k])
            y[t][n] = s
    return np.array(y)


def test_forward_triple_loop():
    d = _layer(5, 8, 12, 0, 1)
    Y = oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], 12)
    ref = _loops_fwd(oracle.widen(d["X"]).tolist(), oracle.widen(d["W_s"]).tolist())
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_bwd_dx_triple_loop():
    T, N, K = 6, 12, 8
    d = _layer(T, N, K, 0, 2)
    dX = oracle.spmm_bwd_dx(d["dY"], d["values_dpT"], d["meta_dpT"], N)
    dy = oracle.widen(d["dY"])
    w_dpT = oracle.widen(oracle.decompress24(d["values_dpT"], d["meta_dpT"], N))  # [K, N]
    ref = np.zeros((T, K))
    for t in range(T):
        for k in range(K):
            ref[t, k] = sum(dy[t, n] * w_dpT[k, n] for n in range(N))
    assert np.allclose(dX, ref, rtol=1e-12, atol=1e-12)


def test_wgrad_triple_loop_and_mask():
    T, N, K = 7, 8, 16
    d = _layer(T, N, K, 0, 3)
    vals, dense = oracle.masked_wgrad(d["dY"], d["X"], d["meta_s"], K)
    dy, x = oracle.widen(d["dY"]), oracle.widen(d["X"])
    for n in range(N):
        for k in range(K):
            g = sum(dy[t, n] * x[t, k] for t in range(T))
            assert np.isclose(dense[n, k], g * d["mask_s"][n, k], rtol=1e-12, atol=1e-12)
    # compressed values sit in W_s's slots: decompressing them gives the dense form
    nz_dense = np.zeros((N, K))
    m = d["mask_s"].reshape(N, K // 4, 4)
    for n in range(N):
        for g in range(K // 4):
            idx = np.flatnonzero(m[n, g])
            nz_dense[n, 4 * g + idx] = vals[n, 2 * g:2 * g + 2]
    assert np.array_equal(nz_dense, dense)


def test_identity_inputs_pin_orientation():
    K = N = 16
    d = _layer(K, N, K, 0, 4)
    eye = _bf16(np.eye(K))
    # X = I  ->  Y = W_s^T
    Y = oracle.spmm_fwd(eye, d["values_s"], d["meta_s"], K)
    assert np.array_equal(Y, oracle.widen(d["W_s"]).T)
    # dY = I ->  dX = W_dp (the transpose of the stored W_dp^T)
    dX = oracle.spmm_bwd_dx(_bf16(np.eye(N)), d["values_dpT"], d["meta_dpT"], N)
    W_dpT = oracle.decompress24(d["values_dpT"], d["meta_dpT"], N)
    assert np.array_equal(dX, oracle.widen(W_dpT).T)
    # T = 1 -> dW is the masked outer product of the two rows
    vals, dense = oracle.masked_wgrad(d["dY"][:1], d["X"][:1], d["meta_s"], K)
    outer = np.multiply.outer(oracle.widen(d["dY"][0]), oracle.widen(d["X"][0]))
    assert np.array_equal(dense, outer * d["mask_s"])


def _loss(dy, x, w):
    # l(X, W) = sum(dY * (X . W^T)), computed by explicit sums
    return float((dy * np.einsum("tk,nk->tn", x, w)).sum())


def test_gradients_by_finite_differences():
    """dW and dX are the derivatives of sum(dY * Y) w.r.t. W_s and X.

    The map is linear in each argument, so a step of size 1 gives the exact
    derivative up to rounding.  dW is checked at kept positions (the static
    mask) and must be 0 elsewhere; dX uses the double-pruned weight.
    """
    T, N, K = 6, 8, 12
    d = _layer(T, N, K, 0, 5)
    dy, x = oracle.widen(d["dY"]), oracle.widen(d["X"])
    w_s = oracle.widen(d["W_s"])
    vals, dense = oracle.masked_wgrad(d["dY"], d["X"], d["meta_s"], K)
    base = _loss(dy, x, w_s)
    for n in range(N):
        for k in range(K):
            if d["mask_s"][n, k]:
                w2 = w_s.copy()
                w2[n, k] += 1.0
                assert np.isclose(_loss(dy, x, w2) - base, dense[n, k], rtol=1e-9, atol=1e-9)
            else:
                assert dense[n, k] == 0.0
    w_dp = oracle.widen(oracle.decompress24(d["values_dpT"], d["meta_dpT"], N)).T
    dX = oracle.spmm_bwd_dx(d["dY"], d["values_dpT"], d["meta_dpT"], N)
    base = _loss(dy, x, w_dp)
    for t in range(T):
        for k in range(K):
            x2 = x.copy()
            x2[t, k] += 1.0
            assert np.isclose(_loss(dy, x2, w_dp) - base, dX[t, k], rtol=1e-9, atol=1e-9)


def test_integer_inputs_are_exact():
    T, N, K = 9, 12, 40
    d = _layer(T, N, K, 4, 6, ints=True)
    Y = oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], K, d["L"], d["R"])
    assert np.array_equal(Y, np.round(Y))
    ref = _loops_fwd(oracle.widen(d["X"]).tolist(), oracle.widen(d["W_s"]).tolist())
    xl = oracle.widen(d["X"]) @ oracle.widen(d["L"])
    for t in range(T):
        for n in range(N):
            ref[t, n] += sum(xl[t, j] * oracle.widen(d["R"])[j, n] for j in range(4))
    assert np.array_equal(Y, ref)


def test_adapter_pins():
    T, N, K, r = 5, 8, 12, 3
    d = _layer(T, N, K, r, 7)
    Y0 = oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], K)
    # L = 0 leaves the forward unchanged, bit for bit
    zeroL = np.zeros_like(d["L"])
    assert np.array_equal(oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], K, zeroL, d["R"]), Y0)
    # rank 1: the adapter adds the outer product (X . l) r^T
    Y1 = oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], K, d["L"][:, :1], d["R"][:1])
    xl = oracle.widen(d["X"]) @ oracle.widen(d["L"][:, 0])
    assert np.allclose(Y1 - Y0, np.multiply.outer(xl, oracle.widen(d["R"][0])), rtol=1e-12, atol=1e-12)
    # W_dense = W_sparse + L R: the adapter equals a dense weight W_s + (L R)^T
    Y = oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], K, d["L"], d["R"])
    w_dense = oracle.widen(d["W_s"]) + (oracle.widen(d["L"]) @ oracle.widen(d["R"])).T
    assert np.allclose(Y, oracle.widen(d["X"]) @ w_dense.T, rtol=1e-12, atol=1e-12)
    # the standalone adapter call adds the same term to an existing output
    XL, Yadd = oracle.lowrank_add(d["X"], d["L"], d["R"], Y_in=np.zeros((T, N), np.uint16))
    assert np.allclose(Yadd, Y - Y0, rtol=1e-12, atol=1e-12)
    assert XL.shape == (T, r)


def test_wgrad_accumulate():
    T, N, K = 4, 8, 8
    d = _layer(T, N, K, 0, 8)
    vals, dense = oracle.masked_wgrad(d["dY"], d["X"], d["meta_s"], K)
    prev_v = _bf16(np.full((N, K // 2), 0.5))
    prev_d = _bf16(np.full((N, K), 0.25))
    v2, d2 = oracle.masked_wgrad(d["dY"], d["X"], d["meta_s"], K, prev_v, prev_d)
    assert np.array_equal(v2, vals + 0.5) and np.array_equal(d2, dense + 0.25)


@pytest.mark.parametrize("K", [4, 36])
def test_ragged_k(K):
    d = _layer(3, 4, K, 0, K)
    Y = oracle.spmm_fwd(d["X"], d["values_s"], d["meta_s"], K)
    assert np.allclose(Y, oracle.widen(d["X"]) @ oracle.widen(d["W_s"]).T)
