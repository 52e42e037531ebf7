"""Pins of the oracle's optimizer step on compressed values.

The discussion page trains SLoPe with AdamW ("Choice of Optimizer") and keeps
two 32-bit moments for the two non-zeros of each group of four ("Memory
Footprint Reduction During Pretraining and Inference").  The float64 step is
pinned against PyTorch's AdamW on CPU (an independent library implementation
of the same published method) and against closed forms; the rounding to the
stored formats against a brute-force nearest-value search; the composition
with the double prune against a case where the update reorders magnitudes.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import f32_to_bf16_bits

HP_SETS = [
    dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(lr=3e-2, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0),
    dict(lr=5e-4, beta1=0.0, beta2=0.5, eps=1e-3, weight_decay=0.3),
]


def _bf16_neighbours(b):
    """The bf16 patterns one step below and above b in value (finite b)."""
    b = b.astype(np.int32)
    mag, neg = b & 0x7FFF, (b & 0x8000) != 0
    up = np.where(neg, b - 1, b + 1)                 # one step away from zero (same sign)
    down = np.where(mag == 0, (b ^ 0x8000) + 1, np.where(neg, b + 1, b - 1))   # toward zero / across it
    return down.astype(np.uint16), up.astype(np.uint16)


def test_round_bf16_is_nearest_ties_to_even():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.normal(size=20000),
        rng.normal(size=4000) * 2.0 ** rng.integers(-140, -120, size=4000),   # bf16 subnormal range
        rng.normal(size=4000) * 2.0 ** rng.integers(100, 127, size=4000),
        # exact midpoints between neighbouring bf16 values
        (rng.integers(-2 ** 15, 2 ** 15, size=4000) * 2 + 1) * 2.0 ** rng.integers(-20, 20, size=4000) * 2.0 ** -9,
    ])
    b = oracle.round_bf16(x)
    got = oracle.widen(b)
    assert np.isfinite(got).all()
    down, up = _bf16_neighbours(b)
    err = np.abs(x - got)
    for nb in (down, up):
        alt = oracle.widen(nb)
        ok = np.isfinite(alt)
        d = np.abs(x - alt)
        assert (err[ok] <= d[ok]).all()                          # no neighbour is nearer
        tie = ok & (err == d) & (err > 0)
        assert ((b[tie] & 1) == 0).all()                          # ties go to the even pattern


def test_round_f16_is_nearest_ties_to_even():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.normal(size=20000) * 100,
                        rng.normal(size=4000) * 2.0 ** rng.integers(-30, -14, size=4000),   # subnormal range
                        # exact midpoints between neighbouring fp16 values
                        (rng.integers(-2 ** 10, 2 ** 10, size=4000) * 2 + 1) * 2.0 ** rng.integers(-20, 4, size=4000)
                        * 2.0 ** -11])
    h = oracle.round_f16(x)
    assert h.dtype == np.float16 and np.isfinite(h).all()
    b = h.view(np.uint16).astype(np.int32)
    for step in (-1, 1):                                   # neighbours by bit pattern (same sign)
        nb = b + step
        ok = ((nb & 0x7FFF) < 0x7C00) & (nb >= 0) & ((nb & 0x7FFF) != 0x7FFF)
        alt = nb[ok].astype(np.uint16).view(np.float16).astype(np.float64)
        err, d = np.abs(x[ok] - h[ok].astype(np.float64)), np.abs(x[ok] - alt)
        assert (err <= d).all()
        tie = (err == d) & (err > 0)
        assert ((b[ok][tie] & 1) == 0).all()
    zero_cross = (b & 0x7FFF) == 0                          # nearest across zero: the other sign's smallest
    assert (np.abs(x[zero_cross]) <= 2.0 ** -25).all()


def _f32_neighbours(f):
    """The fp32 values one representable step below and above each finite f."""
    f = np.asarray(f, dtype=np.float32)
    with np.errstate(over="ignore"):
        return np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))


def test_round_f32_is_nearest_ties_to_even():
    # Brute force: no fp32 value adjacent to the result is nearer to the float64 input, and
    # exact midpoints go to the pattern with an even last bit.  The inputs span normal
    # binades, the subnormal range (quantum 2^-149), values near the overflow threshold,
    # and exact midpoints built from neighbouring fp32 pairs (exact in float64).
    rng = np.random.default_rng(19)
    a = (rng.normal(size=4000) * 2.0 ** rng.integers(-120, 120, size=4000)).astype(np.float32)
    a = a[np.isfinite(a) & (a != 0)]
    lo, hi = _f32_neighbours(a)
    mid = (a.astype(np.float64) + hi.astype(np.float64)) / 2           # exact halfway points
    sub = (rng.integers(-2 ** 23, 2 ** 23, size=3000) * 2 + 1) * 2.0 ** -150  # halfway between subnormals
    x = np.concatenate([
        rng.normal(size=20000),
        rng.normal(size=4000) * 2.0 ** rng.integers(-160, -126, size=4000),   # fp32 subnormal range
        rng.normal(size=4000) * 2.0 ** rng.integers(100, 127, size=4000),
        rng.uniform(-1, 1, size=4000) * 2.0 ** -149 * 3,                      # a few quanta around zero
        mid, sub,
    ])
    r = oracle.round_f32(x)
    assert r.dtype == np.float32 and np.isfinite(r).all()
    got = r.astype(np.float64)
    err = np.abs(x - got)
    down, up = _f32_neighbours(r)
    for nb in (down, up):
        alt = nb.astype(np.float64)
        ok = np.isfinite(alt)
        d = np.abs(x - alt)
        assert (err[ok] <= d[ok]).all()                           # no neighbour is nearer
        tie = ok & (err == d) & (err > 0)
        assert ((r[tie].view(np.uint32) & 1) == 0).all()          # ties go to the even pattern
    # the constructed midpoints are ties, and a truncating rounding would fail them
    nm = len(mid)
    at_mid = r[20000 + 4000 * 3: 20000 + 4000 * 3 + nm]
    assert ((at_mid == a) | (at_mid == hi)).all()
    assert (at_mid.view(np.uint32) & 1 == 0).all()
    assert (at_mid != np.where(np.abs(a) < np.abs(hi), a, hi)).any()   # not always toward zero
    # a value just past a midpoint goes up, just short of it goes down
    above = oracle.round_f32(np.nextafter(mid, np.inf * np.sign(mid)))
    assert np.array_equal(above, np.where(np.abs(hi) > np.abs(a), hi, a))


def test_round_f32_exact_values_and_specials():
    rng = np.random.default_rng(20)
    pats = np.concatenate([rng.integers(0, 2 ** 32, size=50000, dtype=np.uint64).astype(np.uint32),
                           np.arange(0, 4096, dtype=np.uint32)])                 # subnormals and zero
    vals = pats.view(np.float32)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.round_f32(vals[fin].astype(np.float64)).view(np.uint32), pats[fin])
    big = (2 - 2 ** -24) * 2.0 ** 127                                 # midpoint above the largest finite fp32
    assert oracle.round_f32(np.array([big]))[0] == np.inf
    assert oracle.round_f32(np.array([np.nextafter(big, 0)]))[0] == np.float32(3.4028234663852886e38)
    assert oracle.round_f32(np.array([2.0 ** -150]))[0] == 0.0        # halfway to the smallest subnormal: even (0)
    assert oracle.round_f32(np.array([3 * 2.0 ** -150]))[0] == np.float32(2.0 ** -148)   # 1.5 quanta -> 2
    assert np.isnan(oracle.round_f32(np.array([np.nan]))).all()


def test_round_bf16_exact_values_and_specials():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.widen(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.round_bf16(vals[fin]), bits[fin])     # representable values are kept
    assert np.array_equal(oracle.round_bf16(np.array([np.inf, -np.inf])), np.array([0x7F80, 0xFF80], np.uint16))
    assert np.isnan(oracle.widen(oracle.round_bf16(np.array([np.nan])))).all()
    big = (2 - 2 ** -8) * 2.0 ** 127                                    # midpoint above the largest finite
    assert oracle.round_bf16(np.array([big]))[0] == 0x7F80
    assert oracle.round_bf16(np.array([np.nextafter(big, 0)]))[0] == 0x7F7F


@pytest.mark.parametrize("hp", HP_SETS)
def test_adamw_update_matches_torch_adamw(hp):
    rng = np.random.default_rng(12)
    p0 = rng.normal(size=(7, 9)) * 0.05
    grads = [rng.normal(size=(7, 9)) * s for s in (1.0, 0.3, 2.0, 0.01, 1.0, 0.5)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for step, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_update(p, g, m, v, step, **hp)
        st = opt.state[tp]
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-300)


def test_adamw_first_step_closed_form():
    # from zero moments the bias-corrected moments are g and g^2 exactly
    rng = np.random.default_rng(13)
    p, g = rng.normal(size=50), rng.normal(size=50)
    lr, wd, eps = 0.01, 0.1, 1e-4
    z = np.zeros(50)
    p1, m1, v1 = oracle.adamw_update(p, g, z, z, 1, lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=wd)
    np.testing.assert_allclose(p1, p - lr * wd * p - lr * g / (np.abs(g) + eps), rtol=1e-14)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-12)
    # no gradient and no history: only the decoupled decay acts
    p2, _, _ = oracle.adamw_update(p, z, z, z, 5, lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=wd)
    np.testing.assert_allclose(p2, p * (1 - lr * wd), rtol=1e-15)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_adamw_compressed_sign_descent_is_exact(dt):
    # beta1 = beta2 = 0, eps = 0, no decay: the step is p - lr * sign(g), m = g, v = g^2, all exact
    rng = np.random.default_rng(14)
    pv = rng.integers(-40, 41, size=(6, 8)).astype(np.float32) / 16
    gv = rng.integers(1, 9, size=(6, 8)).astype(np.float32) * rng.choice([-1.0, 1.0], size=(6, 8)).astype(np.float32)
    enc = {"bf16": f32_to_bf16_bits, "f16": lambda a: a.astype(np.float16), "f32": lambda a: a.view(np.uint32)}[dt]
    m0 = rng.normal(size=(6, 8)).astype(np.float32)                   # ignored when beta1 = 0
    v0 = np.abs(rng.normal(size=(6, 8))).astype(np.float32)
    vals, m1, v1 = oracle.adamw_compressed(enc(pv), enc(gv), m0, v0, 3, lr=0.25, beta1=0.0, beta2=0.0, eps=0.0,
                                           weight_decay=0.0)
    assert vals.dtype == {"bf16": np.uint16, "f16": np.float16, "f32": np.uint32}[dt]
    assert np.array_equal(oracle.widen(vals), pv - 0.25 * np.sign(gv))
    assert m1.dtype == np.float32 and np.array_equal(m1, gv)
    assert v1.dtype == np.float32 and np.array_equal(v1, gv * gv)


def test_adamw_compressed_rounds_once_to_storage():
    rng = np.random.default_rng(15)
    p = f32_to_bf16_bits((rng.normal(size=(16, 32)) * 0.02).astype(np.float32))
    g = f32_to_bf16_bits(rng.normal(size=(16, 32)).astype(np.float32))
    m = (rng.normal(size=(16, 32)) * 0.1).astype(np.float32)
    v = (np.abs(rng.normal(size=(16, 32))) * 0.01).astype(np.float32)
    hp = HP_SETS[0]
    vals, m1, v1 = oracle.adamw_compressed(p, g, m, v, 7, **hp)
    pe, me, ve = oracle.adamw_update(oracle.widen(p), oracle.widen(g), m, v, 7, **hp)
    # each stored value is one of the two representable neighbours of the exact result, the nearer one
    got = oracle.widen(vals)
    down, up = _bf16_neighbours(vals)
    assert (np.abs(got - pe) <= np.abs(oracle.widen(down) - pe)).all()
    assert (np.abs(got - pe) <= np.abs(oracle.widen(up) - pe)).all()
    assert np.array_equal(m1, me.astype(np.float32)) and np.array_equal(v1, ve.astype(np.float32))
    # the update moved the weights (a dropped term would leave them)
    assert (vals != p).mean() > 0.5


def test_adamw_double_prune_follows_updated_weights():
    # W_s rows [a, b] at columns {0, 1} of one group: two rows n = 0..3 in one column group.
    # Before the update column 0's magnitudes rank rows 0, 1 highest; the step pushes rows 2, 3 up.
    N, K = 4, 4
    dense = np.zeros((N, K), np.float32)
    dense[:, 0] = [4.0, 3.0, 1.0, 0.5]
    dense[:, 1] = [1.0, 1.0, 1.0, 1.0]
    vals_f = dense.view(np.uint32)
    mask, _ = oracle.prune24(vals_f)
    values_s, meta_s, _ = oracle.compress24(vals_f, mask)
    grad_dense = np.zeros((N, K), np.float32)
    grad_dense[:, 0] = [1.0, 1.0, -1.0, -1.0]                         # sign descent: rows 2, 3 grow
    grad_dense[:, 1] = [-1.0, -1.0, -1.0, -1.0]                       # (eps = 0 needs g != 0)
    grad_vals, _, _ = oracle.compress24(grad_dense.view(np.uint32), mask)
    z = np.zeros(values_s.shape, np.float32)
    before = oracle.double_prune(values_s, meta_s, N, K)[2]
    out = oracle.adamw_double_prune(values_s, meta_s, grad_vals, z, z, N, K, 1, lr=3.0, beta1=0.0, beta2=0.0,
                                    eps=0.0, weight_decay=0.0)
    vals1, mask_dpT = out[0], out[5]
    w1 = oracle.widen(oracle.decompress24(vals1, meta_s, K))
    assert np.array_equal(w1[:, 0], [1.0, 0.0, 4.0, 3.5]) and np.array_equal(w1[:, 1], [4.0] * 4)
    assert list(before[0]) == [1, 1, 0, 0] and list(mask_dpT[0]) == [0, 0, 1, 1]
    assert all(np.array_equal(a, b) for a, b in zip(out[3:], oracle.double_prune(vals1, meta_s, N, K)))
