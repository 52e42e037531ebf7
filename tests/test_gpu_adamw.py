"""GPU parity of the optimizer step on compressed 2:4 values and of the fused
update + double prune, against the oracle.

The kernels compute AdamW in fp32; the oracle in float64 with one rounding to
the stored format.  The elementwise bound used here follows from the kernel's
operations: every stored value is within one spacing of its format (both
sides round the same real number, from either side of a rounding point) plus
the fp32 error of the step, at most a few units of 2^-24 relative in each of
the decayed weight, the moments' two terms and the update; the moments
likewise.  Decisions taken on stored bits (the double prune of the updated
weight) must match bit for bit: the oracle double-prunes the values the GPU
stored.  The fused entry point must equal the two separate calls bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import f32_to_bf16_bits

from gpu_util import Compressed, check_adamw_update as _check_update, dev, dev_meta, host, say

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()


def _inputs(rng, n, dt, gdt, scale_p=0.02):
    p = (rng.standard_normal(n) * scale_p).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    m = (rng.standard_normal(n) * 0.05).astype(np.float32)
    v = (np.abs(rng.standard_normal(n)) * 0.01).astype(np.float32)
    enc = {"bf16": f32_to_bf16_bits, "f32": lambda a: a.view(np.uint32).copy()}
    return enc[dt](p), enc[gdt](g), m, v


_dev_vals, _host_vals = dev, host


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


@pytest.mark.parametrize("dt,gdt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("n", [1, 7, 8, 1000, 4099, 9_000_003])
def test_adamw_elementwise(n, dt, gdt):
    say(f"[adamw] n={n} {dt}/{gdt}")
    rng = np.random.default_rng(n)
    p0, g, m0, v0 = _inputs(rng, n, dt, gdt)
    p, gd, m, v = _dev_vals(p0), _dev_vals(g), _dev_f32(m0), _dev_f32(v0)
    S.slope_adamw(p, gd, m, v, 5, **HP)
    torch.cuda.synchronize()
    _check_update(p0, g, m0, v0, 5, HP, _host_vals(p), m.cpu().numpy(), v.cpu().numpy())
    assert np.array_equal(host(gd), g)                                  # the gradient is not touched


def test_adamw_successive_steps_and_closed_forms():
    rng = np.random.default_rng(3)
    n = 5000
    p0, g, _, _ = _inputs(rng, n, "bf16", "bf16")
    m0, v0 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    p, m, v = _dev_vals(p0), _dev_f32(m0), _dev_f32(v0)
    for step in (1, 2, 3):
        g = f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
        pb, mb, vb = _host_vals(p), m.cpu().numpy(), v.cpu().numpy()
        S.slope_adamw(p, _dev_vals(g), m, v, step, **HP)
        torch.cuda.synchronize()
        _check_update(pb, g, mb, vb, step, HP, _host_vals(p), m.cpu().numpy(), v.cpu().numpy())
    # no gradient, no history: the decoupled decay alone, p (1 - lr wd)
    p0 = np.linspace(-1, 1, 64, dtype=np.float32)
    z = np.zeros(64, np.float32)
    p = _dev_f32(p0)
    S.slope_adamw(p, _dev_f32(z), _dev_f32(z), _dev_f32(z), 4, lr=0.5, weight_decay=0.25)
    want = (p0.astype(np.float64) * (1 - 0.125)).astype(np.float32)
    assert np.array_equal(p.cpu().numpy(), want)
    # sign descent (beta1 = beta2 = 0, eps = 0): p - lr sign(g), exact
    g = np.where(np.arange(64) % 2 == 0, 3.0, -0.5).astype(np.float32)
    p, m, v = _dev_f32(p0), _dev_f32(z), _dev_f32(z)
    S.slope_adamw(p, _dev_f32(g), m, v, 9, lr=0.25, beta1=0.0, beta2=0.0, eps=0.0, weight_decay=0.0)
    assert np.array_equal(p.cpu().numpy(), p0 - 0.25 * np.sign(g))
    assert np.array_equal(m.cpu().numpy(), g) and np.array_equal(v.cpu().numpy(), g * g)


def _compressed(rng, N, K, dt):
    W = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    Wb = f32_to_bf16_bits(W) if dt == "bf16" else W.view(np.uint32).copy()
    mask, _ = oracle.prune24(Wb)
    vals, meta, _ = oracle.compress24(Wb, mask)
    return vals, meta


FUSED = [(256, 256, "bf16", "bf16"), (272, 528, "bf16", "bf16"), (1024, 1024, "bf16", "f32"),
         (16, 2064, "bf16", "bf16"), (100, 68, "bf16", "bf16"), (36, 8, "bf16", "f32"), (64, 256, "f32", "f32"),
         (20, 44, "f32", "bf16")]


@pytest.mark.parametrize("N,K,dt,gdt", FUSED)
def test_adamw_double_prune(N, K, dt, gdt):
    say(f"[adamw_double_prune] N={N} K={K} {dt}/{gdt}")
    rng = np.random.default_rng(N * 7 + K)
    vals0, meta = _compressed(rng, N, K, dt)
    _, g, m0, v0 = _inputs(rng, vals0.size, dt, gdt)
    g, m0, v0 = g.reshape(N, K // 2), m0.reshape(N, K // 2), v0.reshape(N, K // 2)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    vs, ms, m, v = _dev_vals(vals0), dev_meta(meta), _dev_f32(m0), _dev_f32(v0)
    dp = Compressed(K, N, tdt)
    mask_dp = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    hp = dict(HP, lr=0.02)                    # large enough to reorder magnitudes in many column groups
    S.slope_adamw_double_prune(vs, ms, _dev_vals(g), m, v, N, K, dp.values, dp.meta, 6, mask_dpT=mask_dp, **hp)
    torch.cuda.synchronize()
    new_vals = _host_vals(vs)
    _check_update(vals0, g, m0, v0, 6, hp, new_vals, m.cpu().numpy(), v.cpu().numpy())
    assert np.array_equal(host(ms), meta)                               # the static mask does not move
    vdp_ref, mdp_ref, mask_ref = oracle.double_prune(new_vals, meta, N, K)
    assert np.array_equal(host(dp.values), vdp_ref)
    assert np.array_equal(host(dp.meta), mdp_ref)
    assert np.array_equal(host(mask_dp), mask_ref)
    # the update changed the double-pruned mask somewhere (it follows the current weights)
    assert not np.array_equal(mask_ref, oracle.double_prune(vals0, meta, N, K)[2])
    # the fused call equals the two separate calls, bit for bit
    vs2, m2, v2 = _dev_vals(vals0), _dev_f32(m0), _dev_f32(v0)
    dp2 = Compressed(K, N, tdt)
    S.slope_adamw(vs2, _dev_vals(g), m2, v2, 6, **hp)
    S.slope_double_prune(vs2, ms, N, K, dp2.values, dp2.meta)
    torch.cuda.synchronize()
    assert np.array_equal(_host_vals(vs2), new_vals)
    assert torch.equal(m2, m) and torch.equal(v2, v)
    assert np.array_equal(host(dp2.values), host(dp.values)) and np.array_equal(host(dp2.meta), host(dp.meta))


def test_adamw_empty():
    z = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    zf = torch.empty(0, dtype=torch.float32, device="cuda")
    S.slope_adamw(z, z, zf, zf, 1, lr=1e-3)
    dp = Compressed(0, 0, torch.bfloat16)
    S.slope_adamw_double_prune(z, torch.empty(0, dtype=torch.int32, device="cuda"), z, zf, zf, 0, 0, dp.values,
                               dp.meta, 1, lr=1e-3)
    torch.cuda.synchronize()
