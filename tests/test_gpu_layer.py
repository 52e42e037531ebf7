"""The training-side layer (SparseLinear, its autograd function, SparseAdamW)
against the oracle: one forward / backward / optimizer step / forward cycle.

The layer only orchestrates C-ABI calls, so this checks that it feeds each
call the right operands: construction state bit-exact (mask, compression, the
tile chunks of W_s and of its double prune), products and gradients within the
bf16 tolerance, the update within the optimizer bound of the values the
backward produced, both operands' tile chunks bit-exact against the oracle's
values and double prune of the stored values, and the next forward against
the oracle on the updated weights.  The tile-chunk layout comes from a numpy
restatement of include/slope.h.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_02_amd.layer import SparseAdamW, SparseLinear, training_state_bytes
from workloads import layer_inputs

from gpu_util import TOL, check_adamw_update, dev, host, host_f64, normwise, pack_sparse_reference, say


def _chunks_match(layer, vals, meta, vdp, mdp):
    """The layer's packed W_s and W_dp^T equal the tile chunks of the given
    compressed values (raw bits) and metadata."""
    N, K = layer.out_features, layer.in_features
    bits = lambda a: np.asarray(a).view(np.uint16)
    want_s = pack_sparse_reference(bits(vals), meta, N, K)
    want_dp = pack_sparse_reference(bits(vdp), mdp, K, N)
    return (np.array_equal(layer.packed_s.cpu().numpy()[:want_s.size], want_s)
            and np.array_equal(layer.packed_dpT.cpu().numpy()[:want_dp.size], want_dp))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,N,K,r", [(200, 512, 256, 8), (64, 272, 528, 16), (300, 256, 1024, 0)])
def test_layer_forward_backward_step(T, N, K, r):
    say(f"[layer] T={T} N={N} K={K} r={r}")
    d = layer_inputs(K, N, T, max(r, 1), "bf16", seed=5)
    W, X, dY = dev(d["W"]), dev(d["X"]), dev(d["dY"])
    L, R = (dev(d["L"]), dev(d["R"])) if r else (None, None)
    layer = SparseLinear(W, L, R)
    x = X.clone().requires_grad_(True)
    y = layer(x)
    y.backward(dY)
    torch.cuda.synchronize()

    mask_ref, _ = oracle.prune24(d["W"])
    vs_ref, ms_ref, _ = oracle.compress24(d["W"], mask_ref)
    vdp_ref, mdp_ref, _ = oracle.double_prune(vs_ref, ms_ref, N, K)
    assert np.array_equal(host(layer.values), vs_ref) and np.array_equal(host(layer.meta), ms_ref)
    assert _chunks_match(layer, vs_ref, ms_ref, vdp_ref, mdp_ref)

    La, Ra = (d["L"], d["R"]) if r else (None, None)
    tol = TOL["bf16"]
    assert normwise(host_f64(y), oracle.spmm_fwd(d["X"], vs_ref, ms_ref, K, La, Ra)) <= tol
    dx_ref = oracle.spmm_bwd_dx(d["dY"], vdp_ref, mdp_ref, N)
    if r:
        _, dL_ref, dR_ref = oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])
        dx_ref = dx_ref + oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])[0]
        assert normwise(host_f64(layer.L.grad), dL_ref) <= tol
        assert normwise(host_f64(layer.R.grad), dR_ref) <= tol
    assert normwise(host_f64(x.grad), dx_ref) <= tol
    dw_ref, _ = oracle.masked_wgrad(d["dY"], d["X"], ms_ref, K)
    assert normwise(host_f64(layer.values.grad), dw_ref) <= tol

    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    opt = SparseAdamW([layer], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                      weight_decay=hp["weight_decay"])
    g = host(layer.values.grad)
    zeros = np.zeros(g.shape, np.float32)
    adapter = [(p, host(p), host(p.grad)) for p in (layer.L, layer.R) if p is not None]
    opt.step()
    torch.cuda.synchronize()
    new_vs = host(layer.values)
    st = opt.state[layer.values]
    check_adamw_update(vs_ref, g, zeros, zeros, 1, hp, new_vs, st["exp_avg"].cpu().numpy(),
                       st["exp_avg_sq"].cpu().numpy())
    for p, p0, gp in adapter:
        z = np.zeros(p0.shape, np.float32)
        check_adamw_update(p0, gp, z, z, 1, hp, host(p), opt.state[p]["exp_avg"].cpu().numpy(),
                           opt.state[p]["exp_avg_sq"].cpu().numpy())
    assert np.array_equal(host(layer.meta), ms_ref)
    vdp1, mdp1, _ = oracle.double_prune(new_vs, ms_ref, N, K)
    assert _chunks_match(layer, new_vs, ms_ref, vdp1, mdp1)

    # the next forward and dX run on the updated, repacked weights
    x2 = X.clone().requires_grad_(True)
    y2 = layer(x2)
    y2.backward(dY)
    torch.cuda.synchronize()
    La1, Ra1 = (host(layer.L), host(layer.R)) if r else (None, None)
    assert normwise(host_f64(y2), oracle.spmm_fwd(d["X"], new_vs, ms_ref, K, La1, Ra1)) <= tol
    dx2 = oracle.spmm_bwd_dx(d["dY"], vdp1, mdp1, N)
    if r:
        dx2 = dx2 + oracle.lowrank_bwd(d["X"], d["dY"], La1, Ra1)[0]
    assert normwise(host_f64(x2.grad), dx2) <= tol

    # training state against a dense bf16 layer with AdamW: 7.25 of 12 bytes per weight
    # (values of W_s and W_dp^T, gradient, two fp32 moments, plus metadata words rounded up per row;
    # W_dp^T is held as tile chunks of 256 rows x 64 columns, 18432 bytes each)
    acc = training_state_bytes(layer, opt)
    words = lambda cols: -(-(cols // 4) // 8)
    chunks = lambda rows, cols: -(-rows // 256) * -(-cols // 64) * 18432
    assert acc["canonical"] == 6 * N * K + 4 * N * words(K) + chunks(K, N)
    if K % 256 == 0 and N % 64 == 0:
        assert acc["canonical"] == 7 * N * K + 4 * N * words(K) + 4 * K * words(N)
        assert abs(acc["canonical_ratio"] - 7.25 / 12) < 1e-12
    assert acc["dense_adamw"] == 12 * N * K


def test_layer_f16_step():
    """The same cycle in fp16: forward, backward, optimizer step against the oracle."""
    T, N, K, r = 96, 272, 528, 8
    d = layer_inputs(K, N, T, r, "f16", seed=8)
    layer = SparseLinear(dev(d["W"]), dev(d["L"]), dev(d["R"]))
    assert layer.values.dtype == torch.float16
    x = dev(d["X"]).clone().requires_grad_(True)
    y = layer(x)
    y.backward(dev(d["dY"]))
    mask_ref, _ = oracle.prune24(d["W"])
    vs_ref, ms_ref, _ = oracle.compress24(d["W"], mask_ref)
    vdp_ref, mdp_ref, _ = oracle.double_prune(vs_ref, ms_ref, N, K)
    tol = TOL["f16"]
    assert normwise(host_f64(y), oracle.spmm_fwd(d["X"], vs_ref, ms_ref, K, d["L"], d["R"])) <= tol
    term, dL_ref, dR_ref = oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])
    assert normwise(host_f64(x.grad), oracle.spmm_bwd_dx(d["dY"], vdp_ref, mdp_ref, N) + term) <= tol
    assert normwise(host_f64(layer.values.grad), oracle.masked_wgrad(d["dY"], d["X"], ms_ref, K)[0]) <= tol
    assert normwise(host_f64(layer.L.grad), dL_ref) <= tol and normwise(host_f64(layer.R.grad), dR_ref) <= tol
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-6, weight_decay=0.1)
    opt = SparseAdamW([layer], lr=hp["lr"], eps=hp["eps"], weight_decay=hp["weight_decay"])
    g = host(layer.values.grad)
    opt.step()
    torch.cuda.synchronize()
    z = np.zeros(g.shape, np.float32)
    st = opt.state[layer.values]
    check_adamw_update(vs_ref, g, z, z, 1, hp, host(layer.values), st["exp_avg"].cpu().numpy(),
                       st["exp_avg_sq"].cpu().numpy())
    vdp1, mdp1, _ = oracle.double_prune(host(layer.values), ms_ref, N, K)
    assert _chunks_match(layer, host(layer.values), ms_ref, vdp1, mdp1)


def test_two_layer_mlp_gradients_flow():
    """dX of the second layer is the first layer's output gradient (autograd chains the kernels)."""
    T, D, H = 128, 256, 512
    d1 = layer_inputs(D, H, T, 8, "bf16", seed=21, index=0)
    d2 = layer_inputs(H, D, T, 8, "bf16", seed=21, index=1)
    l1 = SparseLinear(dev(d1["W"]), dev(d1["L"]), dev(d1["R"]))
    l2 = SparseLinear(dev(d2["W"]), dev(d2["L"]), dev(d2["R"]))
    x = dev(d1["X"])
    h = l1(x)
    h.retain_grad()
    out = l2(h)
    out.backward(dev(d2["dY"]))
    torch.cuda.synchronize()
    # each stage against the oracle given the operands it received
    vs2, ms2, _ = oracle.compress24(d2["W"], oracle.prune24(d2["W"])[0])
    vdp2, mdp2, _ = oracle.double_prune(vs2, ms2, D, H)
    h_bits = host(h)
    dh_ref = oracle.spmm_bwd_dx(d2["dY"], vdp2, mdp2, D) + oracle.lowrank_bwd(h_bits, d2["dY"], d2["L"], d2["R"])[0]
    assert normwise(host_f64(h.grad), dh_ref) <= TOL["bf16"]
    vs1, ms1, _ = oracle.compress24(d1["W"], oracle.prune24(d1["W"])[0])
    dw1_ref, _ = oracle.masked_wgrad(host(h.grad), d1["X"], ms1, D)
    assert normwise(host_f64(l1.values.grad), dw1_ref) <= TOL["bf16"]
    _, dL1, dR1 = oracle.lowrank_bwd(d1["X"], host(h.grad), d1["L"], d1["R"])
    assert normwise(host_f64(l1.L.grad), dL1) <= TOL["bf16"]
    assert normwise(host_f64(l1.R.grad), dR1) <= TOL["bf16"]
