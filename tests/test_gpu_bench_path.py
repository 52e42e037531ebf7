"""GPU parity of the benchmark's own call sequence at the OPT-66B layer shape
(T = 8192 tokens, adapter rank 72, bf16), linear by linear, with the same
buffers reused the way bench.py reuses them:

    slope_prune_compress24 (W_s's tile chunks written) -> slope_double_prune_packed
    -> slope_spmm_fwd_packed_tokens (+ adapter, workspace ws; X's token chunks)
    -> slope_spmm_bwd_dx_packed_tokens (+ the adapter's dX term, workspace
       ws_bwd; dY's token chunks) -> slope_masked_wgrad_packed (split workspace:
       the last round's tiles in token ranges)
    -> slope_lowrank_grads_packed (X . L and dY . R^T taken from ws and ws_bwd)

and the training step's weight update, slope_adamw_double_prune_packed.

Checks (the oracle computes only sampled outputs at this size):
* the token chunks the two products write equal slope_pack_tokens' chunks
  byte for byte;
* the packed double prune equals slope_double_prune followed by
  slope_pack_sparse byte for byte, and sampled column groups of that canonical
  W_dp^T equal the oracle's double prune bit for bit;
* Y on a sampled token x feature block, dX (sparse product plus the adapter
  term) on sampled tokens x sampled column groups, dW on sampled rows, dL on
  sampled rows and dR on sampled columns, against the oracle within the bf16
  normwise tolerance;
* the packed update equals the canonical fused update followed by
  slope_pack_sparse of both operands, bit for bit, and its sampled rows stay
  within the AdamW bound of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import WORKLOADS, layer_inputs, optimizer_inputs

from gpu_util import TOL, Compressed, check_adamw_update, dev, host, host_f64, normwise, say

pytestmark = pytest.mark.gpu

WL = WORKLOADS["opt_66b"]
IDS = [l.name for l in WL.linears]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rows(rng, n, k):
    return np.sort(rng.choice(n, size=min(k, n), replace=False))


def _group_cols(rng, K, n):
    return np.sort(rng.choice(K // 4, size=min(n, K // 4), replace=False)) * 4


def _u8(nbytes):
    return torch.empty(max(16, nbytes), dtype=torch.uint8, device="cuda")


def _col_group_ref(W, c0, N):
    """The oracle's W_dp^T rows c0 .. c0+3: W_s restricted to four columns, double-pruned."""
    Wc = np.ascontiguousarray(W[:, c0:c0 + 4])
    mc, _ = oracle.prune24(Wc)
    vc, mcw, _ = oracle.compress24(Wc, mc)
    return oracle.double_prune(vc, mcw, N, 4)[:2]


@pytest.mark.parametrize("idx", range(len(WL.linears)), ids=IDS)
def test_bench_step_opt66b(idx):
    lin = WL.linears[idx]
    T, N, K, r = WL.T, lin.N, lin.K, WL.r
    say(f"[bench-path] opt_66b {lin.name}: T={T} K={K} N={N} r={r}")
    d = layer_inputs(K, N, T, r, "bf16", seed=0, index=idx, threads=16)
    W, X, dY, L, R = (dev(d[k]) for k in ("W", "X", "dY", "L", "R"))
    bf = torch.bfloat16
    c = Compressed(N, K, bf)
    ps = _u8(S.slope_packed_sparse_bytes(N, K))
    pd = _u8(S.slope_packed_sparse_bytes(K, N))
    ws = _u8(S.slope_lowrank_workspace_bytes(T, K, r, N))
    ws_bwd = _u8(S.slope_lowrank_workspace_bytes(T, N, r, K))
    ws_g = _u8(S.slope_lowrank_grads_workspace_bytes(T, K, r, N))
    Xp = _u8(S.slope_packed_tokens_bytes(T, K))
    dYp = _u8(S.slope_packed_tokens_bytes(T, N))
    Y = torch.empty((T, N), dtype=bf, device="cuda")
    dX = torch.empty((T, K), dtype=bf, device="cuda")
    dW = torch.empty((N, K // 2), dtype=bf, device="cuda")
    dL = torch.empty((K, r), dtype=bf, device="cuda")
    dR = torch.empty((r, N), dtype=bf, device="cuda")

    # the benchmark's step, in its order and with its buffer reuse
    S.slope_prune_compress24(W, c.values, c.meta, packed=ps)
    S.slope_double_prune_packed(c.values, c.meta, N, K, pd)
    S.slope_spmm_fwd_packed_tokens(X, ps, N, Y, Xp, L=L, R=R, workspace=ws)
    S.slope_spmm_bwd_dx_packed_tokens(dY, pd, K, dX, dYp, L=L, R=R, workspace=ws_bwd)
    wsp = _u8(S.slope_wgrad_split_workspace_bytes(T, N, K))    # the last round's tiles in token ranges
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, c.meta, dW, split_workspace=wsp)
    S.slope_lowrank_grads_packed(X, dY, Xp, dYp, L, R, ws_g, dL, dR, fwd_workspace=ws, bwd_workspace=ws_bwd)

    # the token chunks against the packing pass
    chunks_ref = _u8(max(Xp.numel(), dYp.numel()))
    S.slope_pack_tokens(dY, chunks_ref[:dYp.numel()])
    torch.cuda.synchronize()
    assert torch.equal(dYp, chunks_ref[:dYp.numel()])
    S.slope_pack_tokens(X, chunks_ref[:Xp.numel()])
    torch.cuda.synchronize()
    assert torch.equal(Xp, chunks_ref[:Xp.numel()])
    del chunks_ref

    # the packed double prune against the canonical one, then packed
    dp = Compressed(K, N, bf)
    S.slope_double_prune(c.values, c.meta, N, K, dp.values, dp.meta)
    pd_ref = torch.empty_like(pd)
    S.slope_pack_sparse(dp.values, dp.meta, K, N, pd_ref)
    torch.cuda.synchronize()
    assert torch.equal(pd, pd_ref)
    del pd_ref, W, Xp, dYp, ws_g
    torch.cuda.empty_cache()

    rng = np.random.default_rng(5000 + idx)
    tol = TOL["bf16"]
    gcols = _group_cols(rng, K, 4)
    refs = {c0: _col_group_ref(d["W"], c0, N) for c0 in gcols}
    for c0, (vdp_ref, mdp_ref) in refs.items():
        assert np.array_equal(host(dp.values[c0:c0 + 4]), vdp_ref), c0
        assert np.array_equal(host(dp.meta[c0:c0 + 4]), mdp_ref), c0

    # Y on sampled tokens x features (sparse product + adapter)
    ts = _rows(rng, T, 32)
    ns = _rows(rng, N, 48)
    vsub, msub, _ = oracle.compress24(d["W"][ns], oracle.prune24(d["W"][ns])[0])
    y_ref = oracle.spmm_fwd(d["X"][ts], vsub, msub, K, d["L"], np.ascontiguousarray(d["R"][:, ns]))
    assert normwise(host_f64(Y[ts][:, ns]), y_ref) <= tol

    # dX on sampled tokens x the sampled column groups, with the adapter's term
    term = oracle.lowrank_bwd(d["X"][ts], d["dY"][ts], d["L"], d["R"])[0]
    for c0, (vdp_ref, mdp_ref) in refs.items():
        ref = oracle.spmm_bwd_dx(d["dY"][ts], vdp_ref, mdp_ref, N) + term[:, c0:c0 + 4]
        assert normwise(host_f64(dX[ts][:, c0:c0 + 4]), ref) <= tol, c0

    # dW on sampled rows x a 64-column window, over all tokens
    nw = _rows(rng, N, 8)
    kw0 = int(rng.integers(0, K // 64)) * 64
    Wsub = np.ascontiguousarray(d["W"][nw][:, kw0:kw0 + 64])
    _, msub, _ = oracle.compress24(Wsub, oracle.prune24(Wsub)[0])
    dwv_ref, _ = oracle.masked_wgrad(np.ascontiguousarray(d["dY"][:, nw]), np.ascontiguousarray(d["X"][:, kw0:kw0 + 64]),
                                     msub, 64)
    assert normwise(host_f64(dW[nw][:, kw0 // 2:kw0 // 2 + 32]), dwv_ref) <= tol
    # ... and in the bottom-right output tile, always one of the last round's (token-range) tiles
    nw = np.sort(rng.choice(np.arange(N - 256, N), size=8, replace=False))
    kw0 = K - 64
    Wsub = np.ascontiguousarray(d["W"][nw][:, kw0:kw0 + 64])
    _, msub, _ = oracle.compress24(Wsub, oracle.prune24(Wsub)[0])
    dwv_ref, _ = oracle.masked_wgrad(np.ascontiguousarray(d["dY"][:, nw]), np.ascontiguousarray(d["X"][:, kw0:kw0 + 64]),
                                     msub, 64)
    assert normwise(host_f64(dW[nw][:, kw0 // 2:kw0 // 2 + 32]), dwv_ref) <= tol

    # dR on sampled columns, dL on sampled rows (sums over all 8192 tokens)
    nr = _rows(rng, N, 24)
    dR_ref = oracle.lowrank_bwd(d["X"], np.ascontiguousarray(d["dY"][:, nr]), d["L"],
                                np.ascontiguousarray(d["R"][:, nr]))[2]
    assert normwise(host_f64(dR[:, nr]), dR_ref) <= tol
    ks = _rows(rng, K, 24)
    dL_ref = oracle.lowrank_bwd(np.ascontiguousarray(d["X"][:, ks]), d["dY"], np.ascontiguousarray(d["L"][ks]),
                                d["R"])[1]
    assert normwise(host_f64(dL[ks]), dL_ref) <= tol


UPDATE_HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.mark.parametrize("idx", [0, 3], ids=[IDS[0], IDS[3]])
def test_bench_update_opt66b(idx):
    """slope_adamw_double_prune_packed at full size, as the benchmark's weight
    update runs it: equal bit for bit to the canonical fused update followed by
    slope_pack_sparse of both operands; sampled rows within the AdamW bound."""
    lin = WL.linears[idx]
    N, K = lin.N, lin.K
    say(f"[bench-update] opt_66b {lin.name}: K={K} N={N}")
    Wb = layer_inputs(K, N, 1, 1, "bf16", seed=0, index=idx, which=("W",), threads=16)["W"]
    opt = optimizer_inputs(N, K, "bf16", seed=0, index=idx, threads=16)
    bf = torch.bfloat16
    c = Compressed(N, K, bf)
    ps = _u8(S.slope_packed_sparse_bytes(N, K))
    S.slope_prune_compress24(dev(Wb), c.values, c.meta, packed=ps)
    G = dev(opt["G"])
    step = 5
    vs0 = c.values.clone()

    # canonical: the fused update, then both operands packed
    m_a, v_a = torch.from_numpy(opt["M"]).cuda(), torch.from_numpy(opt["V"]).cuda()
    vs_a = vs0.clone()
    dp = Compressed(K, N, bf)
    S.slope_adamw_double_prune(vs_a, c.meta, G, m_a, v_a, N, K, dp.values, dp.meta, step, **UPDATE_HP)
    ref_s = torch.empty_like(ps)
    ref_dp = _u8(S.slope_packed_sparse_bytes(K, N))
    S.slope_pack_sparse(vs_a, c.meta, N, K, ref_s)
    S.slope_pack_sparse(dp.values, dp.meta, K, N, ref_dp)
    del dp

    # packed: the benchmark's call on W_s's chunks from the one-pass prune
    m_b, v_b = torch.from_numpy(opt["M"]).cuda(), torch.from_numpy(opt["V"]).cuda()
    vs_b = vs0.clone()
    pk_dp = torch.full_like(ref_dp, 0x5A)
    S.slope_adamw_double_prune_packed(vs_b, c.meta, G, m_b, v_b, N, K, ps, pk_dp, step, **UPDATE_HP)
    torch.cuda.synchronize()
    assert torch.equal(vs_b.view(torch.int16), vs_a.view(torch.int16))
    assert torch.equal(m_b, m_a) and torch.equal(v_b, v_a)
    assert torch.equal(ps, ref_s)
    assert torch.equal(pk_dp, ref_dp)

    rng = np.random.default_rng(6000 + idx)
    rows = _rows(rng, N, 8)
    m_ref, _ = oracle.prune24(Wb[rows])
    v0, meta_ref, _ = oracle.compress24(Wb[rows], m_ref)
    assert np.array_equal(host(c.meta[rows]), meta_ref)
    check_adamw_update(v0, opt["G"][rows], opt["M"][rows], opt["V"][rows], step, UPDATE_HP, host(vs_b[rows]),
                       m_b[rows].cpu().numpy(), v_b[rows].cpu().numpy())
