"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, checked on sampled outputs the oracle computes one by one and
on properties that hold at any size.

For every linear of every workload (toy fp32; GPT-2-small, BERT-Large, OPT-13B
and OPT-66B layers in bf16; the decode token counts of OPT-13B and OPT-66B) the
whole path runs on the GPU: prune24 -> compress24 -> double_prune ->
spmm_fwd (+ adapter) -> spmm_bwd_dx -> masked_wgrad.  Then:

* masks / compressed values / metadata: sampled rows bit-exact against the
  oracle run on the same rows; every group of the full mask keeps exactly two;
* double pruning: sampled column groups of W_s, pruned again by the oracle,
  bit-exact against the matching rows of W_dp^T;
* products: sampled token x feature blocks against the oracle (normwise 1e-2
  for bf16 outputs, 1e-5 for the fp32 workload); the weight gradient goes
  through the packed operands as the benchmark runs it, and so do the sparse
  products (tile-chunk weights);
* the weight update (AdamW on the compressed values fused with the double
  prune): sampled rows of values and moments within the bound the optimizer
  tests derive; sampled column groups of the new W_dp^T bit-exact against the
  oracle's double prune of the values the GPU stored.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import WORKLOADS, layer_inputs, optimizer_inputs

from gpu_util import (TOL, Compressed, check_adamw_update as _check_update, dev, host, host_f64, normwise, say,
                      torch_dtype, workspace)

pytestmark = pytest.mark.gpu

CASES = [(wl, i) for wl in WORKLOADS for i in range(len(WORKLOADS[wl].linears))]
DECODE = [(wl, i, T) for wl in WORKLOADS for T in WORKLOADS[wl].decode_T for i in range(len(WORKLOADS[wl].linears))]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _same_bits(a, b):
    """Bit-for-bit equality (fp16 arrays compared as their 16-bit patterns)."""
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if b.dtype == np.float16:
        b = b.view(np.uint16)
    return a.dtype == b.dtype and np.array_equal(a, b)


def _group_cols(rng, K, n):
    """n random column groups of 4 (start columns, multiples of 4)."""
    return np.sort(rng.choice(K // 4, size=min(n, K // 4), replace=False)) * 4


def _rows(rng, n, k):
    return np.sort(rng.choice(n, size=min(k, n), replace=False))


def _run_path(d, T, N, K, r, tdt):
    """The whole hot path on the GPU; returns device tensors."""
    W, X, dY, L, R = (dev(d[k]) for k in ("W", "X", "dY", "L", "R"))
    out = {}
    out["mask"] = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    S.slope_prune24(W, out["mask"])
    c = Compressed(N, K, tdt)
    S.slope_compress24(W, out["mask"], c.values, c.meta)
    dp = Compressed(K, N, tdt)
    S.slope_double_prune(c.values, c.meta, N, K, dp.values, dp.meta)
    Y = torch.empty((T, N), dtype=tdt, device="cuda")
    dX = torch.empty((T, K), dtype=tdt, device="cuda")
    if tdt != torch.float32:   # the benchmark's form: tile-chunk weights
        ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
        pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
        S.slope_pack_sparse(c.values, c.meta, N, K, ps)
        S.slope_pack_sparse(dp.values, dp.meta, K, N, pd)
        S.slope_spmm_fwd_packed(X, ps, N, Y, L=L, R=R, workspace=workspace(T, K, r, N))
        S.slope_spmm_bwd_dx_packed(dY, pd, K, dX)
        del ps, pd
    else:
        S.slope_spmm_fwd(X, c.values, c.meta, N, Y, L=L, R=R, workspace=workspace(T, K, r, N))
        S.slope_spmm_bwd_dx(dY, dp.values, dp.meta, K, dX)
    dW = torch.empty((N, K // 2), dtype=tdt, device="cuda")
    if tdt != torch.float32:   # the benchmark's form: packed operands, then the GEMM
        Xp = torch.empty(S.slope_packed_tokens_bytes(T, K), dtype=torch.uint8, device="cuda")
        dYp = torch.empty(S.slope_packed_tokens_bytes(T, N), dtype=torch.uint8, device="cuda")
        S.slope_pack_tokens(X, Xp)
        S.slope_pack_tokens(dY, dYp)
        S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, c.meta, dW)
    else:
        S.slope_masked_wgrad(dY, X, c.meta, dW)
    torch.cuda.synchronize()
    out.update(vs=c.values, ms=c.meta, vdp=dp.values, mdp=dp.meta, Y=Y, dX=dX, dW=dW)
    return out


F16_CASES = [("opt_66b", 0), ("gpt2_small", 2)]


@pytest.mark.parametrize("wl,idx", CASES, ids=[f"{w}-{WORKLOADS[w].linears[i].name}" for w, i in CASES])
def test_full_path_sampled(wl, idx):
    _full_path_sampled(wl, idx, WORKLOADS[wl].dtype)


@pytest.mark.parametrize("wl,idx", F16_CASES, ids=[f"{w}-{WORKLOADS[w].linears[i].name}-f16" for w, i in F16_CASES])
def test_full_path_sampled_f16(wl, idx):
    """The same full-size checks on the fp16 instantiation of the path."""
    _full_path_sampled(wl, idx, "f16")


def _full_path_sampled(wl, idx, dtype):
    w = WORKLOADS[wl]
    lin = w.linears[idx]
    T, N, K, r = w.T, lin.N, lin.K, w.r
    say(f"[fullsize] {wl} {lin.name}: T={T} K={K} N={N} r={r} dtype={dtype}")
    d = layer_inputs(K, N, T, r, dtype, seed=0, index=idx)
    tdt = torch_dtype(dtype)
    tol = TOL[dtype]
    o = _run_path(d, T, N, K, r, tdt)
    rng = np.random.default_rng(1000 + idx)

    # --- masks and compression: every group keeps exactly two; sampled rows bit-exact
    assert bool((o["mask"].view(-1, 4).sum(dim=1, dtype=torch.int32) == 2).all())
    rows = _rows(rng, N, 24)
    mask_ref, _ = oracle.prune24(d["W"][rows])
    assert (host(o["mask"][rows]) == mask_ref).all()
    v_ref, m_ref, _ = oracle.compress24(d["W"][rows], mask_ref)
    assert _same_bits(host(o["vs"][rows]), v_ref)
    assert (host(o["ms"][rows]) == m_ref).all()

    # --- double pruning on sampled column groups (all N rows of W_s for 4 columns)
    gcols = _group_cols(rng, K, 6)
    for c0 in gcols:
        Wc = np.ascontiguousarray(d["W"][:, c0:c0 + 4])
        mc, _ = oracle.prune24(Wc)                 # W_s restricted to these columns
        vc, mcw, _ = oracle.compress24(Wc, mc)
        vdp_ref, mdp_ref, _ = oracle.double_prune(vc, mcw, N, 4)
        assert _same_bits(host(o["vdp"][c0:c0 + 4]), vdp_ref), c0
        assert (host(o["mdp"][c0:c0 + 4]) == mdp_ref).all(), c0

    # --- forward with adapter on a sampled token x feature block
    ts = _rows(rng, T, 48)
    ns = _rows(rng, N, 48)
    vsub, msub, _ = oracle.compress24(d["W"][ns], oracle.prune24(d["W"][ns])[0])
    y_ref = oracle.spmm_fwd(d["X"][ts], vsub, msub, K, d["L"], np.ascontiguousarray(d["R"][:, ns]))
    assert normwise(host_f64(o["Y"][ts][:, ns]), y_ref) <= tol

    # --- dX on sampled tokens x sampled column groups (W_dp columns from the oracle)
    for c0 in gcols[:3]:
        Wc = np.ascontiguousarray(d["W"][:, c0:c0 + 4])
        mc, _ = oracle.prune24(Wc)
        vc, mcw, _ = oracle.compress24(Wc, mc)
        vdp_ref, mdp_ref, _ = oracle.double_prune(vc, mcw, N, 4)
        dx_ref = oracle.spmm_bwd_dx(d["dY"][ts], vdp_ref, mdp_ref, N)
        assert normwise(host_f64(o["dX"][ts][:, c0:c0 + 4]), dx_ref) <= tol

    # --- dW on sampled rows x a 64-column window (full token reduction)
    nw = _rows(rng, N, 16)
    kw0 = int(rng.integers(0, max(1, K // 64))) * 64
    kw = min(64, K - kw0)
    Wsub = np.ascontiguousarray(d["W"][nw][:, kw0:kw0 + kw])
    _, msub, _ = oracle.compress24(Wsub, oracle.prune24(Wsub)[0])
    dwv_ref, _ = oracle.masked_wgrad(np.ascontiguousarray(d["dY"][:, nw]),
                                     np.ascontiguousarray(d["X"][:, kw0:kw0 + kw]), msub, kw)
    got = host_f64(o["dW"][nw][:, kw0 // 2:(kw0 + kw) // 2])
    assert normwise(got, dwv_ref) <= tol
    del o
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl,idx,T", DECODE, ids=[f"{w}-{WORKLOADS[w].linears[i].name}-T{t}" for w, i, t in DECODE])
def test_decode_forward_sampled(wl, idx, T):
    """Inference shapes: the few-token forward with the unmerged adapter at T = 1..64."""
    w = WORKLOADS[wl]
    lin = w.linears[idx]
    N, K, r = lin.N, lin.K, w.r
    say(f"[decode] {wl} {lin.name}: T={T} K={K} N={N} r={r}")
    d = layer_inputs(K, N, T, r, w.dtype, seed=7, index=idx, which=("W", "X", "L", "R"))
    Wd = dev(d["W"])
    mask = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    S.slope_prune24(Wd, mask)
    c = Compressed(N, K, torch.bfloat16)
    S.slope_compress24(Wd, mask, c.values, c.meta)
    Y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(c.values, c.meta, N, K, ps)
    ws = torch.empty(S.slope_decode_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    S.slope_spmm_fwd_decode(dev(d["X"]), ps, N, Y, ws, L=dev(d["L"]), R=dev(d["R"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(idx + T)
    ns = _rows(rng, N, 64)
    vsub, msub, _ = oracle.compress24(d["W"][ns], oracle.prune24(d["W"][ns])[0])
    y_ref = oracle.spmm_fwd(d["X"], vsub, msub, K, d["L"], np.ascontiguousarray(d["R"][:, ns]))
    assert normwise(host_f64(Y[:, ns]), y_ref) <= TOL["bf16"]


ADAPTER_CASES = [(wl, i) for wl in ("gpt2_small", "bert_large") for i in range(len(WORKLOADS[wl].linears))]


@pytest.mark.parametrize("wl,idx", ADAPTER_CASES, ids=[f"{w}-{WORKLOADS[w].linears[i].name}" for w, i in ADAPTER_CASES])
def test_adapter_backward_sampled(wl, idx):
    """The adapter's backward at full size: the dX term through the packed dX
    product, dL and dR from token chunks; sampled rows / columns against the oracle."""
    w = WORKLOADS[wl]
    lin = w.linears[idx]
    T, N, K, r = w.T, lin.N, lin.K, w.r
    say(f"[fullsize-adapter] {wl} {lin.name}: T={T} K={K} N={N} r={r}")
    d = layer_inputs(K, N, T, r, w.dtype, seed=0, index=idx)
    W, X, dY, L, R = (dev(d[k]) for k in ("W", "X", "dY", "L", "R"))
    mask = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    S.slope_prune24(W, mask)
    c = Compressed(N, K, torch.bfloat16)
    S.slope_compress24(W, mask, c.values, c.meta)
    dp = Compressed(K, N, torch.bfloat16)
    S.slope_double_prune(c.values, c.meta, N, K, dp.values, dp.meta)
    pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dp.values, dp.meta, K, N, pd)
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    wsx = torch.empty(S.slope_lowrank_workspace_bytes(T, N, r, K), dtype=torch.uint8, device="cuda")
    S.slope_spmm_bwd_dx_packed(dY, pd, K, dX, L=L, R=R, workspace=wsx)
    Xp = torch.empty(S.slope_packed_tokens_bytes(T, K), dtype=torch.uint8, device="cuda")
    dYp = torch.empty(S.slope_packed_tokens_bytes(T, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_tokens(X, Xp)
    S.slope_pack_tokens(dY, dYp)
    dL = torch.empty((K, r), dtype=torch.bfloat16, device="cuda")
    dR = torch.empty((r, N), dtype=torch.bfloat16, device="cuda")
    wsg = torch.empty(S.slope_lowrank_grads_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    S.slope_lowrank_grads_packed(X, dY, Xp, dYp, L, R, wsg, dL, dR)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2000 + idx)
    tol = TOL[w.dtype]
    # dX on sampled tokens: the sparse product (oracle double prune of sampled column groups) + the adapter term
    ts = _rows(rng, T, 32)
    term = oracle.lowrank_bwd(d["X"][ts], d["dY"][ts], d["L"], d["R"])[0]
    for c0 in _group_cols(rng, K, 3):
        Wc = np.ascontiguousarray(d["W"][:, c0:c0 + 4])
        mc, _ = oracle.prune24(Wc)
        vc, mcw, _ = oracle.compress24(Wc, mc)
        vdp_ref, mdp_ref, _ = oracle.double_prune(vc, mcw, N, 4)
        ref = oracle.spmm_bwd_dx(d["dY"][ts], vdp_ref, mdp_ref, N) + term[:, c0:c0 + 4]
        assert normwise(host_f64(dX[ts][:, c0:c0 + 4]), ref) <= tol
    # dR on sampled columns (all tokens), dL on sampled rows (all tokens)
    ns = _rows(rng, N, 48)
    dR_ref = oracle.lowrank_bwd(d["X"], np.ascontiguousarray(d["dY"][:, ns]), d["L"],
                                np.ascontiguousarray(d["R"][:, ns]))[2]
    assert normwise(host_f64(dR[:, ns]), dR_ref) <= tol
    ks = _rows(rng, K, 48)
    dL_ref = oracle.lowrank_bwd(np.ascontiguousarray(d["X"][:, ks]), d["dY"], np.ascontiguousarray(d["L"][ks]),
                                d["R"])[1]
    assert normwise(host_f64(dL[ks]), dL_ref) <= tol


UPDATE_HP = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.mark.parametrize("wl,idx", CASES, ids=[f"{w}-{WORKLOADS[w].linears[i].name}" for w, i in CASES])
def test_weight_update_sampled(wl, idx):
    """AdamW on the compressed values fused with the double prune, at full size."""
    w = WORKLOADS[wl]
    lin = w.linears[idx]
    N, K = lin.N, lin.K
    say(f"[fullsize-update] {wl} {lin.name}: K={K} N={N} dtype={w.dtype}")
    Wb = layer_inputs(K, N, w.T, w.r, w.dtype, seed=0, index=idx, which=("W",))["W"]
    opt = optimizer_inputs(N, K, w.dtype, seed=0, index=idx)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Wd = dev(Wb)
    mask = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    S.slope_prune24(Wd, mask)
    c = Compressed(N, K, tdt)
    S.slope_compress24(Wd, mask, c.values, c.meta)
    del Wd, mask
    G = dev(opt["G"])
    M = torch.from_numpy(opt["M"]).to("cuda:0")
    V = torch.from_numpy(opt["V"]).to("cuda:0")
    dp = Compressed(K, N, tdt)
    step = 11
    S.slope_adamw_double_prune(c.values, c.meta, G, M, V, N, K, dp.values, dp.meta, step, **UPDATE_HP)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3000 + idx)
    # sampled rows: the oracle's own compression of W, then its update
    rows = _rows(rng, N, 16)
    mask_ref, _ = oracle.prune24(Wb[rows])
    v0, m_ref, _ = oracle.compress24(Wb[rows], mask_ref)
    assert (host(c.meta[rows]) == m_ref).all()
    _check_update(v0, opt["G"][rows], opt["M"][rows], opt["V"][rows], step, UPDATE_HP, host(c.values[rows]),
                  M[rows].cpu().numpy(), V[rows].cpu().numpy())
    # sampled column groups: all N rows of W_s for 4 columns
    for c0 in _group_cols(rng, K, 4):
        Wc = np.ascontiguousarray(Wb[:, c0:c0 + 4])
        mc, _ = oracle.prune24(Wc)
        vc, mcw, _ = oracle.compress24(Wc, mc)
        sl = slice(c0 // 2, c0 // 2 + 2)
        new_vc = host(c.values[:, sl])
        _check_update(vc, opt["G"][:, sl], opt["M"][:, sl], opt["V"][:, sl], step, UPDATE_HP, new_vc,
                      M[:, sl].cpu().numpy(), V[:, sl].cpu().numpy())
        vdp_ref, mdp_ref, _ = oracle.double_prune(new_vc, mcw, N, 4)
        assert _same_bits(host(dp.values[c0:c0 + 4]), vdp_ref), c0
        assert (host(dp.meta[c0:c0 + 4]) == mdp_ref).all(), c0
    del c, dp, G, M, V
    torch.cuda.empty_cache()



@pytest.mark.parametrize("idx", [0, 3])
def test_prune_compress24_full_size(idx):
    """The one-pass prune at OPT-66B QKV / FC2 weight size (many grid-stride
    iterations per lane, with the (row, pair) step carrying across rows):
    mask, values, metadata and W_s's tile chunks equal the separate prune24,
    compress24 and pack_sparse calls bit for bit, and sampled rows equal the
    oracle."""
    lin = WORKLOADS["opt_66b"].linears[idx]
    K, N = lin.K, lin.N
    say(f"[prune_compress24 full] {lin.name}: {N}x{K}")
    Wh = layer_inputs(K, N, 1, 1, "bf16", seed=41 + idx, which=("W",), threads=16)["W"]
    W = dev(Wh)
    mask = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    c = Compressed(N, K, torch.bfloat16)
    pk = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_prune_compress24(W, c.values, c.meta, mask=mask, packed=pk)
    mask2 = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    c2 = Compressed(N, K, torch.bfloat16)
    pk2 = torch.empty_like(pk)
    S.slope_prune24(W, mask2)
    S.slope_compress24(W, mask2, c2.values, c2.meta)
    S.slope_pack_sparse(c2.values, c2.meta, N, K, pk2)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2)
    assert torch.equal(c.values.view(torch.int16), c2.values.view(torch.int16))
    assert torch.equal(c.meta, c2.meta)
    assert torch.equal(pk, pk2)
    rows = np.sort(np.random.default_rng(42).choice(N, size=32, replace=False))
    m_ref, _ = oracle.prune24(Wh[rows])
    v_ref, meta_ref, _ = oracle.compress24(Wh[rows], m_ref)
    idx_t = torch.from_numpy(rows).cuda()
    assert (host(mask.index_select(0, idx_t)) == m_ref).all()
    assert (host(c.values.index_select(0, idx_t)) == v_ref).all()
    assert (host(c.meta.index_select(0, idx_t)) == meta_ref).all()
