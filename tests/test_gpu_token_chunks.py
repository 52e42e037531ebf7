"""GPU checks of the packed products that also write their dense operand as
token chunks (slope_spmm_fwd_packed_tokens, slope_spmm_bwd_dx_packed_tokens).

* The chunks equal slope_pack_tokens' output byte for byte, and every byte is
  written: the buffer starts filled with a marker, and the layout itself is
  checked against the numpy construction of the header's description.
* The products' outputs equal the plain packed calls bit for bit (with and
  without the adapter), so the oracle parity of those calls carries over.
* Shapes take every tile path of the product: narrow tiles only (one round of
  blocks), full-width rows plus narrow rows, and full-width tiles only; token
  counts that end inside a 32-token chunk, and reduction widths that end
  inside a 64-wide stage and inside a 256-row chunk column (rows no stage
  covers must come out zero).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import layer_inputs

from gpu_util import Compressed, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _u8(nbytes, fill=None):
    t = torch.empty(max(16, nbytes), dtype=torch.uint8, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def _layout(bits, T, C):
    """The token-chunk layout as include/slope.h states it, built with numpy."""
    Tch, Cch = -(-T // 32), -(-C // 256)
    pad = np.zeros((Tch * 32, Cch * 256), dtype=np.uint16)
    pad[:T, :C] = bits
    blk = pad.reshape(Tch, 32, Cch, 256).transpose(2, 0, 3, 1).reshape(Cch, Tch, 256, 4, 8)  # [c][s][row][g][tok]
    out = np.empty_like(blk)
    rows = np.arange(256)
    for g in range(4):
        out[:, :, rows, g ^ ((rows >> 2) & 3)] = blk[:, :, rows, g]
    return out.reshape(-1)


# (T, K, N): the product's reduction width is K for the forward and N for dX.
# (both widths multiples of 16). Tile paths on 256 compute units: (1000, 272,
# 528) one round, narrow tiles only (both products); (4096, 4608, 4608)
# full-width rows plus narrow rows; (8192, 1040, 4096) full width only;
# (777, 528, 336) tokens ending inside a chunk, widths ending inside a stage
# and inside a chunk column; (96, 64, 256) one stage, three token groups
SHAPES = [(1000, 272, 528), (777, 528, 336), (4096, 4608, 4608), (8192, 1040, 4096), (96, 64, 256)]


@pytest.mark.parametrize("adapter", [False, True])
@pytest.mark.parametrize("T,K,N", SHAPES)
def test_products_write_token_chunks(T, K, N, adapter):
    r = 24 if adapter else 0
    say(f"[token chunks] T={T} K={K} N={N} r={r}")
    d = layer_inputs(K, N, T, max(r, 1), "bf16", seed=T + K + N, which=("W", "X", "dY", "L", "R"))
    W, X, dY = dev(d["W"]), dev(d["X"]), dev(d["dY"])
    L, R = (dev(d["L"]), dev(d["R"])) if adapter else (None, None)
    bf = torch.bfloat16
    c = Compressed(N, K, bf)
    ps, pd = _u8(S.slope_packed_sparse_bytes(N, K)), _u8(S.slope_packed_sparse_bytes(K, N))
    S.slope_prune_compress24(W, c.values, c.meta, packed=ps)
    S.slope_double_prune_packed(c.values, c.meta, N, K, pd)
    ws = _u8(S.slope_lowrank_workspace_bytes(T, K, r, N)) if adapter else None
    wsb = _u8(S.slope_lowrank_workspace_bytes(T, N, r, K)) if adapter else None

    # forward: Y and X's chunks
    xb = S.slope_packed_tokens_bytes(T, K)
    Xp, Xp_ref = _u8(xb, 0xAB), _u8(xb, 0xCD)
    Y, Y_ref = (torch.empty((T, N), dtype=bf, device="cuda") for _ in range(2))
    S.slope_spmm_fwd_packed_tokens(X, ps, N, Y, Xp, L=L, R=R, workspace=ws)
    S.slope_spmm_fwd_packed(X, ps, N, Y_ref, L=L, R=R, workspace=ws)
    S.slope_pack_tokens(X, Xp_ref)
    # dX: dX and dY's chunks
    yb = S.slope_packed_tokens_bytes(T, N)
    dYp, dYp_ref = _u8(yb, 0xAB), _u8(yb, 0xCD)
    dX, dX_ref = (torch.empty((T, K), dtype=bf, device="cuda") for _ in range(2))
    S.slope_spmm_bwd_dx_packed_tokens(dY, pd, K, dX, dYp, L=L, R=R, workspace=wsb)
    S.slope_spmm_bwd_dx_packed(dY, pd, K, dX_ref, L=L, R=R, workspace=wsb)
    S.slope_pack_tokens(dY, dYp_ref)
    torch.cuda.synchronize()

    assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16))
    assert torch.equal(dX.view(torch.int16), dX_ref.view(torch.int16))
    assert torch.equal(Xp[:xb], Xp_ref[:xb])
    assert torch.equal(dYp[:yb], dYp_ref[:yb])
    if T * max(K, N) <= 1 << 21:   # the layout itself, on the host, where it is quick
        assert np.array_equal(Xp[:xb].cpu().numpy().view(np.uint16), _layout(d["X"], T, K))
        assert np.array_equal(dYp[:yb].cpu().numpy().view(np.uint16), _layout(d["dY"], T, N))


@pytest.mark.parametrize("adapter", [False, True])
def test_products_write_token_chunks_f16(adapter):
    """The fp16 instantiations: the same bytes as the packing pass, the same outputs as the plain calls."""
    T, K, N = 777, 528, 336
    r = 16 if adapter else 0
    say(f"[token chunks f16] T={T} K={K} N={N} r={r}")
    d = layer_inputs(K, N, T, max(r, 1), "f16", seed=5, which=("W", "X", "dY", "L", "R"))
    W, X, dY = dev(d["W"]), dev(d["X"]), dev(d["dY"])
    L, R = (dev(d["L"]), dev(d["R"])) if adapter else (None, None)
    h = torch.float16
    c = Compressed(N, K, h)
    ps, pd = _u8(S.slope_packed_sparse_bytes(N, K)), _u8(S.slope_packed_sparse_bytes(K, N))
    S.slope_prune_compress24(W, c.values, c.meta, packed=ps)
    S.slope_double_prune_packed(c.values, c.meta, N, K, pd)
    ws = _u8(S.slope_lowrank_workspace_bytes(T, K, r, N)) if adapter else None
    wsb = _u8(S.slope_lowrank_workspace_bytes(T, N, r, K)) if adapter else None
    xb, yb = S.slope_packed_tokens_bytes(T, K), S.slope_packed_tokens_bytes(T, N)
    Xp, Xq, dYp, dYq = _u8(xb, 0xAB), _u8(xb, 0xCD), _u8(yb, 0xAB), _u8(yb, 0xCD)
    Y, Y_ref = (torch.empty((T, N), dtype=h, device="cuda") for _ in range(2))
    dX, dX_ref = (torch.empty((T, K), dtype=h, device="cuda") for _ in range(2))
    S.slope_spmm_fwd_packed_tokens(X, ps, N, Y, Xp, L=L, R=R, workspace=ws)
    S.slope_spmm_fwd_packed(X, ps, N, Y_ref, L=L, R=R, workspace=ws)
    S.slope_spmm_bwd_dx_packed_tokens(dY, pd, K, dX, dYp, L=L, R=R, workspace=wsb)
    S.slope_spmm_bwd_dx_packed(dY, pd, K, dX_ref, L=L, R=R, workspace=wsb)
    S.slope_pack_tokens(X, Xq)
    S.slope_pack_tokens(dY, dYq)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16))
    assert torch.equal(dX.view(torch.int16), dX_ref.view(torch.int16))
    assert torch.equal(Xp[:xb], Xq[:xb]) and torch.equal(dYp[:yb], dYq[:yb])


def test_chunks_feed_the_weight_gradient():
    """The chunks the products write serve the weight gradient as the packing
    pass's do: dW from them equals dW from slope_pack_tokens bit for bit, and
    matches the oracle."""
    T, K, N = 777, 528, 336
    d = layer_inputs(K, N, T, 1, "bf16", seed=11, which=("W", "X", "dY"))
    W, X, dY = dev(d["W"]), dev(d["X"]), dev(d["dY"])
    bf = torch.bfloat16
    c = Compressed(N, K, bf)
    ps, pd = _u8(S.slope_packed_sparse_bytes(N, K)), _u8(S.slope_packed_sparse_bytes(K, N))
    S.slope_prune_compress24(W, c.values, c.meta, packed=ps)
    S.slope_double_prune_packed(c.values, c.meta, N, K, pd)
    Xp, dYp = _u8(S.slope_packed_tokens_bytes(T, K)), _u8(S.slope_packed_tokens_bytes(T, N))
    Y, dX = torch.empty((T, N), dtype=bf, device="cuda"), torch.empty((T, K), dtype=bf, device="cuda")
    S.slope_spmm_fwd_packed_tokens(X, ps, N, Y, Xp)
    S.slope_spmm_bwd_dx_packed_tokens(dY, pd, K, dX, dYp)
    dW = torch.empty((N, K // 2), dtype=torch.float32, device="cuda")
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, c.meta, dW)
    Xq, dYq = _u8(S.slope_packed_tokens_bytes(T, K)), _u8(S.slope_packed_tokens_bytes(T, N))
    S.slope_pack_tokens(X, Xq)
    S.slope_pack_tokens(dY, dYq)
    dW_ref = torch.empty_like(dW)
    S.slope_masked_wgrad_packed(dYq, Xq, T, N, K, c.meta, dW_ref)
    torch.cuda.synchronize()
    assert torch.equal(dW, dW_ref)
    mask, _ = oracle.prune24(d["W"])
    _, ms, _ = oracle.compress24(d["W"], mask)
    v_ref, _ = oracle.masked_wgrad(d["dY"], d["X"], ms, K)
    got = dW.cpu().double().numpy()
    assert np.linalg.norm(got - v_ref) <= 1e-5 * np.linalg.norm(v_ref)
    assert np.array_equal(host(c.meta), ms)
