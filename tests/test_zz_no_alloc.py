"""The allocation-free few-token forward (slope_spmm_fwd_decode_noalloc),
called through the C ABI, against the workspace form slope_spmm_fwd_decode on
the same inputs.  Both run the same kernels in the same split order, so their
outputs must agree bit for bit.  Calls follow each other on one stream, the
second smaller than the first (the static scratch keeps the first call's
contents, and nothing read may depend on them), then the first size again.  A
size whose scratch need exceeds the static array is rejected before anything
is written.  The smallest case is also checked against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import layer_inputs

from gpu_util import TOL, dev, host, host_f64, normwise, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()


class Case:
    """A compressed weight in tile-chunk form, inputs and both outputs of one size."""

    def __init__(self, T, K, N, r, seed):
        self.T, self.K, self.N, self.r = T, K, N, r
        self.d = layer_inputs(K, N, T, r, "bf16", seed=seed, which=("W", "X", "L", "R"), threads=16)
        W = dev(self.d["W"])
        vals = torch.empty((N, K // 2), dtype=torch.bfloat16, device="cuda")
        meta = torch.empty((N, (K // 4 + 7) // 8), dtype=torch.int32, device="cuda")
        self.ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
        S.slope_prune_compress24(W, vals, meta, packed=self.ps)
        self.X, self.L, self.R = dev(self.d["X"]), dev(self.d["L"]), dev(self.d["R"])
        self.ws = torch.empty(max(16, S.slope_decode_workspace_bytes(T, K, r, N)), dtype=torch.uint8, device="cuda")
        self.Y_ref = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        S.slope_spmm_fwd_decode(self.X, self.ps, N, self.Y_ref, self.ws, L=self.L, R=self.R)

    def noalloc(self):
        """One call of the allocation-free entry point straight through ctypes."""
        Y = torch.full((self.T, self.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        lib = S.library()
        st = lib.slope_spmm_fwd_decode_noalloc(1, 1, self.X.data_ptr(), self.T, self.K, self.ps.data_ptr(),
                                               self.ps.numel(), self.N, self.L.data_ptr(), self.R.data_ptr(), self.r,
                                               Y.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, S.STATUS.get(st, st)
        return Y

    def same(self, Y):
        return torch.equal(Y.view(torch.int16), self.Y_ref.view(torch.int16))


def test_noalloc_decode_matches_workspace_form():
    # OPT-66B QKV at 16 tokens (6.8 MiB of scratch), then a small ragged layer
    big = Case(16, 9216, 27648, 72, seed=3)
    small = Case(3, 528, 272, 8, seed=4)
    assert S.slope_decode_workspace_bytes(16, 9216, 72, 27648) <= S.DECODE_NOALLOC_SCRATCH_BYTES
    say("[noalloc] big, small, big")
    y1 = big.noalloc()
    y2 = small.noalloc()
    y3 = big.noalloc()
    torch.cuda.synchronize()
    assert big.same(y1)
    assert small.same(y2)
    assert big.same(y3)
    # the small case against the oracle as well
    mask, _ = oracle.prune24(small.d["W"])
    vs, ms, _ = oracle.compress24(small.d["W"], mask)
    ref = oracle.spmm_fwd(small.d["X"], vs, ms, small.K, small.d["L"], small.d["R"])
    assert normwise(host_f64(y2), ref) <= TOL["bf16"]


def test_noalloc_decode_without_adapter_and_fp32_output():
    c = Case(64, 2048, 1024, 16, seed=5)
    Y = torch.empty((64, 1024), dtype=torch.float32, device="cuda")
    Yw = torch.empty_like(Y)
    S.slope_spmm_fwd_decode_noalloc(c.X, c.ps, 1024, Y)
    S.slope_spmm_fwd_decode(c.X, c.ps, 1024, Yw, c.ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yw)


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    # OPT-66B FC1 at 64 tokens needs 36 MiB of scratch: refused, nothing written
    T, K, N, r = 64, 9216, 36864, 72
    assert S.slope_decode_workspace_bytes(T, K, r, N) > S.DECODE_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    ps = torch.zeros(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    L = torch.zeros((K, r), dtype=torch.bfloat16, device="cuda")
    R = torch.zeros((r, N), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S.SlopeError) as e:
        S.slope_spmm_fwd_decode_noalloc(X, ps, N, Y, L=L, R=R)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())
