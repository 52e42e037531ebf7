"""GPU parity of the weight gradient's token split (slope_masked_wgrad_packed
with a split workspace): for shapes whose output tiles leave most compute
units idle, the token reduction runs in ranges whose fp32 partial sums a
second kernel adds in order.

* normal inputs: values and the masked dense copy within the bf16 tolerance of
  the oracle, for bf16 and fp32 outputs, with and without accumulation;
* integer inputs: every product and partial sum is exact in fp32, so fp32
  outputs equal the oracle bit for bit, and so do the split and unsplit forms
  (bf16 and fp16 inputs, 16-bit outputs included);
* the split workspace size query is 0 exactly where no split is made, and the
  unsplit call is unchanged by a workspace it does not need.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import layer_inputs

from gpu_util import TOL, dev, dev_meta, empty, host_f64, normwise, say, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()


def _bits(a, dt):
    a = np.asarray(a, dtype=np.float32)
    if dt == "f16":
        return a.astype(np.float16)
    return (a.view(np.uint32) >> 16).astype(np.uint16)      # small integers are exact in bf16


def _inputs(T, N, K, dt, seed, ints):
    if ints:
        rng = np.random.default_rng(seed)
        d = {"W": _bits(rng.integers(-3, 4, size=(N, K)), dt), "X": _bits(rng.integers(-3, 4, size=(T, K)), dt),
             "dY": _bits(rng.integers(-3, 4, size=(T, N)), dt)}
    else:
        d = layer_inputs(K, N, T, 1, dt, seed=seed, which=("W", "X", "dY"))
    mask, _ = oracle.prune24(d["W"])
    _, ms, _ = oracle.compress24(d["W"], mask)
    d["ms"], d["mask"] = ms, mask
    return d


def _chunks(M):
    p = torch.empty(max(16, S.slope_packed_tokens_bytes(*M.shape)), dtype=torch.uint8, device="cuda")
    S.slope_pack_tokens(M, p)
    return p


def _split_ws(T, N, K):
    return torch.empty(max(16, S.slope_wgrad_split_workspace_bytes(T, N, K)), dtype=torch.uint8, device="cuda")


# (T, N, K): one or two output tiles with long token ranges (16 splits), a
# ragged shape (N, K not multiples of 256, T not of 32), GPT-2-small's O and
# QKV (9 and 27 tiles), BERT-Large's QKV (48 tiles)
SHAPES = [(4096, 256, 512), (1000, 264, 520), (8192, 768, 768), (8192, 2304, 768), (16384, 3072, 1024)]


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K", SHAPES)
def test_wgrad_split_matches_oracle(T, N, K, out_dt):
    need = S.slope_wgrad_split_workspace_bytes(T, N, K)
    say(f"[wgrad split] T={T} N={N} K={K} out={out_dt} split bytes={need}")
    assert need > 0
    d = _inputs(T, N, K, "bf16", seed=T + N + K, ints=False)
    X, dY = dev(d["X"]), dev(d["dY"])
    Xp, dYp, ws = _chunks(X), _chunks(dY), _split_ws(T, N, K)
    ms = dev_meta(d["ms"])
    dWv = empty((N, K // 2), torch_dtype(out_dt))
    dWd = empty((N, K), torch_dtype(out_dt))
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, dWv, dWd, split_workspace=ws, in_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    v_ref, d_ref = oracle.masked_wgrad(d["dY"], d["X"], d["ms"], K)
    assert normwise(host_f64(dWv), v_ref) <= TOL["bf16"]
    assert normwise(host_f64(dWd), d_ref) <= TOL["bf16"]
    assert (host_f64(dWd)[d["mask"] == 0] == 0).all()
    # against the unsplit form: the same sums grouped differently
    dWu = empty((N, K // 2), torch_dtype(out_dt))
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, dWu, in_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert normwise(host_f64(dWv), host_f64(dWu)) <= (TOL["bf16"] if out_dt == "bf16" else 1e-5)
    # accumulation: values and dense copy both add to what is there
    base = torch.randn((N, K // 2), device="cuda").to(torch_dtype(out_dt))
    based = torch.randn((N, K), device="cuda").to(torch_dtype(out_dt))
    acc, accd = base.clone(), based.clone()
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, acc, accd, accumulate=True, split_workspace=ws,
                                in_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert normwise(host_f64(acc), v_ref + host_f64(base)) <= TOL["bf16"]
    assert normwise(host_f64(accd), d_ref + host_f64(based)) <= TOL["bf16"]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("T,N,K", [(4096, 256, 512), (1000, 264, 520), (8192, 768, 768)])
def test_wgrad_split_integer_exact(T, N, K, dt):
    """Integer inputs in [-3, 3]: T * 9 < 2^24, so every partial sum is exact in
    fp32; the split fp32 output equals the oracle and the unsplit output bit for bit."""
    say(f"[wgrad split integer] T={T} N={N} K={K} {dt}")
    d = _inputs(T, N, K, dt, seed=7 * T + N, ints=True)
    tdt = torch_dtype(dt)
    X, dY = dev(d["X"]), dev(d["dY"])
    Xp, dYp, ws = _chunks(X), _chunks(dY), _split_ws(T, N, K)
    ms = dev_meta(d["ms"])
    a, b = empty((N, K // 2), torch.float32), empty((N, K // 2), torch.float32)
    ad = empty((N, K), torch.float32)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, a, ad, split_workspace=ws, in_dtype=tdt)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, b, in_dtype=tdt)
    torch.cuda.synchronize()
    v_ref, d_ref = oracle.masked_wgrad(d["dY"], d["X"], d["ms"], K)
    assert np.array_equal(host_f64(a), v_ref)
    assert np.array_equal(host_f64(ad), d_ref)
    assert torch.equal(a, b)
    # a 16-bit output rounds the same exact sum once: equal to the unsplit one
    h1, h2 = empty((N, K // 2), tdt), empty((N, K // 2), tdt)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, h1, split_workspace=ws, in_dtype=tdt)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, h2, in_dtype=tdt)
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))


def test_wgrad_split_not_needed_is_unchanged():
    """Where the tiles fill the device (or too few tokens to split) the query
    reports 0 and a given workspace changes nothing: bitwise the unsplit result."""
    T, N, K = 512, 4096, 4096
    assert S.slope_wgrad_split_workspace_bytes(T, N, K) == 0
    d = _inputs(T, N, K, "bf16", seed=3, ints=False)
    X, dY = dev(d["X"]), dev(d["dY"])
    Xp, dYp = _chunks(X), _chunks(dY)
    ms = dev_meta(d["ms"])
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    a, b = empty((N, K // 2), torch.bfloat16), empty((N, K // 2), torch.bfloat16)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, a, split_workspace=ws)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# Tail split: 17 x 16 = 272 output tiles on 256 compute units leave a last round
# of 16 tiles; with a split workspace those run in 4 token ranges (T = 1024: 32
# chunks, at least 8 per range), their fp32 sums added in range order.  The
# tail tiles are the last logical ids: k tiles 8..15 x n tiles 15..16 (rows
# 3840 .. 4351, columns 2048 .. 4095).
TAIL = (1024, 4352, 4096)


def _tail_rows(rng, N):
    rows = np.concatenate([rng.choice(np.arange(3840, N), size=24, replace=False),
                           rng.choice(np.arange(0, 3840), size=8, replace=False)])
    return np.sort(rows)


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_wgrad_tail_split_matches_oracle(out_dt):
    T, N, K = TAIL
    need = S.slope_wgrad_split_workspace_bytes(T, N, K)
    say(f"[wgrad tail split] T={T} N={N} K={K} out={out_dt} workspace={need}")
    assert need == 4 * 16 * 256 * 128 * 4
    d = _inputs(T, N, K, "bf16", seed=91, ints=False)
    X, dY = dev(d["X"]), dev(d["dY"])
    Xp, dYp, ws = _chunks(X), _chunks(dY), _split_ws(T, N, K)
    ms = dev_meta(d["ms"])
    tdt = torch_dtype(out_dt)
    dWv, dWd = empty((N, K // 2), tdt), empty((N, K), tdt)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, dWv, dWd, split_workspace=ws, in_dtype=torch.bfloat16)
    dWu = empty((N, K // 2), tdt)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, dWu, in_dtype=torch.bfloat16)
    base = torch.randn((N, K // 2), device="cuda").to(tdt)
    acc = base.clone()
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, acc, accumulate=True, split_workspace=ws,
                                in_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _tail_rows(np.random.default_rng(92), N)
    v_ref, d_ref = oracle.masked_wgrad(np.ascontiguousarray(d["dY"][:, rows]), d["X"], d["ms"][rows], K)
    got_v, got_d = host_f64(dWv)[rows], host_f64(dWd)[rows]
    assert normwise(got_v, v_ref) <= TOL["bf16"]
    assert normwise(got_d, d_ref) <= TOL["bf16"]
    assert (got_d[d["mask"][rows] == 0] == 0).all()
    assert normwise(host_f64(acc)[rows], v_ref + host_f64(base)[rows]) <= TOL["bf16"]
    # the whole matrix against the unsplit form: tiles of whole rounds bitwise, the tail's within the rounding
    a, b = host_f64(dWv), host_f64(dWu)
    assert np.array_equal(a[:3840], b[:3840]) and np.array_equal(a[:, :1024], b[:, :1024])
    assert normwise(a, b) <= (TOL["bf16"] if out_dt == "bf16" else 1e-5)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_wgrad_tail_split_integer_exact(dt):
    """Integer inputs: every partial sum is exact in fp32, so the tail split's
    fp32 output equals the unsplit one and the oracle bit for bit."""
    T, N, K = TAIL
    say(f"[wgrad tail split integer] T={T} N={N} K={K} {dt}")
    d = _inputs(T, N, K, dt, seed=93, ints=True)
    tdt = torch_dtype(dt)
    X, dY = dev(d["X"]), dev(d["dY"])
    Xp, dYp, ws = _chunks(X), _chunks(dY), _split_ws(T, N, K)
    ms = dev_meta(d["ms"])
    a, b = empty((N, K // 2), torch.float32), empty((N, K // 2), torch.float32)
    ad = empty((N, K), torch.float32)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, a, ad, split_workspace=ws, in_dtype=tdt)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, ms, b, in_dtype=tdt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    rows = _tail_rows(np.random.default_rng(94), N)
    v_ref, d_ref = oracle.masked_wgrad(np.ascontiguousarray(d["dY"][:, rows]), d["X"], d["ms"][rows], K)
    assert np.array_equal(host_f64(a)[rows], v_ref)
    assert np.array_equal(host_f64(ad)[rows], d_ref)
