"""GPU parity at oracle-friendly sizes: every entry point against the CPU oracle.

Masks, metadata, compressed values and the pruned weights must match bit for
bit; products must stay within the normwise tolerance (bf16 outputs 1e-2, fp32
path 1e-5, max |gpu - oracle| / max |oracle|), and integer-valued inputs whose
sums are exact must match bit for bit.  Sizes span several tiles of the fast
kernels (256 x 256 output tiles, 64-wide reduction stages) and ragged tails;
shapes whose rows are not 16-byte aligned exercise the generic kernels.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_02_amd as S
from workloads import f32_to_bf16_bits, layer_inputs

from gpu_util import (TOL, Compressed, dev, dev_meta, empty, host, host_f64, normwise, pack_sparse_reference, say,
                      torch_dtype, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()  # raises if the library was not built
    yield
    torch.cuda.synchronize()


def _bits(vals, dt):
    v = np.asarray(vals, dtype=np.float32)
    return f32_to_bf16_bits(v) if dt == "bf16" else v.view(np.uint32).copy()


def _special_matrix(rows, cols, dt, seed):
    """Ties, signed zeros, denormals, infinities and NaN mixed into Gaussian values."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32) * 0.02
    pick = rng.integers(0, 10, size=(rows, cols))
    v[pick == 0] = 0.0
    v[pick == 1] = -0.0
    v[pick == 2] = np.round(v[pick == 2] * 100) / 100          # many ties after rounding
    v[pick == 3] = -v[pick == 3]
    bits = _bits(v, dt)
    flat = bits.reshape(-1)
    n = flat.size
    idx = rng.choice(n, size=max(1, n // 50), replace=False)
    if dt == "bf16":
        specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x8003, 0x7F7F], dtype=np.uint16)
    else:
        specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x00000001, 0x80000005, 0x7F7FFFFF], dtype=np.uint32)
    flat[idx] = specials[rng.integers(0, len(specials), size=idx.size)]
    return bits


# ------------------------------------------------------------------ prune / compress / double prune

PRUNE_SHAPES = [(64, 256), (100, 68), (256, 1024), (7, 4), (33, 36)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", PRUNE_SHAPES)
def test_prune24_bit_exact(dt, rows, cols):
    say(f"prune24 {dt} {rows}x{cols}")
    W = _special_matrix(rows, cols, dt, rows * cols)
    mask_ref, Ws_ref = oracle.prune24(W)
    Wd = dev(W)
    mask = empty((rows, cols), torch.uint8)
    Ws = empty((rows, cols), torch_dtype(dt))
    S.slope_prune24(Wd, mask, Ws)
    torch.cuda.synchronize()
    assert (host(mask) == mask_ref).all()
    assert (host(Ws) == Ws_ref).all()
    # W_s is optional
    mask2 = empty((rows, cols), torch.uint8)
    S.slope_prune24(Wd, mask2)
    assert (host(mask2) == mask_ref).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", PRUNE_SHAPES)
def test_compress24_bit_exact(dt, rows, cols):
    say(f"compress24 {dt} {rows}x{cols}")
    W = _special_matrix(rows, cols, dt, 7 + rows)
    mask_ref, _ = oracle.prune24(W)
    vals_ref, meta_ref, inv_ref = oracle.compress24(W, mask_ref)
    c = Compressed(rows, cols, torch_dtype(dt))
    inv = torch.zeros(1, dtype=torch.int32, device="cuda")
    S.slope_compress24(dev(W), dev(mask_ref), c.values, c.meta, inv)
    torch.cuda.synchronize()
    assert (host(c.values) == vals_ref).all()
    assert (host(c.meta) == meta_ref).all()
    assert int(inv.item()) == inv_ref == 0


# ragged last metadata words (cols 68, 36, 4, 272), a partial last chunk
# column (272, 80) and whole chunks
FUSED_PRUNE_SHAPES = PRUNE_SHAPES + [(300, 272), (520, 1040), (2, 80)]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,cols", FUSED_PRUNE_SHAPES)
def test_prune_compress24_fused(dt, rows, cols):
    """One pass equals prune24 + compress24 (+ pack_sparse) of the oracle, bit
    for bit, with and without the optional mask and tile-chunk outputs."""
    say(f"prune_compress24 {dt} {rows}x{cols}")
    if dt == "f16":
        W = layer_inputs(cols, rows, 1, 1, "f16", seed=rows + cols, which=("W",))["W"]
    else:
        W = _special_matrix(rows, cols, dt, 3 * rows + cols)
    bits = lambda a: np.asarray(a).view(np.uint16) if np.asarray(a).dtype == np.float16 else np.asarray(a)
    mask_ref, _ = oracle.prune24(W)
    vals_ref, meta_ref, _ = oracle.compress24(W, mask_ref)
    c = Compressed(rows, cols, torch_dtype(dt))
    mask = torch.full((rows, cols), 7, dtype=torch.uint8, device="cuda")
    pk = None
    if dt != "f32" and cols % 16 == 0:
        pk = torch.full((S.slope_packed_sparse_bytes(rows, cols),), 0x5A, dtype=torch.uint8, device="cuda")
    S.slope_prune_compress24(dev(W), c.values, c.meta, mask=mask, packed=pk)
    torch.cuda.synchronize()
    assert (host(mask) == mask_ref).all()
    assert (bits(host(c.values)) == bits(vals_ref)).all()
    assert (host(c.meta) == meta_ref).all()
    if pk is not None:
        assert np.array_equal(pk.cpu().numpy(), pack_sparse_reference(bits(vals_ref), meta_ref, rows, cols))
    c2 = Compressed(rows, cols, torch_dtype(dt))
    S.slope_prune_compress24(dev(W), c2.values, c2.meta)
    torch.cuda.synchronize()
    assert (bits(host(c2.values)) == bits(vals_ref)).all() and (host(c2.meta) == meta_ref).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_compress24_user_masks(dt):
    say(f"compress24 user masks {dt}")
    rng = np.random.default_rng(11)
    rows, cols = 40, 100
    W = _bits(rng.standard_normal((rows, cols)), dt)
    mask = (rng.integers(0, 4, size=(rows, cols)) == 0).astype(np.uint8) * rng.integers(1, 255, size=(rows, cols)).astype(np.uint8)
    mask[0, :8] = [1, 1, 1, 1, 0, 0, 0, 0]   # four kept, then none
    vals_ref, meta_ref, inv_ref = oracle.compress24(W, mask)
    assert inv_ref > 0
    c = Compressed(rows, cols, torch_dtype(dt))
    inv = torch.zeros(1, dtype=torch.int32, device="cuda")
    S.slope_compress24(dev(W), dev(mask), c.values, c.meta, inv)
    torch.cuda.synchronize()
    assert (host(c.values) == vals_ref).all()
    assert (host(c.meta) == meta_ref).all()
    assert int(inv.item()) == inv_ref


DP_SHAPES = [(64, 128), (100, 68), (256, 384), (36, 260), (4, 4), (520, 132),
             (144, 272), (400, 528), (16, 16), (1040, 144), (1024, 2048)]  # last five: 16-aligned kernel


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("N,K", DP_SHAPES)
def test_double_prune_bit_exact(dt, N, K):
    say(f"double_prune {dt} N={N} K={K}")
    W = _special_matrix(N, K, dt, N + K)
    mask_s, _ = oracle.prune24(W)
    vs, ms, _ = oracle.compress24(W, mask_s)
    v_ref, m_ref, mask_ref = oracle.double_prune(vs, ms, N, K)
    out = Compressed(K, N, torch_dtype(dt))
    mask = empty((K, N), torch.uint8)
    S.slope_double_prune(dev(vs), dev_meta(ms), N, K, out.values, out.meta, mask)
    torch.cuda.synchronize()
    assert (host(out.values) == v_ref).all()
    assert (host(out.meta) == m_ref).all()
    assert (host(mask) == mask_ref).all()
    out2 = Compressed(K, N, torch_dtype(dt))
    S.slope_double_prune(dev(vs), dev_meta(ms), N, K, out2.values, out2.meta)
    assert (host(out2.meta) == m_ref).all()


def test_chain_prune_compress_double_prune_on_device():
    say("chain prune -> compress -> double prune")
    N, K = 300, 520
    W = _special_matrix(N, K, "bf16", 99)
    mask_s, _ = oracle.prune24(W)
    vs, ms, _ = oracle.compress24(W, mask_s)
    v_ref, m_ref, _ = oracle.double_prune(vs, ms, N, K)
    Wd = dev(W)
    mask = empty((N, K), torch.uint8)
    S.slope_prune24(Wd, mask)
    c = Compressed(N, K, torch.bfloat16)
    S.slope_compress24(Wd, mask, c.values, c.meta)
    out = Compressed(K, N, torch.bfloat16)
    S.slope_double_prune(c.values, c.meta, N, K, out.values, out.meta)
    torch.cuda.synchronize()
    assert (host(out.values) == v_ref).all() and (host(out.meta) == m_ref).all()


# ------------------------------------------------------------------ products

def _layer(T, N, K, r, dt, seed, ints=False):
    if ints:
        rng = np.random.default_rng(seed)
        mk = lambda *s: _bits(rng.integers(-3, 4, size=s), dt)
        d = {"W": mk(N, K), "X": mk(T, K), "dY": mk(T, N), "L": mk(K, r), "R": mk(r, N)}
    else:
        d = layer_inputs(K, N, T, r, dt, seed=seed)
    mask_s, W_s = oracle.prune24(d["W"])
    vs, ms, _ = oracle.compress24(d["W"], mask_s)
    vdp = mdp = None
    if N % 4 == 0:  # double pruning groups along N
        vdp, mdp, _ = oracle.double_prune(vs, ms, N, K)
    d.update(mask_s=mask_s, vs=vs, ms=ms, vdp=vdp, mdp=mdp)
    return d


# (T, N, K): several 256-wide output tiles, 64-wide stages, ragged tails;
# K % 16 != 0 or N % 4 != 0 route to the generic kernels.
GEMM_SHAPES = [(64, 256, 256), (300, 520, 272), (512, 768, 1024), (37, 100, 68), (1, 64, 128), (130, 36, 4),
               (257, 260, 528), (50, 102, 64)]


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("adapter", [False, True])
@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
def test_spmm_fwd(T, N, K, adapter, out_dt):
    say(f"spmm_fwd T={T} N={N} K={K} adapter={adapter} out={out_dt}")
    r = 8 if adapter else 0
    d = _layer(T, N, K, max(r, 1), "bf16", seed=T + N + K)
    L, R = (d["L"][:, :r], d["R"][:r]) if adapter else (None, None)
    ref = oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, L, R)
    Y = empty((T, N), torch_dtype(out_dt))
    S.slope_spmm_fwd(dev(d["X"]), dev(d["vs"]), dev_meta(d["ms"]), N, Y,
                     L=dev(np.ascontiguousarray(L)) if adapter else None,
                     R=dev(np.ascontiguousarray(R)) if adapter else None,
                     workspace=workspace(T, K, r, N) if adapter else None)
    torch.cuda.synchronize()
    err = normwise(host_f64(Y), ref)
    assert err <= TOL["bf16"], err
    if out_dt == "f32":  # fp32 output keeps the fp32 accumulation: much tighter
        assert err <= 2e-5 * max(1.0, np.sqrt(K / 256)), err


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
def test_spmm_bwd_dx(T, N, K, out_dt):
    if N % 4:
        pytest.skip("double pruning needs N % 4 == 0")
    say(f"spmm_bwd_dx T={T} N={N} K={K} out={out_dt}")
    d = _layer(T, N, K, 1, "bf16", seed=3 * T + N + K)
    ref = oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N)
    dX = empty((T, K), torch_dtype(out_dt))
    S.slope_spmm_bwd_dx(dev(d["dY"]), dev(d["vdp"]), dev_meta(d["mdp"]), K, dX)
    torch.cuda.synchronize()
    err = normwise(host_f64(dX), ref)
    assert err <= TOL["bf16"], err


# ------------------------------------------------------------------ packed sparse operands (tile chunks)

@pytest.mark.parametrize("rows,cols", [(256, 64), (300, 272), (4, 16), (520, 1040)])
def test_pack_sparse_layout(rows, cols):
    say(f"pack_sparse rows={rows} cols={cols}")
    W = _special_matrix(rows, cols, "bf16", rows + cols)
    mask, _ = oracle.prune24(W)
    vs, ms, _ = oracle.compress24(W, mask)
    packed = torch.empty(S.slope_packed_sparse_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    packed.fill_(0xCD)
    S.slope_pack_sparse(dev(vs), dev_meta(ms), rows, cols, packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), pack_sparse_reference(vs, ms, rows, cols))


PACKED_SHAPES = [(64, 256, 256), (300, 528, 272), (512, 768, 1024), (1, 64, 128), (257, 272, 528), (0, 64, 64),
                 (700, 1040, 1296)]


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("adapter", [False, True])
@pytest.mark.parametrize("T,N,K", PACKED_SHAPES)
def test_spmm_packed_matches_unpacked(T, N, K, adapter, out_dt):
    """The packed products read the same values in the same order: bitwise
    equal to the unpacked ones, and within tolerance of the oracle."""
    say(f"spmm packed T={T} N={N} K={K} adapter={adapter} out={out_dt}")
    r = 8 if adapter else 0
    d = _layer(T, N, K, max(r, 1), "bf16", seed=7 * T + N + K)
    L = dev(np.ascontiguousarray(d["L"][:, :r])) if adapter else None
    R = dev(np.ascontiguousarray(d["R"][:r])) if adapter else None
    ws = workspace(T, K, r, N) if adapter else None
    od = torch_dtype(out_dt)
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vs"]), dev_meta(d["ms"]), N, K, ps)
    Yp, Yu = empty((T, N), od), empty((T, N), od)
    S.slope_spmm_fwd_packed(dev(d["X"]), ps, N, Yp, L=L, R=R, workspace=ws)
    S.slope_spmm_fwd(dev(d["X"]), dev(d["vs"]), dev_meta(d["ms"]), N, Yu, L=L, R=R, workspace=ws)
    pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vdp"]), dev_meta(d["mdp"]), K, N, pd)
    dXp, dXu = empty((T, K), od), empty((T, K), od)
    S.slope_spmm_bwd_dx_packed(dev(d["dY"]), pd, K, dXp)
    S.slope_spmm_bwd_dx(dev(d["dY"]), dev(d["vdp"]), dev_meta(d["mdp"]), K, dXu)
    torch.cuda.synchronize()
    assert np.array_equal(host(Yp), host(Yu))
    assert np.array_equal(host(dXp), host(dXu))
    if T:
        ref = oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"][:, :r] if adapter else None,
                              d["R"][:r] if adapter else None)
        assert normwise(host_f64(Yp), ref) <= TOL["bf16"]
        assert normwise(host_f64(dXp), oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N)) <= TOL["bf16"]


# Token counts near 8192 with 256-row output tiles: on a 256-CU device the
# sparse products run (T, M) = (8142, 2000) in full-width tiles only (one full
# round), (8142, 2224) as eight rows of full-width tiles plus one row of
# half-width tiles, and M = 96 in half-width tiles only; M is N for the
# forward and K for dX.  Rows, tokens and the reduction (96 = 1.5 stages) are
# ragged.
SPLIT_SHAPES = [(8142, 2000, 96), (8142, 96, 2000), (8142, 2224, 96), (8142, 96, 2224)]


@pytest.mark.parametrize("r", [8, 100, 128])
@pytest.mark.parametrize("ints", [False, True], ids=["normal", "integer"])
@pytest.mark.parametrize("T,N,K", SPLIT_SHAPES)
def test_spmm_tile_split(T, N, K, ints, r):
    """Forward with the adapter and dX with the adapter's dX term, packed and
    unpacked, whichever mix of tile widths the launch takes: within tolerance
    of the oracle, and bit-exact in fp32 for integer inputs (every sum exact).
    Ranks above 96 take the epilogue's rank slices through LDS in two chunks
    on the 256-token tiles (six slices fit) and, at 128, on the 128-token tiles."""
    say(f"spmm tile split T={T} N={N} K={K} ints={ints} r={r}")
    d = _layer(T, N, K, r, "bf16", seed=29 * T + N + K, ints=ints)
    od = torch.float32 if ints else torch.bfloat16
    L, R = dev(d["L"]), dev(d["R"])
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vs"]), dev_meta(d["ms"]), N, K, ps)
    pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vdp"]), dev_meta(d["mdp"]), K, N, pd)
    Yp, Yu, dXp = empty((T, N), od), empty((T, N), od), empty((T, K), od)
    S.slope_spmm_fwd_packed(dev(d["X"]), ps, N, Yp, L=L, R=R, workspace=workspace(T, K, r, N))
    S.slope_spmm_fwd(dev(d["X"]), dev(d["vs"]), dev_meta(d["ms"]), N, Yu, L=L, R=R, workspace=workspace(T, K, r, N))
    S.slope_spmm_bwd_dx_packed(dev(d["dY"]), pd, K, dXp, L=L, R=R, workspace=workspace(T, N, r, K))
    torch.cuda.synchronize()
    ref_y = oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"], d["R"])
    ref_dx = oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N) + oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])[0]
    assert np.array_equal(host(Yp), host(Yu))
    if ints:
        assert np.array_equal(host_f64(Yp), ref_y)
        assert np.array_equal(host_f64(dXp), ref_dx)
    else:
        assert normwise(host_f64(Yp), ref_y) <= TOL["bf16"]
        assert normwise(host_f64(dXp), ref_dx) <= TOL["bf16"]


DECODE_SHAPES = [(1, 256, 256), (5, 520, 272), (16, 768, 1024), (33, 260, 528), (64, 1040, 1296), (0, 64, 64),
                 (3, 64, 4096)]


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("adapter", [False, True])
@pytest.mark.parametrize("T,N,K", DECODE_SHAPES)
def test_spmm_fwd_decode(T, N, K, adapter, out_dt):
    say(f"spmm_fwd_decode T={T} N={N} K={K} adapter={adapter} out={out_dt}")
    r = 8 if adapter else 0
    d = _layer(T, N, K, max(r, 1), "bf16", seed=11 * T + N + K)
    L = dev(np.ascontiguousarray(d["L"][:, :r])) if adapter else None
    R = dev(np.ascontiguousarray(d["R"][:r])) if adapter else None
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vs"]), dev_meta(d["ms"]), N, K, ps)
    ws = torch.empty(max(16, S.slope_decode_workspace_bytes(T, K, r, N)), dtype=torch.uint8, device="cuda")
    Y = empty((T, N), torch_dtype(out_dt))
    S.slope_spmm_fwd_decode(dev(d["X"]), ps, N, Y, ws, L=L, R=R)
    Y2 = empty((T, N), torch_dtype(out_dt))
    S.slope_spmm_fwd_decode(dev(d["X"]), ps, N, Y2, ws, L=L, R=R)
    torch.cuda.synchronize()
    assert np.array_equal(host(Y), host(Y2))          # fixed reduction order
    if T:
        ref = oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"][:, :r] if adapter else None,
                              d["R"][:r] if adapter else None)
        err = normwise(host_f64(Y), ref)
        assert err <= TOL["bf16"], err
        if out_dt == "f32":
            assert err <= 2e-5 * max(1.0, np.sqrt(K / 256)), err


@pytest.mark.parametrize("T,N,K,r", [(1, 256, 9216, 72), (4, 520, 1040, 128), (2, 64, 131072, 33), (1, 64, 16, 1),
                                     (3, 272, 4112, 17), (40, 520, 1040, 128), (17, 264, 4112, 33),
                                     (64, 136, 2064, 100)])
def test_spmm_fwd_decode_adapter_ranks(T, N, K, r):
    """Few tokens with the adapter: ranks up to 128, long reductions, ragged
    sizes; above four tokens token spans that end inside a wave's tokens."""
    say(f"spmm_fwd_decode adapter T={T} N={N} K={K} r={r}")
    d = _layer(T, N, K, r, "bf16", seed=5 * T + N + K + r)
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vs"]), dev_meta(d["ms"]), N, K, ps)
    ws = torch.empty(S.slope_decode_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    Y = empty((T, N), torch.float32)
    S.slope_spmm_fwd_decode(dev(d["X"]), ps, N, Y, ws, L=dev(d["L"]), R=dev(d["R"]))
    torch.cuda.synchronize()
    ref = oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"], d["R"])
    assert normwise(host_f64(Y), ref) <= 2e-5 * max(1.0, np.sqrt(K / 256))


@pytest.mark.parametrize("T,K", [(3, 1040), (7, 1040), (40, 1040), (40, 8224)])
def test_spmm_fwd_decode_integer_exact(T, K):
    """Integer inputs: every partial sum is exact, so fp32 output equals the
    oracle (K = 8224: a longer reduction, X . L over all of it)."""
    N, r = 520, 4
    say(f"decode integer probe T={T} K={K}")
    d = _layer(T, N, K, r, "bf16", seed=23, ints=True)
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vs"]), dev_meta(d["ms"]), N, K, ps)
    ws = torch.empty(S.slope_decode_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    Y = empty((T, N), torch.float32)
    S.slope_spmm_fwd_decode(dev(d["X"]), ps, N, Y, ws, L=dev(d["L"]), R=dev(d["R"]))
    torch.cuda.synchronize()
    assert np.array_equal(host_f64(Y), oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"], d["R"]))


# ------------------------------------------------------------------ adapter backward

ADAPTER_BWD_SHAPES = [(64, 256, 256, 8), (300, 528, 272, 40), (37, 64, 136, 72), (512, 768, 1024, 128),
                      (1, 64, 64, 1), (130, 272, 520, 33), (96, 256, 512, 24), (200, 512, 256, 96)]


def _chunks(M):
    T, C = M.shape
    p = torch.empty(S.slope_packed_tokens_bytes(T, C), dtype=torch.uint8, device="cuda")
    S.slope_pack_tokens(M, p)
    return p


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K,r", ADAPTER_BWD_SHAPES)
def test_spmm_bwd_dx_packed_with_adapter(T, N, K, r, out_dt):
    say(f"bwd dX + adapter T={T} N={N} K={K} r={r} out={out_dt}")
    d = _layer(T, N, K, r, "bf16", seed=13 * T + N + K + r)
    pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vdp"]), dev_meta(d["mdp"]), K, N, pd)
    ws = torch.empty(max(16, S.slope_lowrank_workspace_bytes(T, N, r, K)), dtype=torch.uint8, device="cuda")
    dX = empty((T, K), torch_dtype(out_dt))
    S.slope_spmm_bwd_dx_packed(dev(d["dY"]), pd, K, dX, L=dev(d["L"]), R=dev(d["R"]), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N) + oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])[0]
    err = normwise(host_f64(dX), ref)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K,r", ADAPTER_BWD_SHAPES + [(0, 64, 64, 8)])
def test_lowrank_grads_packed(T, N, K, r, out_dt):
    say(f"adapter grads T={T} N={N} K={K} r={r} out={out_dt}")
    d = _layer(T, N, K, r, "bf16", seed=17 * T + N + K + r)
    X, dY, L, R = dev(d["X"]), dev(d["dY"]), dev(d["L"]), dev(d["R"])
    ws = torch.empty(max(16, S.slope_lowrank_grads_workspace_bytes(T, K, r, N)), dtype=torch.uint8, device="cuda")
    od = torch_dtype(out_dt)
    dL, dR = empty((K, r), od), empty((r, N), od)
    S.slope_lowrank_grads_packed(X, dY, _chunks(X), _chunks(dY), L, R, ws, dL, dR)
    dL2, dR2 = empty((K, r), od), empty((r, N), od)
    S.slope_lowrank_grads_packed(X, dY, _chunks(X), _chunks(dY), L, R, ws, dL2, dR2)
    torch.cuda.synchronize()
    assert np.array_equal(host(dL), host(dL2)) and np.array_equal(host(dR), host(dR2))   # fixed order
    _, dL_ref, dR_ref = oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])
    assert normwise(host_f64(dL), dL_ref) <= TOL["bf16"]
    assert normwise(host_f64(dR), dR_ref) <= TOL["bf16"]
    # accumulation adds to what is there
    bL = torch.randn((K, r), device="cuda").to(od)
    bR = torch.randn((r, N), device="cuda").to(od)
    aL, aR = bL.clone(), bR.clone()
    S.slope_lowrank_grads_packed(X, dY, _chunks(X), _chunks(dY), L, R, ws, aL, aR, accumulate=True)
    torch.cuda.synchronize()
    assert normwise(host_f64(aL), dL_ref + host_f64(bL)) <= TOL["bf16"]
    assert normwise(host_f64(aR), dR_ref + host_f64(bR)) <= TOL["bf16"]


@pytest.mark.parametrize("T,N,K,r", [(300, 528, 272, 40), (64, 256, 256, 8)])
def test_lowrank_grads_reuse_workspaces(T, N, K, r):
    """Handing over the forward's and the dX product's adapter workspaces skips
    recomputing X . L and dY . R^T; the gradients are bitwise the same."""
    say(f"adapter grads with reused workspaces T={T} N={N} K={K} r={r}")
    d = _layer(T, N, K, r, "bf16", seed=31 * T + r)
    X, dY, L, R = dev(d["X"]), dev(d["dY"]), dev(d["L"]), dev(d["R"])
    ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vs"]), dev_meta(d["ms"]), N, K, ps)
    pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vdp"]), dev_meta(d["mdp"]), K, N, pd)
    wf = torch.empty(S.slope_lowrank_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    wb = torch.empty(S.slope_lowrank_workspace_bytes(T, N, r, K), dtype=torch.uint8, device="cuda")
    S.slope_spmm_fwd_packed(X, ps, N, empty((T, N), torch.bfloat16), L=L, R=R, workspace=wf)
    S.slope_spmm_bwd_dx_packed(dY, pd, K, empty((T, K), torch.bfloat16), L=L, R=R, workspace=wb)
    ws = torch.empty(S.slope_lowrank_grads_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    out = []
    for reuse in (False, True):
        dL, dR = empty((K, r), torch.bfloat16), empty((r, N), torch.bfloat16)
        S.slope_lowrank_grads_packed(X, dY, _chunks(X), _chunks(dY), L, R, ws, dL, dR,
                                     fwd_workspace=wf if reuse else None, bwd_workspace=wb if reuse else None)
        torch.cuda.synchronize()
        out.append((host(dL), host(dR)))
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])


def test_adapter_backward_integer_exact():
    """Integer inputs: X . L and dY . R^T are exact in the hi/lo pair, every
    product and sum is exact in fp32, so fp32 outputs equal the oracle."""
    T, N, K, r = 70, 272, 528, 12
    say("adapter backward integer probe")
    d = _layer(T, N, K, r, "bf16", seed=29, ints=True)
    X, dY, L, R = dev(d["X"]), dev(d["dY"]), dev(d["L"]), dev(d["R"])
    ws = torch.empty(S.slope_lowrank_grads_workspace_bytes(T, K, r, N), dtype=torch.uint8, device="cuda")
    dL, dR = empty((K, r), torch.float32), empty((r, N), torch.float32)
    S.slope_lowrank_grads_packed(X, dY, _chunks(X), _chunks(dY), L, R, ws, dL, dR)
    pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_sparse(dev(d["vdp"]), dev_meta(d["mdp"]), K, N, pd)
    wsx = torch.empty(S.slope_lowrank_workspace_bytes(T, N, r, K), dtype=torch.uint8, device="cuda")
    dX = empty((T, K), torch.float32)
    S.slope_spmm_bwd_dx_packed(dY, pd, K, dX, L=L, R=R, workspace=wsx)
    torch.cuda.synchronize()
    dXa, dL_ref, dR_ref = oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])
    assert np.array_equal(host_f64(dL), dL_ref)
    assert np.array_equal(host_f64(dR), dR_ref)
    assert np.array_equal(host_f64(dX), oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N) + dXa)


WGRAD_SHAPES = [(64, 256, 256), (300, 520, 272), (512, 768, 1024), (37, 100, 68), (1, 64, 128), (130, 36, 4),
                (0, 64, 64), (257, 264, 520), (288, 256, 512), (416, 776, 264)]


def wgrad_ws(T, N, K):
    return torch.empty(max(16, S.slope_wgrad_workspace_bytes(T, N, K)), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("packed", [False, True], ids=["direct", "packed"])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K", WGRAD_SHAPES)
def test_masked_wgrad(T, N, K, out_dt, packed):
    say(f"masked_wgrad T={T} N={N} K={K} out={out_dt} packed={packed}")
    d = _layer(T, N, K, 1, "bf16", seed=5 * T + N + K)
    v_ref, d_ref = oracle.masked_wgrad(d["dY"], d["X"], d["ms"], K)
    ws = wgrad_ws(T, N, K) if packed else None
    dWv = empty((N, K // 2), torch_dtype(out_dt))
    dWd = empty((N, K), torch_dtype(out_dt))
    S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dWv, dWd, workspace=ws)
    torch.cuda.synchronize()
    assert normwise(host_f64(dWv), v_ref) <= TOL["bf16"]
    assert normwise(host_f64(dWd), d_ref) <= TOL["bf16"]
    assert (host_f64(dWd)[d["mask_s"] == 0] == 0).all()
    # accumulation adds to what is there
    base = torch.randn((N, K // 2), device="cuda").to(torch_dtype(out_dt))
    acc = base.clone()
    S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), acc, accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    assert normwise(host_f64(acc), v_ref + host_f64(base)) <= TOL["bf16"]


# (70, 8136, 2000) and (70, 8136, 2224): 256 and 288 output tiles, a whole
# round of blocks and a partly filled second one, ragged in k and n.  The
# token-chunk counts 3, 5, 9 and 13 sit on either side of the packed kernel's
# four-stage register ring and eight-stage X ring (its loop runs whole groups
# of four stages, the extra ones reading zeros).
@pytest.mark.parametrize("T,N,K", [(300, 520, 272), (257, 264, 520), (1, 64, 128), (2048, 512, 768), (32, 8, 1032),
                                   (64, 256, 1032), (97, 264, 776), (70, 8136, 2000), (70, 8136, 2224),
                                   (96, 264, 520), (160, 520, 272), (288, 256, 512), (416, 776, 264)])
def test_masked_wgrad_packed_matches_direct(T, N, K):
    """Both kernels feed the same operands to the same MFMA positions in the
    same token order, so with and without the workspace results are bitwise equal."""
    say(f"masked_wgrad packed==direct T={T} N={N} K={K}")
    d = _layer(T, N, K, 1, "bf16", seed=11 * T + N + K)
    out = []
    for ws in (None, wgrad_ws(T, N, K)):
        dWv = empty((N, K // 2), torch.bfloat16)
        S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dWv, workspace=ws)
        torch.cuda.synchronize()
        out.append(host(dWv))
    assert np.array_equal(out[0], out[1])


def _pack_reference(bits, T, C):
    """The token-chunk layout as include/slope.h states it, built with numpy."""
    Tch, Cch = -(-T // 32), -(-C // 256)
    pad = np.zeros((Tch * 32, Cch * 256), dtype=np.uint16)
    pad[:T, :C] = bits
    out = np.zeros((Cch, Tch, 256, 4, 8), dtype=np.uint16)
    for c in range(Cch):
        for s in range(Tch):
            blk = pad[32 * s:32 * s + 32, 256 * c:256 * c + 256].T.reshape(256, 4, 8)   # [row][granule][token]
            for row in range(256):
                for g in range(4):
                    out[c, s, row, g ^ ((row >> 2) & 3)] = blk[row, g]
    return out.reshape(-1)


@pytest.mark.parametrize("T,C", [(32, 256), (70, 264), (1, 8), (257, 520)])
def test_pack_tokens_layout(T, C):
    say(f"pack_tokens T={T} C={C}")
    rng = np.random.default_rng(T * 1000 + C)
    bits = rng.integers(0, 1 << 16, size=(T, C), dtype=np.uint16)
    packed = torch.empty(S.slope_packed_tokens_bytes(T, C), dtype=torch.uint8, device="cuda")
    packed.fill_(0xAB)
    S.slope_pack_tokens(dev(bits), packed)
    torch.cuda.synchronize()
    got = packed.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _pack_reference(bits, T, C))


@pytest.mark.parametrize("T,N,K", [(300, 520, 272), (33, 8, 1032)])
def test_masked_wgrad_packed_entry(T, N, K):
    """Packing by hand and calling the packed GEMM equals the one-call form."""
    say(f"masked_wgrad_packed T={T} N={N} K={K}")
    d = _layer(T, N, K, 1, "bf16", seed=T + 7 * K)
    Xd, dYd = dev(d["X"]), dev(d["dY"])
    Xp = torch.empty(S.slope_packed_tokens_bytes(T, K), dtype=torch.uint8, device="cuda")
    dYp = torch.empty(S.slope_packed_tokens_bytes(T, N), dtype=torch.uint8, device="cuda")
    S.slope_pack_tokens(Xd, Xp)
    S.slope_pack_tokens(dYd, dYp)
    a = empty((N, K // 2), torch.bfloat16)
    dd = empty((N, K), torch.bfloat16)
    S.slope_masked_wgrad_packed(dYp, Xp, T, N, K, dev_meta(d["ms"]), a, dd)
    b = empty((N, K // 2), torch.bfloat16)
    S.slope_masked_wgrad(dYd, Xd, dev_meta(d["ms"]), b)
    torch.cuda.synchronize()
    assert np.array_equal(host(a), host(b))
    v_ref, d_ref = oracle.masked_wgrad(d["dY"], d["X"], d["ms"], K)
    assert normwise(host_f64(a), v_ref) <= TOL["bf16"]
    assert normwise(host_f64(dd), d_ref) <= TOL["bf16"]


def test_masked_wgrad_short_workspace():
    T, N, K = 64, 256, 256
    d = _layer(T, N, K, 1, "bf16", seed=1)
    dWv = empty((N, K // 2), torch.bfloat16)
    short = torch.empty(S.slope_wgrad_workspace_bytes(T, N, K) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(S.SlopeError):
        S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dWv, workspace=short)


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K,r", [(64, 256, 256, 8), (300, 520, 272, 72), (37, 100, 68, 5), (513, 260, 1024, 40),
                                     (8, 64, 64, 130)])
def test_lowrank_add(T, N, K, r, out_dt):
    say(f"lowrank_add T={T} N={N} K={K} r={r} out={out_dt}")
    d = layer_inputs(K, N, T, r, "bf16", seed=T + r)
    Y0 = torch.randn((T, N), device="cuda").to(torch_dtype(out_dt))
    y0_bits = host(Y0)
    _, ref = oracle.lowrank_add(d["X"], d["L"], d["R"], Y_in=y0_bits)
    Y = Y0.clone()
    S.slope_lowrank_add(dev(d["X"]), dev(d["L"]), dev(d["R"]), workspace(T, K, r, N), Y)
    torch.cuda.synchronize()
    assert normwise(host_f64(Y), ref) <= TOL["bf16"]


# ------------------------------------------------------------------ fp32 path (toy workload precision)

@pytest.mark.parametrize("T,N,K", [(64, 256, 256), (37, 100, 68)])
def test_fp32_path(T, N, K):
    say(f"fp32 path T={T} N={N} K={K}")
    r = 8
    d = _layer(T, N, K, r, "f32", seed=T * N)
    Y = empty((T, N), torch.float32)
    S.slope_spmm_fwd(dev(d["X"]), dev(d["vs"]), dev_meta(d["ms"]), N, Y, L=dev(d["L"]), R=dev(d["R"]),
                     workspace=workspace(T, K, r, N))
    dX = empty((T, K), torch.float32)
    S.slope_spmm_bwd_dx(dev(d["dY"]), dev(d["vdp"]), dev_meta(d["mdp"]), K, dX)
    dWv = empty((N, K // 2), torch.float32)
    S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dWv)
    torch.cuda.synchronize()
    assert normwise(host_f64(Y), oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"], d["R"])) <= TOL["f32"]
    assert normwise(host_f64(dX), oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N)) <= TOL["f32"]
    assert normwise(host_f64(dWv), oracle.masked_wgrad(d["dY"], d["X"], d["ms"], K)[0]) <= TOL["f32"]


# ------------------------------------------------------------------ exact integer probes

@pytest.mark.parametrize("T,N,K", [(300, 520, 512), (64, 256, 256), (37, 100, 68)])
def test_integer_inputs_bit_exact(T, N, K):
    """Integers in [-3, 3]: every product and partial sum is exact in fp32, so
    fp32 outputs must equal the oracle exactly (pins orientation and slots)."""
    say(f"integer probe T={T} N={N} K={K}")
    r = 4
    d = _layer(T, N, K, r, "bf16", seed=17, ints=True)
    Y = empty((T, N), torch.float32)
    S.slope_spmm_fwd(dev(d["X"]), dev(d["vs"]), dev_meta(d["ms"]), N, Y, L=dev(d["L"]), R=dev(d["R"]),
                     workspace=workspace(T, K, r, N))
    dX = empty((T, K), torch.float32)
    S.slope_spmm_bwd_dx(dev(d["dY"]), dev(d["vdp"]), dev_meta(d["mdp"]), K, dX)
    dWv = empty((N, K // 2), torch.float32)
    S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dWv)
    dWp = empty((N, K // 2), torch.float32)
    S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dWp, workspace=wgrad_ws(T, N, K))
    torch.cuda.synchronize()
    assert np.array_equal(host_f64(Y), oracle.spmm_fwd(d["X"], d["vs"], d["ms"], K, d["L"], d["R"]))
    assert np.array_equal(host_f64(dX), oracle.spmm_bwd_dx(d["dY"], d["vdp"], d["mdp"], N))
    dw_ref = oracle.masked_wgrad(d["dY"], d["X"], d["ms"], K)[0]
    assert np.array_equal(host_f64(dWv), dw_ref)
    assert np.array_equal(host_f64(dWp), dw_ref)


def test_empty_and_degenerate():
    say("empty and degenerate sizes")
    # T = 0: nothing written, no error
    X = empty((0, 64), torch.bfloat16)
    c = Compressed(32, 64, torch.bfloat16)
    Y = empty((0, 32), torch.bfloat16)
    S.slope_spmm_fwd(X, c.values, c.meta, 32, Y)
    # K = 0: Y is the empty sum, 0
    Y = torch.full((5, 8), 7.0, device="cuda", dtype=torch.bfloat16)
    S.slope_spmm_fwd(empty((5, 0), torch.bfloat16), empty((8, 0), torch.bfloat16),
                     torch.empty((8, 0), dtype=torch.int32, device="cuda"), 8, Y)
    torch.cuda.synchronize()
    assert (Y.float() == 0).all()
    # rows = 0 prune / compress
    S.slope_prune24(empty((0, 8), torch.bfloat16), empty((0, 8), torch.uint8))
    # an all-zero weight keeps positions 0 and 1 of every group (ties to the lower index)
    W = torch.zeros((8, 16), device="cuda", dtype=torch.bfloat16)
    mask = empty((8, 16), torch.uint8)
    S.slope_prune24(W, mask)
    torch.cuda.synchronize()
    assert (mask.view(8, 4, 4).cpu() == torch.tensor([1, 1, 0, 0], dtype=torch.uint8)).all()


def test_deterministic_repeat():
    say("bitwise determinism")
    T, N, K, r = 300, 520, 528, 16
    d = _layer(T, N, K, r, "bf16", seed=1)
    args = (dev(d["X"]), dev(d["vs"]), dev_meta(d["ms"]), N)
    outs = []
    for _ in range(2):
        Y = empty((T, N), torch.bfloat16)
        S.slope_spmm_fwd(*args, Y, L=dev(d["L"]), R=dev(d["R"]), workspace=workspace(T, K, r, N))
        dW = empty((N, K // 2), torch.bfloat16)
        S.slope_masked_wgrad(dev(d["dY"]), dev(d["X"]), dev_meta(d["ms"]), dW)
        torch.cuda.synchronize()
        outs.append((host(Y), host(dW)))
    assert all((a == b).all() for a, b in zip(outs[0], outs[1]))


def test_single_hip_runtime_loaded():
    """torch's HIP runtime and the library's must be the same mapped object."""
    import re
    maps = open("/proc/self/maps").read()
    libs = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(libs) == 1, libs
