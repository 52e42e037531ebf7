"""Pins of the oracle's 8-bit (E4M3) variant.

The format is pinned against PyTorch's float8_e4m3fn (an independent library
implementation of the same OCP FP8 E4M3 format) and against the format's
published constants; the rounding against a brute-force nearest-neighbour
search over the codes with ties to even; the scaled product against the
16-bit oracle product, which it must equal exactly when the scales are powers
of two and every input is representable (no quantization error).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import f32_to_bf16_bits


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().double().numpy()


def _torch_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_and_the_format_constants():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.decode_e4m3(codes), _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2        # 0x7F, 0xFF only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))  # -0 at 0x80
    # published constants: largest normal S.1111.110 = 448, smallest normal 2^-6,
    # smallest subnormal 2^-9, one at exponent field 7
    assert oracle.decode_e4m3(np.array([0x7E, 0x08, 0x01, 0x38, 0xFE], np.uint8)).tolist() == \
        [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -448.0]
    pos = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()                                        # codes ordered by value


def _midpoints():
    pos = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    return (pos[:-1] + pos[1:]) / 2


def test_round_is_nearest_ties_to_even():
    rng = np.random.default_rng(31)
    mids = _midpoints()
    x = np.concatenate([rng.normal(size=20000) * 2.0 ** rng.integers(-12, 9, size=20000),
                        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                        rng.uniform(-448, 448, size=5000)])
    x = x[np.abs(x) <= 448]
    q = oracle.round_e4m3(x)
    got = oracle.decode_e4m3(q)
    err = np.abs(x - got)
    # brute force: the codes one step below and above the result (same sign) are not nearer
    mag = q & 0x7F
    for step in (-1, 1):
        nb = mag.astype(np.int64) + step
        ok = (nb >= 0) & (nb <= 0x7E)
        alt = oracle.decode_e4m3((nb[ok] | (q[ok] & 0x80)).astype(np.uint8))
        d = np.abs(x[ok] - alt)
        assert (err[ok] <= d).all()
        tie = (err[ok] == d) & (err[ok] > 0)
        assert ((q[ok][tie] & 1) == 0).all()
    # across zero: a value nearer the other sign's smallest subnormal than 0 cannot occur
    assert (np.abs(x[mag == 0]) <= 2.0 ** -10).all()
    # every midpoint is a tie that went to the even code
    qm = oracle.round_e4m3(mids)
    assert ((qm & 1) == 0).all()


def test_round_matches_torch_within_range():
    rng = np.random.default_rng(32)
    mids = _midpoints()
    x = np.concatenate([rng.normal(size=50000) * 2.0 ** rng.integers(-14, 9, size=50000), mids, -mids,
                        [0.0, -0.0, 448.0, -448.0, 460.0, 464.0, -464.0]]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    assert np.array_equal(oracle.round_e4m3(x.astype(np.float64)), _torch_round(x))


def test_round_specials_and_saturation():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_e4m3(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(oracle.round_e4m3(vals[fin]), codes[fin])         # representable values map to themselves
    big = np.array([464.0001, 500.0, 1e30, np.inf, -465.0, -np.inf])
    assert oracle.round_e4m3(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.round_e4m3(np.array([np.nan]))[0] == 0x7F
    assert oracle.round_e4m3(np.array([-0.0, 0.0])).tolist() == [0x80, 0x00]


def test_scale_and_quantize():
    rng = np.random.default_rng(33)
    x = (rng.normal(size=(64, 96)) * 0.02).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    s = oracle.e4m3_scale(bits)
    assert s.dtype == np.float32
    amax = np.abs(oracle.widen(bits)).max()
    assert abs(float(s) * amax - 448.0) <= 448.0 * 2.0 ** -23                # one float32 rounding of 448 / amax
    q = oracle.quantize_e4m3(bits, s)
    dq = oracle.decode_e4m3(q)
    assert np.nanmax(np.abs(dq)) == 448.0                                   # the largest magnitude lands on 448
    xs = oracle.widen(bits) * float(s)
    normal = np.abs(xs) >= 2.0 ** -6
    assert (np.abs(dq - xs)[normal] <= 2.0 ** -4 * np.abs(xs)[normal] * (1 + 2.0 ** -20)).all()
    assert (np.abs(dq - xs)[~normal] <= 2.0 ** -10 * (1 + 2.0 ** -20)).all()
    # zero tensor: scale 1, codes 0; a power-of-two amax gives a power-of-two scale
    assert oracle.e4m3_scale(np.zeros(8, np.uint16)) == 1.0
    assert oracle.e4m3_scale(f32_to_bf16_bits(np.array([3.5, -1.0], np.float32))) == 128.0
    # representable values with scale 1 round-trip (bf16 holds every E4M3 value)
    codes = np.arange(0x7F, dtype=np.uint8)
    v = oracle.decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(oracle.quantize_e4m3(f32_to_bf16_bits(v), np.float32(1.0)), codes)


@pytest.mark.parametrize("K", [64, 256])
def test_scaled_product_equals_the_16bit_product_when_quantization_is_exact(K):
    """Integer inputs in [-3, 3] with one entry 3.5 per tensor: amax = 3.5, so
    both scales are 448 / 3.5 = 128, every scaled value is an E4M3 value and
    the 8-bit product divided by the scales equals the 16-bit oracle product."""
    rng = np.random.default_rng(34 + K)
    T, N = 40, 24
    X = rng.integers(-3, 4, size=(T, K)).astype(np.float32)
    W = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    X[0, 0] = 3.5
    W[5, 8] = 3.5                       # the largest magnitude of its group: kept by the prune
    Xb, Wb = f32_to_bf16_bits(X), f32_to_bf16_bits(W)
    mask, _ = oracle.prune24(Wb)
    vs, ms, _ = oracle.compress24(Wb, mask)
    sx, sw = oracle.e4m3_scale(Xb), oracle.e4m3_scale(vs)
    assert sx == 128.0 and sw == 128.0
    y8 = oracle.spmm_e4m3(oracle.quantize_e4m3(Xb, sx), sx, oracle.quantize_e4m3(vs, sw), ms, K, sw)
    assert np.array_equal(y8, oracle.spmm_fwd(Xb, vs, ms, K))
    # the backward orientation: dX = dY . W_dp through the double-pruned compressed
    # weight (3.5 is also the largest of its column group, so W_dp^T keeps it)
    dYf = rng.integers(-3, 4, size=(T, N)).astype(np.float32)
    dYf[1, 2] = -3.5
    dY = f32_to_bf16_bits(dYf)
    vdp, mdp, _ = oracle.double_prune(vs, ms, N, K)
    sdy, sdp = oracle.e4m3_scale(dY), oracle.e4m3_scale(vdp)
    assert sdy == 128.0 and sdp == 128.0
    dx8 = oracle.spmm_e4m3(oracle.quantize_e4m3(dY, sdy), sdy, oracle.quantize_e4m3(vdp, sdp), mdp, N, sdp)
    assert np.array_equal(dx8, oracle.spmm_bwd_dx(dY, vdp, mdp, N))


def test_scaled_product_triple_loop():
    """Tiny case against a triple loop over the decoded dense operands."""
    rng = np.random.default_rng(35)
    T, N, K = 3, 5, 8
    Xq = rng.integers(0, 0x7E, size=(T, K)).astype(np.uint8) | (rng.integers(0, 2, size=(T, K)) * 0x80).astype(np.uint8)
    W = f32_to_bf16_bits(rng.normal(size=(N, K)).astype(np.float32))
    mask, _ = oracle.prune24(W)
    vs, ms, _ = oracle.compress24(W, mask)
    sw = oracle.e4m3_scale(vs)
    vq = oracle.quantize_e4m3(vs, sw)
    dense_q = oracle.decompress24(vq, ms, K)
    y = oracle.spmm_e4m3(Xq, np.float32(0.5), vq, ms, K, sw)
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += oracle.decode_e4m3(Xq[t, k:k + 1])[0] * oracle.decode_e4m3(dense_q[n, k:k + 1])[0]
            assert y[t, n] == pytest.approx(acc / (0.5 * float(sw)), rel=1e-12, abs=1e-300)
