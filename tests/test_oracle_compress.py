"""Pins of the oracle's compressed 2:4 format.

Discussion page, "Memory Footprint Reduction During Pretraining and Inference":
a 2:4 weight stores two 16-bit non-zeros plus their indices per four elements.
The bit layout of the indices is this library's reading (two 2-bit positions per
group); the pins are a hand-worked fixture, the round trip, the set of legal
nibbles and the padding / invalid-group rules.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "compress_hand_example.json")


def test_hand_worked_example():
    d = json.load(open(GOLDEN))
    W = np.array(d["W"], dtype=np.float32).view(np.uint32)
    mask, W_s = oracle.prune24(W)
    for r, pairs in enumerate(d["kept_pairs"]):
        for g, (a, b) in enumerate(pairs):
            assert np.flatnonzero(mask[r, 4 * g:4 * g + 4]).tolist() == [a, b], (r, g)
    values, meta, invalid = oracle.compress24(W_s, mask)
    assert invalid == 0
    assert meta.tolist() == d["meta_words"]
    assert [hex(w).upper().replace("X", "x") for w in meta[0]] == d["meta_words_hex"][0]
    assert (values.view(np.float32) == np.array(d["values"], dtype=np.float32)).all()


def test_pair_nibbles():
    # each of the six kept pairs i0 < i1 maps to i0 | i1 << 2
    expected = {(0, 1): 4, (0, 2): 8, (0, 3): 12, (1, 2): 9, (1, 3): 13, (2, 3): 14}
    for (a, b), nib in expected.items():
        m = np.zeros((1, 4), dtype=np.uint8)
        m[0, [a, b]] = 1
        A = np.array([[1, 2, 3, 4]], dtype=np.uint16)
        values, meta, invalid = oracle.compress24(A, m)
        assert invalid == 0 and int(meta[0, 0]) == nib
        assert values.tolist() == [[[1, 2, 3, 4][a], [1, 2, 3, 4][b]]]
    assert oracle.LEGAL_NIBBLES == frozenset(expected.values())


@pytest.mark.parametrize("cols", [4, 32, 36, 100, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_round_trip_and_sizes(cols, dtype):
    rng = np.random.default_rng(cols)
    v = rng.standard_normal((7, cols)).astype(np.float32)
    bits = f32_to_bf16_bits(v) if dtype == "bf16" else v.view(np.uint32)
    mask, A_s = oracle.prune24(bits)
    values, meta, invalid = oracle.compress24(bits, mask)
    assert invalid == 0
    assert values.shape == (7, cols // 2) and meta.shape == (7, -(-cols // 32))
    assert (oracle.decompress24(values, meta, cols) == A_s).all()
    assert (oracle.mask_from_meta(meta, cols) == mask).all()
    groups = cols // 4
    for g in range(groups):
        nib = (meta[:, g // 8] >> (4 * (g % 8))) & 0xF
        assert set(nib.tolist()) <= oracle.LEGAL_NIBBLES
    if groups % 8:  # unused high nibbles of the last word stay clear
        assert ((meta[:, -1] >> (4 * (groups % 8))) == 0).all()


def test_padding_when_fewer_than_two_kept():
    A = np.array([[5, 6, 7, 8, 5, 6, 7, 8]], dtype=np.uint16)
    m = np.array([[0, 0, 1, 0, 0, 0, 0, 0]], dtype=np.uint8)
    values, meta, invalid = oracle.compress24(A, m)
    assert invalid == 0
    # group 0: kept {2}, padded with lowest unkept 0 (value +0) -> (0, 2)
    # group 1: nothing kept -> (0, 1) with +0 values
    assert values.tolist() == [[0, 7, 0, 0]]
    assert int(meta[0, 0]) == (0 | 2 << 2) | ((0 | 1 << 2) << 4)


def test_more_than_two_kept_is_counted():
    A = np.array([[5, 6, 7, 8]], dtype=np.uint16)
    m = np.array([[1, 1, 1, 0]], dtype=np.uint8)
    values, meta, invalid = oracle.compress24(A, m)
    assert invalid == 1 and values.tolist() == [[5, 6]] and int(meta[0, 0]) == 4


def test_decompress_rejects_illegal_nibble():
    with pytest.raises(ValueError):
        oracle.decompress24(np.zeros((1, 2), np.uint16), np.array([[0x0]], np.uint32), 4)
