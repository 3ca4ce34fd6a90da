"""Pins of the oracle's TL2 weight code (edge page: module docstring item 2,
element-wise mirror consolidation; class SignedUnsignedWeightPacker).

The oracle derives index and sign from the balanced-ternary value of a
triplet; its states are checked against the page's own table of base
triplets (tests/golden/tl2_base_triplets.json) and the mirror rule itself
(every one of the 27 ternary triplets is exactly one base triplet or its
negation, and a base triplet is zero or starts with +1), the encodings against
round trips and hand-built bytes, and the size against the page's 5 bits per
3 weights."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import tl2


def _page_table(golden_dir):
    with open(os.path.join(golden_dir, "tl2_base_triplets.json")) as f:
        return [tuple(b) for b in json.load(f)["base_triplets"]]


def test_decoded_states_are_the_pages_table(golden_dir):
    """Index i with sign 0 decodes to the page's i-th base triplet, with sign
    1 to its negation (edge page, SignedUnsignedWeightPacker's table)."""
    page = _page_table(golden_dir)
    idx = np.arange(14, dtype=np.uint8).reshape(1, 14)
    pos = tl2.decode_triplets(idx, np.zeros_like(idx), 42).reshape(14, 3)
    neg = tl2.decode_triplets(idx, np.ones_like(idx), 42).reshape(14, 3)
    assert [tuple(int(v) for v in r) for r in pos] == page
    assert [tuple(int(v) for v in r) for r in neg] == [tuple(-v for v in b) for b in page]


def test_pages_table_follows_the_mirror_rule(golden_dir):
    base = _page_table(golden_dir)
    assert len(base) == 14 == (27 + 1) // 2           # ceil(27 / 2) states
    assert len(set(base)) == 14
    for b in base:
        nz = [v for v in b if v != 0]
        assert not nz or nz[0] == 1                     # canonical: first non-zero is +1
    covered = set(base) | {tuple(-v for v in b) for b in base}
    assert covered == set(itertools.product((-1, 0, 1), repeat=3))


def test_encoding_uses_the_pages_positions(golden_dir):
    """Each of the 27 triplets encodes to the position of the page's entry
    equal to it (sign 0) or to its negation (sign 1)."""
    page = _page_table(golden_dir)
    states = list(itertools.product((-1, 0, 1), repeat=3))
    idx, sign = tl2.encode_triplets(np.array(states, dtype=np.int8).reshape(1, -1))
    for j, st in enumerate(states):
        if st in page:
            assert (idx[0, j], sign[0, j]) == (page.index(st), 0)
        else:
            assert (idx[0, j], sign[0, j]) == (page.index(tuple(-v for v in st)), 1)


def test_decode_rejects_out_of_range_codes():
    with pytest.raises(ValueError):
        tl2.decode_triplets(np.array([[14]], dtype=np.uint8), np.array([[0]], dtype=np.uint8), 3)


def test_every_state_encodes_and_decodes():
    states = np.array(list(itertools.product((-1, 0, 1), repeat=3)), dtype=np.int8)
    t = states.reshape(1, -1)                            # 27 triplets in one row
    idx, sign = tl2.encode_triplets(t)
    for j, (w0, w1, w2) in enumerate(states):
        v = 9 * int(w0) + 3 * int(w1) + int(w2)
        assert idx[0, j] == abs(v)                       # |balanced value| is the index
        assert sign[0, j] == (1 if v < 0 else 0)         # negative value: mirrored
        assert idx[0, j] <= 13 and sign[0, j] <= 1
    np.testing.assert_array_equal(tl2.decode_triplets(idx, sign, 81), t)


@pytest.mark.parametrize("N,K", [(3, 64), (2, 100), (5, 384), (2, 385), (4, 2560), (1, 1)])
def test_round_trips(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    idx, sign = tl2.encode_triplets(t)
    assert idx.shape == (N, (K + 2) // 3)
    np.testing.assert_array_equal(tl2.decode_triplets(idx, sign, K), t)
    packed = tl2.pack(t)
    assert packed.shape == (N, tl2.row_bytes(K))
    np.testing.assert_array_equal(tl2.unpack(packed, K), t)


def test_five_bits_per_three_weights():
    # 80 bytes carry 128 triplets: 4-bit index + 1 sign bit each
    assert tl2.BLOCK_BYTES * 8 == tl2.TRIPLETS_PER_BLOCK * 5
    assert tl2.BLOCK_BYTES * 8 / tl2.BLOCK_K == pytest.approx(5 / 3)
    assert tl2.packed_bytes(6912, 2688) == 6912 * 7 * 80
    # a partial last block keeps only the groups of 96 weights it reaches, 20
    # bytes each rounded up to 16: K = 2560 is 6 whole blocks and 3 groups
    assert tl2.block_groups(2560) == [4] * 6 + [3]
    assert tl2.packed_bytes(6912, 2560) == 6912 * (6 * 80 + 64)
    assert tl2.packed_bytes(1, 16384) == 42 * 80 + 64      # 1.672 bits per weight
    assert [tl2.block_bytes(g) for g in (1, 2, 3, 4)] == [32, 48, 64, 80]


def test_hand_built_block():
    K = 384
    t = np.zeros((1, K), dtype=np.int8)
    t[0, 0:3] = (1, 1, 1)        # triplet 0: index 13, sign 0 -> byte 0 low nibble
    t[0, 12:15] = (-1, 0, 0)     # triplet 4 (i = 1): index 9, sign 1 -> byte 0 high nibble, bit 1 of byte 64
    t[0, 3:6] = (0, -1, 1)       # triplet 1 (tt = 1): -(0, 1, -1) -> index 2, sign 1 -> byte 1, bit 0 of byte 65
    t[0, 96:99] = (0, 0, 1)      # triplet 32 (g = 1): index 1 -> byte 16 low nibble
    t[0, 381:384] = (1, -1, 0)   # triplet 127 (g 3, i 7, tt 3): index 6 -> byte 48+12+3 high nibble
    packed = tl2.pack(t)
    expect = np.zeros(80, dtype=np.uint8)
    expect[0] = 13 | (9 << 4)
    expect[64] = 1 << 1
    expect[1] = 2
    expect[65] = 1 << 0
    expect[16] = 1
    expect[63] = 6 << 4
    np.testing.assert_array_equal(packed[0], expect)


def test_padding_is_zero_weight():
    # K = 2560 is not a multiple of 3 or 384: the last block's three groups
    # reach weight 2592, and the pad encodes zero weights
    rng = np.random.default_rng(9)
    t = rng.integers(-1, 2, size=(2, 2560)).astype(np.int8)
    packed = tl2.pack(t)
    assert tl2.row_bytes(2592) == packed.shape[1]
    full = tl2.unpack(packed, 2592)
    np.testing.assert_array_equal(full[:, :2560], t)
    assert not full[:, 2560:].any()


def test_hand_built_partial_block():
    # K = 484: one whole block, then a block of two groups (48 bytes: indices
    # at 0..31, signs at 32..39, zeros at 40..47)
    K = 484
    t = np.zeros((1, K), dtype=np.int8)
    t[0, 384:387] = (1, 0, 0)    # triplet 128, the tail's triplet 0: index 9 -> byte 80 low nibble
    t[0, 482] = -1               # triplet 160 (g = 1, i = 0, tt = 0) = (0, 0, -1): index 1, sign 1
    packed = tl2.pack(t)
    expect = np.zeros(80 + 48, dtype=np.uint8)
    expect[80] = 9
    expect[80 + 16] = 1
    expect[80 + 32 + 4] = 1      # sign bit 0 of byte 16 G + 4 g + tt, G = 2
    np.testing.assert_array_equal(packed[0], expect)
    np.testing.assert_array_equal(tl2.unpack(packed, K), t)
