"""Pins of the oracle's TL2 weight code (edge page: module docstring item 2,
element-wise mirror consolidation; class SignedUnsignedWeightPacker).

The table is checked against the mirror rule itself (every one of the 27
ternary triplets is exactly one base triplet or its negation, and a base
triplet is zero or starts with +1), the index against a closed form, the
encodings against round trips and hand-built bytes, and the size against the
page's 5 bits per 3 weights."""

import itertools

import numpy as np
import pytest

from oracle import tl2


def test_base_triplets_follow_the_mirror_rule():
    base = tl2.BASE_TRIPLETS
    assert len(base) == 14 == (27 + 1) // 2           # ceil(27 / 2) states
    assert len(set(base)) == 14
    for b in base:
        nz = [v for v in b if v != 0]
        assert not nz or nz[0] == 1                     # canonical: first non-zero is +1
    covered = set(base) | {tuple(-v for v in b) for b in base}
    assert covered == set(itertools.product((-1, 0, 1), repeat=3))


def test_index_is_the_balanced_ternary_value():
    # the page's order: base triplet i has 9 w0 + 3 w1 + w2 == i
    for i, (w0, w1, w2) in enumerate(tl2.BASE_TRIPLETS):
        assert 9 * w0 + 3 * w1 + w2 == i


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
    assert packed.shape == (N, ((K + 383) // 384) * 80)
    np.testing.assert_array_equal(tl2.unpack(packed, K), t)


def test_five_bits_per_three_weights():
    # 80 bytes carry 128 triplets: 4-bit index + 1 sign bit each
    assert tl2.BLOCK_BYTES * 8 == tl2.TRIPLETS_PER_BLOCK * 5
    assert tl2.BLOCK_BYTES * 8 / tl2.BLOCK_K == pytest.approx(5 / 3)
    assert tl2.packed_bytes(6912, 2688) == 6912 * 7 * 80


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
    # K = 2560 is not a multiple of 3 or 384: the pad encodes zero weights
    rng = np.random.default_rng(9)
    t = rng.integers(-1, 2, size=(2, 2560)).astype(np.int8)
    full = tl2.unpack(tl2.pack(t), 7 * 384)
    np.testing.assert_array_equal(full[:, :2560], t)
    assert not full[:, 2560:].any()
