"""Pins of the oracle's low-bit KV-cache quantizer — CPU only.

Engine page: module docstring item 5 (Section 3.1, Tables 2 and 3) and
BitNetV2Attention._quantize_kv_head. Token 0 (BOS) of every head uses the
int8 absmax quantizer; the others use int4 absmean*sqrt7, 3-bit absmax with
scale 3 and clip [-4, 3], or int8.
"""

import numpy as np
import pytest

import oracle


def test_hand_values_each_branch():
    row = np.array([1.0, -2.0, 0.5, 4.0])
    kv = np.stack([row, row])[None]  # [1 head, S=2, D=4]
    eps = 1e-7
    # BOS, int8 absmax: s = 4 + eps, p = 127 x / s = 31.75-, -63.5+, 15.875-, 127-
    # (eps pulls -63.5 towards zero, so it rounds to -63, not to the even -64)
    q8, s8, _ = oracle.kv_quantize(kv, 3)
    assert q8[0, 0].tolist() == [32, -63, 16, 127]
    # 3-bit absmax: p = 3 x / s = 0.75-, -1.5+, 0.375-, 3- -> 1, -1, 0, 3
    assert q8[0, 1].tolist() == [1, -1, 0, 3]
    np.testing.assert_allclose(s8, [[4.0 + eps, 4.0 + eps]], rtol=1e-15)
    # int4 absmean: s = mean|x| + eps = 1.875 + eps, p = sqrt7 x / s
    q4, s4, p4 = oracle.kv_quantize(kv, 4)
    np.testing.assert_allclose(s4[0, 1], 1.875 + eps, rtol=1e-15)
    r7 = np.sqrt(7.0) / 1.875  # 1.41107...
    # 1.411 -> 1, -2.822 -> -3, 0.706 -> 1, 5.644 -> 6
    assert q4[0, 1].tolist() == [1, -3, 1, 6]
    np.testing.assert_allclose(p4[0, 1], r7 * row, rtol=1e-6)


def test_bos_and_branches_reduce_to_the_activation_quantizers():
    rng = np.random.default_rng(1)
    kv = rng.standard_normal((2, 3, 9, 64)) * 3
    for bits in (3, 4, 8):
        q, s, _ = oracle.kv_quantize(kv, bits)
        qb, sb, _ = oracle.quantize_activations(kv[..., 0, :], 8)
        np.testing.assert_array_equal(q[..., 0, :], qb)
        np.testing.assert_allclose(s[..., 0], sb, rtol=0)
        if bits in (4, 8):
            qr, sr, _ = oracle.quantize_activations(kv[..., 1:, :], bits)
            np.testing.assert_array_equal(q[..., 1:, :], qr)
            np.testing.assert_allclose(s[..., 1:], sr, rtol=0)


def test_three_bit_properties():
    rng = np.random.default_rng(2)
    kv = rng.standard_normal((4, 17, 128))
    q, s, _ = oracle.kv_quantize(kv, 3)
    rest = q[:, 1:, :]
    assert rest.min() >= -4 and rest.max() <= 3
    # the largest |x| of a token maps to +-3
    amax = np.argmax(np.abs(kv[:, 1:, :]), axis=-1)
    picked = np.take_along_axis(rest, amax[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(picked) == 3)
    # dequantization error is at most half a step (s / 3 / 2) for every element
    xh = oracle.kv_dequantize(q, s, 3)
    step = s[:, 1:] / 3.0
    assert np.all(np.abs(xh[:, 1:, :] - kv[:, 1:, :]) <= step[..., None] / 2 + 1e-12)
    # positive per-token scaling leaves the codes unchanged (up to eps)
    q2, _, p2 = oracle.kv_quantize(kv * 7.5, 3)
    far = oracle.quant_boundary_distance(p2) > 1e-6
    np.testing.assert_array_equal(q[far], q2[far])


def test_single_token_and_bad_bits():
    kv = np.array([[[3.0, -1.0, 0.0, 0.25]]])
    q, s, _ = oracle.kv_quantize(kv, 3)
    assert q.tolist() == [[[127, -42, 0, 11]]]  # only BOS: int8
    with pytest.raises(ValueError):
        oracle.kv_quantize(kv, 2)


# ---- packed storage of the 3- and 4-bit codes ------------------------------

def test_kv_pack_hand_built_bytes():
    # 4 bits, two's complement nibbles, code 2i in the low nibble of byte i:
    #   1 -> 0001, -1 -> 1111: byte 0 = 1111 0001 = 0xF1
    #   7 -> 0111, -8 -> 1000: byte 1 = 1000 0111 = 0x87
    np.testing.assert_array_equal(oracle.kv_pack(np.array([[1, -1, 7, -8]]), 4), [[0xF1, 0x87]])
    # 3 bits, code k at stream bits 3k .. 3k+2, least significant bit first:
    #   1 = 001, -1 = 111, 3 = 011, -4 = 100, 0 = 000, 2 = 010, -2 = 110, -3 = 101
    #   stream bits 0..7   = 1,0,0, 1,1,1, 1,1   -> byte 0 = 0b11111001 = 0xF9
    #   stream bits 8..15  = 0, 0,0,1, 0,0,0, 0  -> byte 1 = 0b00001000 = 0x08
    #   stream bits 16..23 = 1,0, 0,1,1, 1,0,1   -> byte 2 = 0b10111001 = 0xB9
    q = np.array([[1, -1, 3, -4, 0, 2, -2, -3]])
    np.testing.assert_array_equal(oracle.kv_pack(q, 3), [[0xF9, 0x08, 0xB9]])
    np.testing.assert_array_equal(oracle.kv_unpack(np.array([[0xF9, 0x08, 0xB9]]), 3, 8), q)
    np.testing.assert_array_equal(oracle.kv_unpack(np.array([[0xF1, 0x87]]), 4, 4), [[1, -1, 7, -8]])


@pytest.mark.parametrize("bits,D", [(4, 8), (4, 128), (4, 24), (3, 8), (3, 128), (3, 96)])
def test_kv_pack_round_trip_and_numpy_bit_order(bits, D):
    rng = np.random.default_rng(D + bits)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    q = rng.integers(lo, hi + 1, size=(5, D))
    packed = oracle.kv_pack(q, bits)
    assert packed.shape == (5, D * bits // 8)
    np.testing.assert_array_equal(oracle.kv_unpack(packed, bits, D), q)
    # the same stream through numpy's own little-endian bit packer
    field = (q & ((1 << bits) - 1))[:, :, None]
    stream = ((field >> np.arange(bits)) & 1).astype(np.uint8).reshape(5, D * bits)
    np.testing.assert_array_equal(packed, np.packbits(stream, axis=1, bitorder="little"))


def test_kv_pack_rejects_what_it_cannot_hold():
    with pytest.raises(ValueError):
        oracle.kv_pack(np.array([[8, 0]]), 4)
    with pytest.raises(ValueError):
        oracle.kv_pack(np.array([[-5, 0, 0, 0, 0, 0, 0, 0]]), 3)
    with pytest.raises(ValueError):
        oracle.kv_pack(np.zeros((1, 4), dtype=np.int64), 3)  # 12 bits: not whole bytes
    with pytest.raises(ValueError):
        oracle.kv_pack(np.zeros((1, 8), dtype=np.int64), 8)
