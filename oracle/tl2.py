"""TL2 ternary weight code (1.67 bits per weight) — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may call this.
Nothing here is used by, or uses, the HIP library.

Source: the [edge] page (Quillan-Ronin "bitnet_cpp_edge.py", the bitnet.cpp
simulation): its module docstring item 2 (element-wise mirror consolidation:
the 27 states of a ternary triplet fold onto 14 unsigned states, stored as a
4-bit index plus a sign bit, 5 bits per 3 weights) and class
SignedUnsignedWeightPacker (its table of 14 base triplets and the pack /
unpack of triplets).

Readings where the page is silent or does something this library does not:
  * The page packs only the first floor(K/3) triplets of a row and drops the
    rest; here the row is padded with zero weights to a whole number of
    triplets, so no weight is lost (a zero weight adds nothing to a product).
  * The page keeps indices and sign bits in two byte arrays. The device
    layout below (blocks of 128 triplets, 64 bytes of 4-bit indices and 16
    bytes of sign bits) is a contract of this library, not of the page; it
    stores exactly 5 bits per triplet. A row's last block holds only the
    groups of 32 triplets (96 weights) that the row reaches, so the padding
    is under 96 weights and 16 bytes per row (1.67 bits per weight at
    K = 16384, 1.70 at K = 2560).

Parity status: pinned (tests/test_oracle_tl2.py: the decoded states against
the page's own table of base triplets (tests/golden/tl2_base_triplets.json)
and the mirror rule over all 27 states, round trips, hand built bytes, 5/3
bits per weight).
"""

from __future__ import annotations

import numpy as np

# [edge] module docstring item 2 (mirror consolidation): a ternary triplet
# and its negation share one stored state, so the 27 triplets fold onto 14
# unsigned states plus a sign. Reading a triplet as the balanced-ternary
# number v = 9 w0 + 3 w1 + w2 (v in [-13, 13], negation is v -> -v), the
# unsigned state is |v| (the zero triplet, or one whose leading non-zero digit
# is +1) and the sign is v < 0. The page's SignedUnsignedWeightPacker lists
# the 14 unsigned states in increasing |v|, so the page's index of a state is
# |v| itself (pinned against the page's table in tests/golden).
N_STATES = 14

TRIPLETS_PER_BLOCK = 128
BLOCK_K = 3 * TRIPLETS_PER_BLOCK      # 384 weights per device block
BLOCK_BYTES = 64 + 16                 # 4-bit indices, then sign bits
GROUP_TRIPLETS = 32                   # a group: 16 index bytes and 4 sign bytes


def block_groups(K: int):
    """Groups (of 32 triplets) of each block of a row of K weights: 4 for the
    whole blocks, then, for a partial last block, the ceil(rest / 96) groups
    it reaches."""
    full, rest = divmod(K, BLOCK_K)
    return [4] * full + ([-(-rest // (3 * GROUP_TRIPLETS))] if rest else [])


def block_bytes(groups: int) -> int:
    """Bytes of a block of `groups` groups: 20 per group, rounded up to 16."""
    return -(-20 * groups // 16) * 16


def row_bytes(K: int) -> int:
    return sum(block_bytes(g) for g in block_groups(K))


def triplet_value(t: np.ndarray) -> np.ndarray:
    """Balanced-ternary value 9 w0 + 3 w1 + w2 of each triplet (last axis 3)."""
    t = np.asarray(t, dtype=np.int64)
    return 9 * t[..., 0] + 3 * t[..., 1] + t[..., 2]


def triplets_of_value(v: np.ndarray) -> np.ndarray:
    """Inverse of triplet_value: the balanced-ternary digits (w0, w1, w2) in
    {-1, 0, 1} of v in [-13, 13] (last digit first: w2 = ((v + 1) mod 3) - 1)."""
    v = np.asarray(v, dtype=np.int64)
    w2 = (v + 1) % 3 - 1
    v1 = (v - w2) // 3
    w1 = (v1 + 1) % 3 - 1
    w0 = (v1 - w1) // 3
    return np.stack([w0, w1, w2], axis=-1).astype(np.int8)


def encode_triplets(t: np.ndarray):
    """(index uint8 [N, T], sign uint8 [N, T]) of ternary t [N, K], T = ceil(K/3);
    the row is padded with zero weights to 3 T (reading above)."""
    t = np.asarray(t)
    N, K = t.shape
    if t.size and (t.min() < -1 or t.max() > 1):
        raise ValueError("ternary values must lie in {-1, 0, 1}")
    T = (K + 2) // 3
    padded = np.zeros((N, 3 * T), dtype=np.int64)
    padded[:, :K] = t
    v = triplet_value(padded.reshape(N, T, 3))
    return np.abs(v).astype(np.uint8), (v < 0).astype(np.uint8)


def decode_triplets(idx: np.ndarray, sign: np.ndarray, K: int) -> np.ndarray:
    """Ternary int8 [N, K] from indices and sign bits (the padding dropped)."""
    idx = np.asarray(idx, dtype=np.int64)
    sign = np.asarray(sign, dtype=np.int64)
    if idx.size and (idx.max() >= N_STATES or sign.max() > 1):
        raise ValueError("TL2 index must lie in 0..13 and the sign in {0, 1}")
    N, T = idx.shape
    v = np.where(sign == 1, -idx, idx)
    return triplets_of_value(v).reshape(N, 3 * T)[:, :K]


def _slot(j: int, groups: int = 4):
    """Byte/bit position of triplet j (0 .. 32 groups - 1) of a device block of
    `groups` groups.

    Triplet j = 32 g + 4 i + tt: its index is the nibble 4 (i % 2) of byte
    16 g + 4 (i // 2) + tt, its sign is bit i of byte 16 groups + 4 g + tt
    (64 + 4 g + tt in a whole block)."""
    g, r = divmod(j, 32)
    i, tt = divmod(r, 4)
    return 16 * g + 4 * (i // 2) + tt, 4 * (i % 2), 16 * groups + 4 * g + tt, i


def pack(t: np.ndarray) -> np.ndarray:
    """Device TL2 bytes [N, row_bytes(K)] of ternary t [N, K]: block b holds
    triplets 128 b .. (weights 384 b ..), the last block only the groups of
    32 triplets the row reaches (the part past K is zero weights), and the
    bytes a block is rounded up by are zero."""
    t = np.asarray(t)
    N, K = t.shape
    groups = block_groups(K)
    ntrip = TRIPLETS_PER_BLOCK * (len(groups) - 1) + GROUP_TRIPLETS * groups[-1] if groups else 0
    full = np.zeros((N, 3 * ntrip), dtype=np.int8)
    full[:, :K] = t
    idx, sign = encode_triplets(full)
    out = np.zeros((N, row_bytes(K)), dtype=np.uint8)
    for n in range(N):
        base = 0
        for b, gb in enumerate(groups):
            for j in range(GROUP_TRIPLETS * gb):
                nb, sh, sb, bit = _slot(j, gb)
                tj = b * TRIPLETS_PER_BLOCK + j
                out[n, base + nb] |= np.uint8(int(idx[n, tj]) << sh)
                out[n, base + sb] |= np.uint8(int(sign[n, tj]) << bit)
            base += block_bytes(gb)
    return out


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    """Ternary int8 [N, K] from device TL2 bytes [N, row_bytes(K)]."""
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    groups = block_groups(K)
    if packed.shape[1] != row_bytes(K):
        raise ValueError("not the TL2 bytes of a row of K weights")
    ntrip = TRIPLETS_PER_BLOCK * len(groups)
    idx = np.zeros((N, ntrip), dtype=np.uint8)
    sign = np.zeros_like(idx)
    for n in range(N):
        base = 0
        for b, gb in enumerate(groups):
            for j in range(GROUP_TRIPLETS * gb):
                nb, sh, sb, bit = _slot(j, gb)
                idx[n, b * TRIPLETS_PER_BLOCK + j] = (int(packed[n, base + nb]) >> sh) & 15
                sign[n, b * TRIPLETS_PER_BLOCK + j] = (int(packed[n, base + sb]) >> bit) & 1
            base += block_bytes(gb)
    return decode_triplets(idx, sign, 3 * ntrip)[:, :K]


def packed_bytes(N: int, K: int) -> int:
    return N * row_bytes(K)
