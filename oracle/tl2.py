"""TL2 ternary weight code (1.67 bits per weight) — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may call this.
Nothing here is used by, or uses, the HIP library.

Source: the [edge] page (Quillan-Ronin "bitnet_cpp_edge.py", the bitnet.cpp
simulation): its module docstring item 2 (element-wise mirror consolidation:
the 27 states of a ternary triplet fold onto 14 unsigned states, stored as a
4-bit index plus a sign bit, 5 bits per 3 weights) and class
SignedUnsignedWeightPacker (the table of 14 base triplets and the
pack/unpack of triplets).

Readings where the page is silent or does something this library does not:
  * The page packs only the first floor(K/3) triplets of a row and drops the
    rest; here the row is padded with zero weights to a whole number of
    triplets, so no weight is lost (a zero weight adds nothing to a product).
  * The page keeps indices and sign bits in two byte arrays. The device
    layout below (blocks of 128 triplets, 64 bytes of 4-bit indices and 16
    bytes of sign bits) is a contract of this library, not of the page; it
    stores exactly 5 bits per triplet.

Parity status: pinned (tests/test_oracle_tl2.py: the table against the
mirror rule and all 27 states, a closed form of the index, round trips, hand
built bytes, 5/3 bits per weight).
"""

from __future__ import annotations

import numpy as np

# [edge] SignedUnsignedWeightPacker: the 14 base triplets, in the page's order.
# Each is either all zero or has its first non-zero element equal to +1; a
# triplet is stored as the index of the base triplet equal to it (sign 0) or
# to its negation (sign 1).
BASE_TRIPLETS = [
    (0, 0, 0), (0, 0, 1), (0, 1, -1), (0, 1, 0), (0, 1, 1),
    (1, -1, -1), (1, -1, 0), (1, -1, 1), (1, 0, -1), (1, 0, 0),
    (1, 0, 1), (1, 1, -1), (1, 1, 0), (1, 1, 1),
]

TRIPLETS_PER_BLOCK = 128
BLOCK_K = 3 * TRIPLETS_PER_BLOCK      # 384 weights per device block
BLOCK_BYTES = 64 + 16                 # 4-bit indices, then sign bits


def _tables():
    enc = {}
    dec = {}
    for i, b in enumerate(BASE_TRIPLETS):
        enc[b] = (i, 0)
        dec[(i, 0)] = b
        if b != (0, 0, 0):
            neg = (-b[0], -b[1], -b[2])
            enc[neg] = (i, 1)
            dec[(i, 1)] = neg
    return enc, dec


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
    enc, _ = _tables()
    idx = np.zeros((N, T), dtype=np.uint8)
    sign = np.zeros((N, T), dtype=np.uint8)
    for n in range(N):
        for j in range(T):
            i, s = enc[tuple(int(v) for v in padded[n, 3 * j:3 * j + 3])]
            idx[n, j] = i
            sign[n, j] = s
    return idx, sign


def decode_triplets(idx: np.ndarray, sign: np.ndarray, K: int) -> np.ndarray:
    """Ternary int8 [N, K] from indices and sign bits (the padding dropped)."""
    _, dec = _tables()
    N, T = idx.shape
    out = np.zeros((N, 3 * T), dtype=np.int8)
    for n in range(N):
        for j in range(T):
            out[n, 3 * j:3 * j + 3] = dec[(int(idx[n, j]), int(sign[n, j]))]
    return out[:, :K]


def _slot(j: int):
    """Byte/bit position of triplet j (0..127) of a device block.

    Triplet j = 32 g + 4 i + tt: its index is the nibble 4 (i % 2) of byte
    16 g + 4 (i // 2) + tt, its sign is bit i of byte 64 + 4 g + tt."""
    g, r = divmod(j, 32)
    i, tt = divmod(r, 4)
    return 16 * g + 4 * (i // 2) + tt, 4 * (i % 2), 64 + 4 * g + tt, i


def pack(t: np.ndarray) -> np.ndarray:
    """Device TL2 bytes [N, ceil(K/384) * 80] of ternary t [N, K]: block b holds
    triplets 128 b .. 128 b + 127 (weights 384 b .. 384 b + 383; the part past
    K is zero weights)."""
    t = np.asarray(t)
    N, K = t.shape
    nblk = (K + BLOCK_K - 1) // BLOCK_K
    full = np.zeros((N, nblk * BLOCK_K), dtype=np.int8)
    full[:, :K] = t
    idx, sign = encode_triplets(full)
    out = np.zeros((N, nblk * BLOCK_BYTES), dtype=np.uint8)
    for n in range(N):
        for b in range(nblk):
            base = b * BLOCK_BYTES
            for j in range(TRIPLETS_PER_BLOCK):
                nb, sh, sb, bit = _slot(j)
                tj = b * TRIPLETS_PER_BLOCK + j
                out[n, base + nb] |= np.uint8(int(idx[n, tj]) << sh)
                out[n, base + sb] |= np.uint8(int(sign[n, tj]) << bit)
    return out


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    """Ternary int8 [N, K] from device TL2 bytes."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, nbytes = packed.shape
    nblk = nbytes // BLOCK_BYTES
    idx = np.zeros((N, nblk * TRIPLETS_PER_BLOCK), dtype=np.uint8)
    sign = np.zeros_like(idx)
    for n in range(N):
        for b in range(nblk):
            base = b * BLOCK_BYTES
            for j in range(TRIPLETS_PER_BLOCK):
                nb, sh, sb, bit = _slot(j)
                idx[n, b * TRIPLETS_PER_BLOCK + j] = (int(packed[n, base + nb]) >> sh) & 15
                sign[n, b * TRIPLETS_PER_BLOCK + j] = (int(packed[n, base + sb]) >> bit) & 1
    return decode_triplets(idx, sign, nblk * BLOCK_K)[:, :K]


def packed_bytes(N: int, K: int) -> int:
    return N * ((K + BLOCK_K - 1) // BLOCK_K) * BLOCK_BYTES
