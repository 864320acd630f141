"""Code layouts: one code per element <-> packed storage.  Test infrastructure.

* FP4 nibbles: two 4-bit codes per byte, the code of the even column k in the
  low nibble.  The pages print no nibble order for the FP4 matvec; the only
  order any page states is "u32 low-first" (#683, "Step 2 result"), and this
  is the same rule applied to bytes.
* u32 low-first (affine 4/8-bit, #683 "Step 2 result"): 32/bits codes per
  32-bit word, code j of the word in bits [bits*j, bits*j + bits).

Rows are packed independently: row n of an [N, K] code matrix becomes row n
of the packed array.
"""

import numpy as np


def unpack_nibbles(packed, k):
    """uint8 [N, K/2] -> uint8 codes [N, K]; low nibble is the even column."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    if packed.shape[1] * 2 != k:
        raise ValueError("packed FP4 row has %d bytes, K=%d" % (packed.shape[1], k))
    out = np.empty((n, k), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def pack_nibbles(codes):
    """uint8 codes [N, K] (each 0..15, K even) -> uint8 [N, K/2]."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[1] % 2:
        raise ValueError("K must be even to pack nibbles")
    if (codes > 15).any():
        raise ValueError("FP4 code above 15")
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_u32(packed, k, bits):
    """uint32 [N, K*bits/32] -> uint8 codes [N, K]; code j at bits*j (low first)."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    packed = np.asarray(packed, dtype=np.uint32)
    per = 32 // bits
    n = packed.shape[0]
    if packed.shape[1] * per != k:
        raise ValueError("packed row has %d words, K=%d, bits=%d" % (packed.shape[1], k, bits))
    mask = np.uint32((1 << bits) - 1)
    out = np.empty((n, k), dtype=np.uint8)
    for j in range(per):
        out[:, j::per] = (packed >> np.uint32(bits * j)) & mask
    return out


def pack_u32(codes, bits):
    """uint8 codes [N, K] (K a multiple of 32/bits) -> uint32 [N, K*bits/32]."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    codes = np.asarray(codes, dtype=np.uint8)
    per = 32 // bits
    if codes.shape[1] % per:
        raise ValueError("K must be a multiple of %d" % per)
    if (codes >> bits).any():
        raise ValueError("code does not fit in %d bits" % bits)
    words = np.zeros((codes.shape[0], codes.shape[1] // per), dtype=np.uint32)
    for j in range(per):
        words |= codes[:, j::per].astype(np.uint32) << np.uint32(bits * j)
    return words
