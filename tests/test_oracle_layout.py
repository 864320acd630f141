"""Pins for the oracle's packed-code layouts (CPU only).

Every code value is placed at every position of a word and the packed word is
compared with the closed form "code j of the word sits at bit bits*j" (#683,
"Step 2 result": u32 low-first) and "even column in the low nibble" for FP4.
"""

import numpy as np
import pytest

from oracle import layout as L


def test_nibbles_closed_form_every_code_every_position():
    for v in range(16):
        for pos in range(2):
            codes = np.zeros((1, 2), dtype=np.uint8)
            codes[0, pos] = v
            packed = L.pack_nibbles(codes)
            assert packed.shape == (1, 1)
            assert int(packed[0, 0]) == v << (4 * pos)
            assert np.array_equal(L.unpack_nibbles(packed, 2), codes)


@pytest.mark.parametrize("bits", [4, 8])
def test_u32_closed_form_every_code_every_position(bits):
    per = 32 // bits
    for v in range(1 << bits):
        for pos in range(per):
            codes = np.zeros((1, per), dtype=np.uint8)
            codes[0, pos] = v
            w = L.pack_u32(codes, bits)
            assert w.shape == (1, 1) and w.dtype == np.uint32
            assert int(w[0, 0]) == v << (bits * pos)
            assert np.array_equal(L.unpack_u32(w, per, bits), codes)


@pytest.mark.parametrize("bits,k", [(4, 64), (8, 64), (4, 3840), (8, 128)])
def test_u32_round_trip_random(bits, k):
    rng = np.random.default_rng(bits * 1000 + k)
    codes = rng.integers(0, 1 << bits, (7, k), dtype=np.uint8)
    w = L.pack_u32(codes, bits)
    assert w.shape == (7, k * bits // 32)
    assert np.array_equal(L.unpack_u32(w, k, bits), codes)


def test_nibble_round_trip_random():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (9, 512), dtype=np.uint8)
    p = L.pack_nibbles(codes)
    assert p.shape == (9, 256)
    assert np.array_equal(L.unpack_nibbles(p, 512), codes)


def test_layout_rejects_bad_input():
    with pytest.raises(ValueError):
        L.pack_nibbles(np.full((1, 2), 16, dtype=np.uint8))
    with pytest.raises(ValueError):
        L.pack_u32(np.full((1, 8), 16, dtype=np.uint8), 4)
    with pytest.raises(ValueError):
        L.unpack_u32(np.zeros((1, 3), dtype=np.uint32), 8, 4)
    with pytest.raises(ValueError):
        L.unpack_nibbles(np.zeros((1, 3), dtype=np.uint8), 8)
