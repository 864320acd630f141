"""Pins for the oracle's two-level super-block 4-bit format (CPU only).

* a super-block quantized by hand (tests/golden), record bytes included;
* the record layout against closed forms: each six-bit factor alone at each
  position sets exactly its six bits; codes land in their nibble;
* d and dmin are torch's fp16 rounding of the largest sub-block scale and
  offset over 63; every code is the nearest of the 16 grid points to the
  weight (exact rational search, ties to even, clamped);
* the matvec against exact rational brute force over hand-decoded records,
  one-hot columns, and the bound the quantization error must meet;
* the device layout (repack) decodes to the same weights through a decoder
  written here from the layout's description;
* the byte counts: 4.5 bits per weight stored, 4.625 in the device layout.
A wrong nibble order, a swapped d/dmin, a min added instead of subtracted, an
off-by-one six-bit shift or a floor for rint fails one of these.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import superblock as SB

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16_torch(vals):
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float64)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _golden_weights():
    sub = [np.array([t / 4 for t in range(16)] * 2),
           np.array([-1 + t / 8 for t in range(16)] * 2),
           np.array([1.5, 0.75, float(np.float32(0.1))] + [0.0] * 29),
           np.array([-0.5, -0.25] + [-0.5] * 30)] + [np.zeros(32)] * 4
    return np.concatenate(sub).astype(np.float32)[None, :]


def test_hand_worked_super_block():
    g = json.load(open(os.path.join(GOLDEN, "q4k_superblock_hand_example.json")))
    rec = SB.quantize_q4k(_golden_weights())
    assert rec.shape == (1, 1, 144)
    assert [int(b) for b in rec[0, 0, :16]] == [int(v, 16) for v in g["record_bytes_0_to_15"]]
    d_bits, dmin_bits, sc, m, q = SB.unpack_records(rec)
    assert int(d_bits[0, 0]) == int(g["d_fp16_bits"], 16)
    assert int(dmin_bits[0, 0]) == int(g["dmin_fp16_bits"], 16)
    assert list(sc[0, 0]) == g["sc"] and list(m[0, 0]) == g["m"]
    qq = q[0, 0]
    assert list(qq[0:16]) == g["q_sub0_first16"] and list(qq[16:32]) == g["q_sub0_first16"]
    assert list(qq[32:48]) == g["q_sub1_first16"]
    assert list(qq[64:67]) == g["q_sub2_first3"] and list(qq[96:99]) == g["q_sub3_first3"]
    assert not qq[128:].any()
    # code bytes: the even weight in the low nibble
    assert rec[0, 0, 16] == 0x10 and rec[0, 0, 17] == 0x32


@pytest.mark.parametrize("j", range(8))
def test_six_bit_fields_closed_form(j):
    """A factor of 63 at sub-block j alone sets bits 6j..6j+5 of its 48-bit
    field and nothing else; 1 sets bit 6j."""
    for base, key in ((4, "sc"), (10, "m")):
        for val in (63, 1):
            f = {"sc": np.zeros((1, 1, 8), np.int64), "m": np.zeros((1, 1, 8), np.int64)}
            f[key][0, 0, j] = val
            rec = SB.pack_records(np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16), f["sc"], f["m"],
                                  np.zeros((1, 1, 256), np.int64))
            field = sum(int(rec[0, 0, base + b]) << (8 * b) for b in range(6))
            assert field == val << (6 * j)
            other = 10 if base == 4 else 4
            assert not rec[0, 0, other:other + 6].any() and not rec[0, 0, 16:].any()


def test_pack_unpack_round_trip_and_code_positions():
    rng = np.random.default_rng(1)
    n, nsb = 3, 2
    d = rng.integers(0, 1 << 16, (n, nsb)).astype(np.uint16)
    dm = rng.integers(0, 1 << 16, (n, nsb)).astype(np.uint16)
    sc = rng.integers(0, 64, (n, nsb, 8))
    m = rng.integers(0, 64, (n, nsb, 8))
    q = rng.integers(0, 16, (n, nsb, 256))
    rec = SB.pack_records(d, dm, sc, m, q)
    d2, dm2, sc2, m2, q2 = SB.unpack_records(rec)
    assert np.array_equal(d, d2) and np.array_equal(dm, dm2)
    assert np.array_equal(sc, sc2) and np.array_equal(m, m2) and np.array_equal(q, q2)
    # code i of a super-block: byte 16 + i // 2, nibble i % 2
    for i in (0, 1, 2, 77, 254, 255):
        byte = rec[:, :, 16 + i // 2]
        assert np.array_equal((byte >> (4 * (i % 2))) & 0xF, q[:, :, i])


def _rne_fraction(x):
    fl = x.numerator // x.denominator
    r = x - fl
    if r > Fraction(1, 2):
        return fl + 1
    if r < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def test_quantizer_scales_and_nearest_codes():
    """d, dmin are fp16 (torch's rounding) of max s / 63 and max off / 63;
    every code is the nearest grid point, by exact rational search."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((3, 512)) * np.exp2(rng.uniform(-6, 2, (3, 1)))).astype(np.float32)
    w[1, 256:288] = np.abs(w[1, 256:288])          # an all-positive sub-block: m = 0
    rec = SB.quantize_q4k(w)
    d_bits, dmin_bits, sc, m, q = SB.unpack_records(rec)
    wb = w.astype(np.float64).reshape(3, 2, 8, 32)
    lo = np.minimum(wb.min(axis=3), 0)
    s = (wb.max(axis=3) - lo) / 15
    assert np.array_equal(d_bits, _f16_torch(s.max(axis=2) / 63))
    assert np.array_equal(dmin_bits, _f16_torch((-lo).max(axis=2) / 63))
    assert m[1, 1, 0] == 0                         # row 1, super-block 1, sub-block 0
    d = d_bits.view(np.float16).astype(np.float64)
    dmin = dmin_bits.view(np.float16).astype(np.float64)
    for r in range(3):
        for b in range(2):
            for j in range(8):
                S = Fraction(d[r, b]) * int(sc[r, b, j])
                M = Fraction(dmin[r, b]) * int(m[r, b, j])
                assert int(sc[r, b, j]) == min(63, _rne_fraction(Fraction(s[r, b, j]) / Fraction(d[r, b])))
                for i in range(0, 32, 5):
                    x = Fraction(float(w[r, 256 * b + 32 * j + i]))
                    want = min(15, max(0, _rne_fraction((x + M) / S))) if S else 0
                    assert q[r, b, 32 * j + i] == want


def test_quantization_error_bound():
    """Inside a sub-block, |w - W^| <= S/2 + 15*|s - S| + |off - M|: half a
    step of the stored grid, plus what rounding the six-bit factors moved
    the grid's ends."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 1024)) * 0.02).astype(np.float32)
    rec = SB.quantize_q4k(w)
    what = SB.dequant_q4k(rec)
    d_bits, dmin_bits, sc, m, _ = SB.unpack_records(rec)
    wb = w.astype(np.float64).reshape(8, 4, 8, 32)
    lo = np.minimum(wb.min(axis=3), 0)
    s = (wb.max(axis=3) - lo) / 15
    S = d_bits.view(np.float16).astype(np.float64)[:, :, None] * sc
    M = dmin_bits.view(np.float16).astype(np.float64)[:, :, None] * m
    bound = S / 2 + 15 * np.abs(s - S) + np.abs(-lo - M)
    err = np.abs(wb - what.reshape(8, 4, 8, 32)).max(axis=3)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.max(err) < 0.02                      # and it is a useful bound at N(0, 0.02)


def _brute_weight(rec, r, col):
    """W^[r, col] from the record bytes, decoded here bit by bit."""
    blk = rec[r, col // 256]
    i = col % 256
    j = i // 32
    d = Fraction(float(np.array([int(blk[0]) | (int(blk[1]) << 8)], np.uint16).view(np.float16)[0]))
    dmin = Fraction(float(np.array([int(blk[2]) | (int(blk[3]) << 8)], np.uint16).view(np.float16)[0]))
    f_sc = sum(int(blk[4 + b]) << (8 * b) for b in range(6))
    f_m = sum(int(blk[10 + b]) << (8 * b) for b in range(6))
    sc, mm = (f_sc >> (6 * j)) & 63, (f_m >> (6 * j)) & 63
    code = (int(blk[16 + i // 2]) >> (4 * (i % 2))) & 15
    return d * sc * code - dmin * mm


def test_gemv_exact_brute_force():
    rng = np.random.default_rng(4)
    n, k = 3, 512
    rec = SB.quantize_q4k((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    x = F.f64_to_bf16_bits(rng.standard_normal((2, k)))
    y, a = SB.gemv_q4k(rec, x)
    xf = F.bf16_bits_to_f64(x)
    for b in range(2):
        for r in range(n):
            exact = sum(_brute_weight(rec, r, c) * Fraction(xf[b, c]) for c in range(k))
            absum = sum(abs(_brute_weight(rec, r, c) * Fraction(xf[b, c])) for c in range(k))
            assert abs(Fraction(y[b, r]) - exact) <= absum * Fraction(1, 2 ** 45)
            assert abs(Fraction(a[b, r]) - absum) <= absum * Fraction(1, 2 ** 45)


def test_gemv_one_hot_columns():
    rng = np.random.default_rng(5)
    n, k = 5, 256
    rec = SB.quantize_q4k((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    for col in (0, 31, 32, 100, 255):
        x = np.zeros((1, k))
        x[0, col] = 1.0
        y, _ = SB.gemv_q4k(rec, F.f64_to_bf16_bits(x))
        for r in range(n):
            assert Fraction(y[0, r]) == _brute_weight(rec, r, col)


def test_degenerate_super_blocks():
    w = np.zeros((2, 256), np.float32)
    w[1] = 0.25                                        # constant positive: off = 0, s = 0.25/15
    rec = SB.quantize_q4k(w)
    assert not rec[0].any()                            # all zero: d = dmin = 0, codes 0
    d_bits, dmin_bits, sc, m, q = SB.unpack_records(rec)
    assert dmin_bits[1, 0] == 0 and not m[1].any()
    assert np.all(q[1] == 15) and np.allclose(SB.dequant_q4k(rec)[1], 0.25, rtol=2e-3)


def test_repack_decodes_to_the_same_weights():
    """The device layout, decoded here from its description: code i of a row
    in bits 4(i%8) of word i//8; sub word j = sc | m << 8; super word =
    d | dmin << 16."""
    rng = np.random.default_rng(6)
    n, k = 4, 768
    rec = SB.quantize_q4k((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    codes, sub, sup = SB.repack_q4k(rec)
    assert codes.shape == (n, k // 8) and sub.shape == (n, k // 32) and sup.shape == (n, k // 256)
    assert codes.dtype == np.uint32 and sub.dtype == np.uint16 and sup.dtype == np.uint32
    col = np.arange(k)
    q = (codes[:, col // 8] >> (4 * (col % 8)).astype(np.uint32)) & 0xF
    sc = (sub[:, col // 32] & 0xFF).astype(np.float64)
    m = (sub[:, col // 32] >> 8).astype(np.float64)
    d = (sup[:, col // 256] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    dmin = (sup[:, col // 256] >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(d * sc * q - dmin * m, SB.dequant_q4k(rec))


def test_byte_counts():
    n, k = 15360, 3840
    assert SB.bytes_storage(n, k) * 8 == n * k * 4.5
    assert SB.bytes_device(n, k) * 8 == n * k * 4.625
    rec = SB.quantize_q4k(np.zeros((2, 512), np.float32))
    assert rec.nbytes == SB.bytes_storage(2, 512)
    codes, sub, sup = SB.repack_q4k(rec)
    assert codes.nbytes + sub.nbytes + sup.nbytes == SB.bytes_device(2, 512)
