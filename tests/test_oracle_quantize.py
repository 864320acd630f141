"""Pins for the oracle's offline quantizers (CPU only).

* Exhaustive exact search on small inputs: for every weight, the code the
  quantizer picked is the nearest representable value under the stated
  rounding rule, found by trying every code with rational arithmetic.
* Invariants fixed by the definitions (absmax element -> +-6 / +-448, error
  bounds, all-zero groups).
* The pages' own byte accounting (#683): the affine group-64 layout must cost
  8.5 bits per weight at 8 bits and 4.5 at 4 bits, and with the 144 MLP modules
  of gemma-4-12b that reproduces the printed checkpoint shrink and the ~9 GB of
  8-bit MLP bytes.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q
from oracle.layout import unpack_nibbles, unpack_u32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gauss(n, k, seed, std=0.02):
    return np.random.default_rng(seed).normal(0, std, (n, k)).astype(np.float32)


def _bf16_exact(bits):
    return Fraction(float(F.bf16_bits_to_f64(np.uint16(bits))))


def _nearest_bf16(v):
    """Nearest bf16 to a rational v by scanning the neighbouring patterns."""
    v = Fraction(v)
    approx = int(F.f64_to_bf16_bits(float(v)))
    best = None
    for cand in range(max(0, (approx & 0x7FFF) - 2), min(0x7F80, (approx & 0x7FFF) + 3)):
        bits = cand | (0x8000 if v < 0 else 0)
        d = abs(_bf16_exact(bits) - v)
        key = (d, cand % 2)
        if best is None or key < best[0]:
            best = (key, bits)
    return best[1]


# --------------------------------------------------------------------- FP4

@pytest.mark.parametrize("gs", [32, 64, 128])
def test_fp4_quantizer_exhaustive(gs):
    w = _gauss(3, 256, gs)
    codes, scales = Q.quantize_fp4_e2m1(w, gs)
    c = unpack_nibbles(codes, 256)
    for n in range(3):
        for g in range(256 // gs):
            grp = [Fraction(float(v)) for v in w[n, g * gs:(g + 1) * gs]]
            s_bits = _nearest_bf16(max(abs(v) for v in grp) / 6)
            assert scales[n, g] == s_bits
            s = _bf16_exact(s_bits)
            for i, v in enumerate(grp):
                r = v / s
                a = min(abs(r), Fraction(6))
                best = min(range(8), key=lambda cc: (abs(a - Fraction(F.e2m1_value(cc))), cc % 2))
                assert c[n, g * gs + i] == best + (8 if v < 0 else 0)


def test_fp4_absmax_maps_to_six_and_error_bound():
    w = _gauss(64, 512, 1)
    codes, scales = Q.quantize_fp4_e2m1(w, 32)
    c = unpack_nibbles(codes, 512).reshape(64, 16, 32)
    s = F.bf16_bits_to_f64(scales)
    wg = w.astype(np.float64).reshape(64, 16, 32)
    am = np.abs(wg).argmax(axis=-1)
    top = np.take_along_axis(c, am[..., None], -1)[..., 0]
    assert np.all((top & 7) == 7)                         # magnitude 6
    w_hat = s[..., None] * F.E2M1_TABLE[c]
    # largest gap between neighbouring magnitudes is 2 (between 4 and 6)
    assert np.all(np.abs(wg - w_hat) <= s[..., None] * 1.0 + 1e-30)
    assert c.max() <= 15


def test_fp4_zero_group():
    w = _gauss(2, 64, 2)
    w[1, 32:] = 0.0
    codes, scales = Q.quantize_fp4_e2m1(w, 32)
    assert scales[1, 1] == 0
    assert np.all(unpack_nibbles(codes, 64)[1, 32:] == 0)


# --------------------------------------------------------------------- affine

@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 64), (4, 32)])
def test_affine_quantizer_exhaustive(bits, gs):
    w = _gauss(2, 128, bits + gs)
    codes, scales, biases = Q.quantize_affine(w, bits, gs)
    q = unpack_u32(codes, 128, bits)
    qmax = (1 << bits) - 1
    for n in range(2):
        for g in range(128 // gs):
            grp = [Fraction(float(v)) for v in w[n, g * gs:(g + 1) * gs]]
            mn, mx = min(grp), max(grp)
            s_bits = _nearest_bf16((mx - mn) / qmax)
            b_bits = _nearest_bf16(mn)
            assert scales[n, g] == s_bits and biases[n, g] == b_bits
            s, b = _bf16_exact(s_bits), _bf16_exact(b_bits)
            for i, v in enumerate(grp):
                # nearest integer level, ties to even, clamped to [0, qmax]
                t = (v - b) / s
                best = min(range(qmax + 1), key=lambda qq: (abs(t - qq), qq % 2))
                assert q[n, g * gs + i] == best


def test_affine_invariants_on_gaussian_weights():
    w = _gauss(128, 512, 3)
    for bits in (4, 8):
        codes, scales, biases = Q.quantize_affine(w, bits, 64)
        q = unpack_u32(codes, 512, bits).reshape(128, 8, 64).astype(np.float64)
        s = F.bf16_bits_to_f64(scales)[..., None]
        b = F.bf16_bits_to_f64(biases)[..., None]
        wg = w.astype(np.float64).reshape(128, 8, 64)
        qmax = (1 << bits) - 1
        # min element -> level 0 and max element -> top level.  Rounding s and b to
        # bf16 (half an ulp = 2**-8 relative) moves the ends by at most
        # (|b| + qmax*s) * 2**-8, which is under half a level at 4 bits but can
        # reach one level at 8 bits.
        amin = wg.argmin(-1)[..., None]
        amax = wg.argmax(-1)[..., None]
        ends = 0 if bits == 4 else 1
        assert np.all(np.take_along_axis(q, amin, -1) <= ends)
        assert np.all(np.take_along_axis(q, amax, -1) >= qmax - ends)
        err = np.abs(wg - (s * q + b))
        slack = (np.abs(b) + qmax * s) * 2.0 ** -8
        assert np.all(err <= s / 2 + slack)
        if bits == 4:
            # N(0, 0.02), group 64, 4-bit: the largest reconstruction error
            # stays near half a level (~3e-3)
            assert err.max() < 6e-3


def test_affine_constant_group():
    w = np.full((1, 64), 0.125, dtype=np.float32)
    codes, scales, biases = Q.quantize_affine(w, 4, 64)
    assert scales[0, 0] == 0 and biases[0, 0] == 0x3E00
    assert np.all(codes == 0)


# --------------------------------------------------------------------- FP8

def test_fp8_quantizer_exhaustive_small():
    w = _gauss(4, 32, 4)
    codes, rs = Q.quantize_fp8_e4m3_rowwise(w)
    for n in range(4):
        absmax = np.abs(w[n]).max()
        assert rs[n] == np.float32(absmax) / np.float32(448.0)
        s = Fraction(float(rs[n]))
        for kk in range(32):
            r = Fraction(float(w[n, kk])) / s
            a = min(abs(r), Fraction(448))
            best = min(range(127), key=lambda cc: (abs(a - Fraction(F.e4m3_value(cc))), cc % 2))
            assert codes[n, kk] == best + (128 if r < 0 else 0)


def test_fp8_row_absmax_maps_to_448():
    w = _gauss(32, 3840, 5)
    codes, rs = Q.quantize_fp8_e4m3_rowwise(w)
    am = np.abs(w).argmax(axis=1)
    top = codes[np.arange(32), am]
    assert np.all((top & 0x7F) == 0x7E)
    assert not np.any((codes & 0x7F) == 0x7F)


def test_quantizers_reject_bad_input():
    with pytest.raises(ValueError):
        Q.quantize_fp4_e2m1(np.zeros((2, 48), np.float32), 32)
    with pytest.raises(ValueError):
        Q.quantize_affine(np.zeros((2, 64), np.float64), 4, 64)
    bad = np.zeros((1, 64), np.float32)
    bad[0, 3] = np.inf
    with pytest.raises(ValueError):
        Q.quantize_fp8_e4m3_rowwise(bad)


# --------------------------------------------------------------------- pages' bytes

def _bits_per_weight_affine(bits, gs=64):
    w = _gauss(4, 256, 9)
    codes, scales, biases = Q.quantize_affine(w, bits, gs)
    return 8.0 * (codes.nbytes + scales.nbytes + biases.nbytes) / w.size


def test_affine_layout_bytes_match_paper_accounting():
    g = json.load(open(os.path.join(GOLDEN, "paper_byte_accounting.json")))
    assert _bits_per_weight_affine(8) == 8.5
    assert _bits_per_weight_affine(4) == 4.5
    weights = g["modules"] * g["module_rows"] * g["module_cols"]
    gb8 = weights * 8.5 / 8 / 1e9
    gb4 = weights * 4.5 / 8 / 1e9
    # "~9 GB" of 8-bit MLP bytes
    assert abs(gb8 - g["mlp_8bit_gb_approx"]) <= g["approx_tolerance_gb"]
    # requantizing those modules to 4-bit shrinks the checkpoint 10.99 -> 6.74 GB
    shrink = g["checkpoint_gb_before"] - g["checkpoint_gb_after"]
    assert abs((gb8 - gb4) - shrink) <= g["printed_digits_gb"]


def test_fp4_layout_is_4_5_bits_per_weight_at_group_32():
    w = _gauss(4, 256, 10)
    codes, scales = Q.quantize_fp4_e2m1(w, 32)
    assert 8.0 * (codes.nbytes + scales.nbytes) / w.size == 4.5
