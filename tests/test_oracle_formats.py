"""Pins for the oracle's number formats (CPU only).

Each check compares the oracle with something it does not contain: the golden
values the pages and the format standards fix, torch's own bf16 / float8
conversions, or exact rational arithmetic.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------- E2M1

def test_e2m1_magnitudes_match_golden_set():
    g = _golden("e2m1_values.json")
    assert list(F.E2M1_TABLE[:8]) == g["magnitudes_by_code"]


def test_e2m1_sign_is_bit3():
    g = _golden("e2m1_values.json")
    assert g["sign_bit"] == 3
    for c in range(8):
        neg = F.E2M1_TABLE[c | (1 << g["sign_bit"])]
        assert neg == -F.E2M1_TABLE[c]
        assert np.signbit(neg)          # code 8 is -0.0


def test_e2m1_magnitudes_exact_in_bf16():
    g = _golden("e2m1_values.json")
    bits = F.f64_to_bf16_bits(F.E2M1_TABLE[:8])
    assert ["0x%04X" % b for b in bits] == g["bf16_bits_by_code"]
    assert np.array_equal(F.bf16_bits_to_f64(bits), F.E2M1_TABLE[:8])


def test_e2m1_rne_tie_points():
    g = _golden("e2m1_values.json")["rne_tie_points"]
    for r, code in g.items():
        if r == "comment":
            continue
        assert F.e2m1_rne_codes(float(r)) == code, r
        assert F.e2m1_rne_codes(-float(r)) == code + 8, r


def _e2m1_brute(r):
    """Nearest E2M1 code by exhaustive exact comparison, ties to even code."""
    r = Fraction(r)
    a = min(abs(r), Fraction(6))
    best = None
    for c in range(8):
        d = abs(a - Fraction(F.e2m1_value(c)))
        key = (d, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1] + (8 if r < 0 else 0)


def test_e2m1_rne_matches_exhaustive_search():
    rng = np.random.default_rng(5)
    # a dense grid through every interval and tie, plus random values incl. > 6
    grid = np.arange(-7.0, 7.0001, 0.03125)
    rand = rng.normal(0, 3, 2000)
    vals = np.concatenate([grid, rand, [1e-30, -1e-30, 6.0001, -100.0]])
    got = F.e2m1_rne_codes(vals)
    want = np.array([_e2m1_brute(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------- E4M3

def test_e4m3_all_codes_match_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(ours)
    assert np.array_equal(lib[ok], ours[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(ours[ok]))


def test_e4m3_landmarks():
    g = _golden("e4m3_landmarks.json")
    for key in ("max_finite", "min_subnormal", "min_normal", "one", "minus_two"):
        assert F.E4M3_TABLE[int(g[key]["code"], 16)] == g[key]["value"], key
    for c in g["nan_codes"]:
        assert np.isnan(F.E4M3_TABLE[int(c, 16)])
    assert np.nanmax(F.E4M3_TABLE) == g["max_finite"]["value"]


def test_e4m3_rne_matches_torch_cast_in_range():
    rng = np.random.default_rng(6)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    vals = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    # exact ties: midpoints of neighbouring finite codes
    t = F.E4M3_TABLE[:127]
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids, -mids, np.float32([0.0, 448.0, -448.0])])
    lib = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_rne_codes(vals.astype(np.float64))
    # torch keeps the sign of -0.0 only; every non-zero value must agree bit for bit
    assert np.array_equal(ours, lib)


def test_e4m3_rne_saturates():
    assert F.e4m3_rne_codes(1e9) == 0x7E
    assert F.e4m3_rne_codes(-1e9) == 0xFE
    assert F.e4m3_rne_codes(460.0) == 0x7E


# --------------------------------------------------------------------- bf16

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = F.bf16_bits_to_f64(bits)
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(ours)
    assert np.array_equal(lib[ok], ours[ok])


def test_bf16_rne_matches_torch_on_float32():
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (low half 0x8000) with even and odd kept bits
    ties = (raw[:4000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    vals = np.concatenate([raw, ties]).view(np.float32)
    vals = vals[np.isfinite(vals)]
    extra = np.float32([0.0, -0.0, 3.3895314e38, 3.4028235e38, 1e-45, -1e-45,
                        1.1754942e-38, 9.18355e-41])
    vals = np.concatenate([vals, extra])
    lib = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = F.f64_to_bf16_bits(vals.astype(np.float64))
    assert np.array_equal(ours, lib)


def test_bf16_rne_exact_rational_ties():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7: ties to even -> 1.0
    assert F.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is the midpoint between 1+2^-7 (odd) and 1+2^-6 (even) -> up
    assert F.f64_to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above a tie rounds up; float64 input, no float32 double rounding
    assert F.f64_to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert F.f64_to_bf16_bits(float("inf")) == 0x7F80
    assert F.f64_to_bf16_bits(-float("inf")) == 0xFF80
    assert F.f64_to_bf16_bits(float("nan")) == 0x7FC0


@pytest.mark.parametrize("v", [0.1, 1.0 / 3.0, 6.02e23, 1e-39, 2.0 ** -133, 2.0 ** -134 * 3])
def test_bf16_rne_against_exact_rational(v):
    got = F.bf16_bits_to_f64(F.f64_to_bf16_bits(v))
    # exhaustively compare against the neighbouring bf16 values
    fv = Fraction(v)
    lo = Fraction(float(F.bf16_bits_to_f64(F.f64_to_bf16_bits(v) - 1)))
    hi = Fraction(float(F.bf16_bits_to_f64(F.f64_to_bf16_bits(v) + 1)))
    g = Fraction(float(got))
    assert abs(g - fv) <= abs(lo - fv) and abs(g - fv) <= abs(hi - fv)
