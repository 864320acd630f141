"""Pins for the oracle's RMSNorm (CPU only): a worked example checked by hand,
closed forms, and invariances that a dropped square, a missing square root, a
wrong mean or a misplaced gamma would break."""

import json
import os

import numpy as np

from oracle import formats as F
from oracle import norm as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    return F.f64_to_bf16_bits(np.asarray(vals, dtype=np.float64))


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "rmsnorm_hand_example.json")))
    x, gamma = _bits(g["x"]), _bits(g["gamma"])
    assert np.isclose(N.rms_factor(x, g["eps"])[0], g["r"], rtol=1e-15)
    out = N.rmsnorm_bf16(x, gamma, g["eps"])[0]
    assert [int(v) for v in out] == [int(b, 16) for b in g["expected_bits"]]
    assert list(F.bf16_bits_to_f64(out)) == g["expected_values"]


def test_constant_row_normalizes_to_sign():
    """x = c everywhere: mean(x^2) = c^2, so x~ = sign(c) exactly."""
    for c in (-2.5, 0.375, 96.0):
        x = _bits(np.full(64, c))
        out = N.rmsnorm_bf16(x, _bits(np.ones(64)), 0.0)[0]
        assert np.all(F.bf16_bits_to_f64(out) == np.sign(c))


def test_power_of_two_scaling_of_x_cancels():
    """With eps = 0 the norm is scale-free: x * 2^m gives the same bits."""
    rng = np.random.default_rng(1)
    x = _bits(rng.standard_normal((3, 384)))
    gamma = _bits(rng.uniform(0.5, 1.5, 384))
    base = N.rmsnorm_bf16(x, gamma, 0.0)
    for m in (-5, -1, 3, 7):
        xs = _bits(F.bf16_bits_to_f64(x) * 2.0 ** m)
        assert np.array_equal(N.rmsnorm_bf16(xs, gamma, 0.0), base)


def test_gamma_multiplies_the_output():
    """gamma * 2 doubles every output value exactly."""
    rng = np.random.default_rng(2)
    x = _bits(rng.standard_normal((2, 256)))
    gamma = _bits(rng.uniform(0.25, 2.0, 256))
    a = F.bf16_bits_to_f64(N.rmsnorm_bf16(x, gamma, 1e-6))
    b = F.bf16_bits_to_f64(N.rmsnorm_bf16(x, _bits(F.bf16_bits_to_f64(gamma) * 2), 1e-6))
    assert np.array_equal(b, 2 * a)


def test_unit_gamma_output_has_unit_rms():
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((4, 3840)) * 3)
    out = F.bf16_bits_to_f64(N.rmsnorm_bf16(x, _bits(np.ones(3840)), 0.0))
    rms = np.sqrt(np.mean(out * out, axis=1))
    assert np.all(np.abs(rms - 1) < 2.0 ** -8)


def test_eps_enters_under_the_root():
    """x = 0 with eps > 0 gives zeros, not NaN; a row with mean(x^2) = 3 and
    eps = 1 is divided by exactly 2."""
    z = N.rmsnorm_bf16(_bits(np.zeros(32)), _bits(np.ones(32)), 1e-5)
    assert np.all(F.bf16_bits_to_f64(z) == 0)
    x = _bits([1.0, 1.0, 1.0, 3.0])                               # mean(x^2) = 3
    out = F.bf16_bits_to_f64(N.rmsnorm_bf16(x, _bits(np.ones(4)), 1.0)[0])
    assert list(out) == [0.5, 0.5, 0.5, 1.5]


def test_batch_rows_are_independent():
    rng = np.random.default_rng(4)
    x = _bits(rng.standard_normal((3, 128)))
    gamma = _bits(rng.uniform(0.5, 1.5, 128))
    both = N.rmsnorm_bf16(x, gamma, 1e-6)
    for b in range(3):
        assert np.array_equal(N.rmsnorm_bf16(x[b], gamma, 1e-6)[0], both[b])
