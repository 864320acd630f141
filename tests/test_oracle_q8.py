"""Pins for the oracle's int8 activation route (CPU only).

The quantizer is pinned by a worked example checked by hand, by closed-form
invariants (the block maximum maps to +-127, every code is within half a step
of x / d, signs agree) and by its degenerate cases.  The block matvec is
pinned against a different formula: the dequantized weights of oracle.gemv
(pinned on their own) times the dequantized activations d * q, by exact
integer brute force where d = 1, and by the error bound of the whole route
against the bf16 product.  A dropped bias term, a wrong block-to-group map,
a transposed operand or a lost scale fails one of these.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemv as G
from oracle import layout as L
from oracle import quantize as Q
from oracle import q8 as Q8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    return F.f64_to_bf16_bits(np.asarray(vals, dtype=np.float64))


def _rng(seed):
    return np.random.default_rng(seed)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "q8_block_hand_example.json")))
    x = np.zeros(32 * len(g["x_blocks"]))
    for i, blk in enumerate(g["x_blocks"]):
        x[32 * i:32 * i + len(blk)] = blk
    q, d, s = Q8.quantize_q8_1(_bits(x)[None, :])
    for i, blk in enumerate(g["q_blocks"]):
        want = np.zeros(32, dtype=np.int64)
        want[:len(blk)] = blk
        assert list(q[0, 32 * i:32 * (i + 1)].astype(np.int64)) == list(want)
        assert d[0, i] == np.float32(g["amax"][i]) / np.float32(127) if g["amax"][i] else d[0, i] == 0
        assert int(q[0, 32 * i:32 * (i + 1)].astype(np.int64).sum()) == g["sum_q"][i]
        assert s[0, i] == np.float32(d[0, i] * np.float32(g["sum_q"][i]))


def test_block_invariants_random():
    rng = _rng(11)
    x = _bits(rng.standard_normal((3, 32 * 40)) * np.exp(rng.uniform(-8, 8, (3, 1))))
    q, d, s = Q8.quantize_q8_1(x)
    xf = F.bf16_bits_to_f64(x).reshape(3, 40, 32)
    qb = q.astype(np.int64).reshape(3, 40, 32)
    amax = np.max(np.abs(xf), axis=2)
    # the element of largest magnitude maps to +-127
    assert np.all(np.max(np.abs(qb), axis=2) == 127)
    # d is amax / 127 to fp32 precision
    assert np.allclose(d, amax / 127, rtol=2 ** -23, atol=0)
    # every code is within half a step of x / d (plus fp32 rounding of the product)
    err = np.abs(xf - d.astype(np.float64)[:, :, None] * qb)
    assert np.all(err <= d.astype(np.float64)[:, :, None] * (0.5 + 1e-5))
    # signs agree where the code is not zero
    assert np.all((qb == 0) | (np.sign(qb) == np.sign(xf)))
    # s is d times the code sum
    assert np.allclose(s, d.astype(np.float64) * qb.sum(axis=2), rtol=2 ** -23, atol=0)


def test_degenerate_blocks():
    # an all-zero row quantizes to zero codes and zero pairs
    q, d, s = Q8.quantize_q8_1(np.zeros((1, 64), dtype=np.uint16))
    assert not q.any() and not d.any() and not s.any()
    # a block of equal values maps every one to 127
    q, d, s = Q8.quantize_q8_1(_bits(np.full(32, -0.375))[None, :])
    assert np.all(q == -127) and s[0, 0] == np.float32(d[0, 0] * np.float32(-127 * 32))
    # scaling x by a power of two scales d and s and keeps the codes
    rng = _rng(5)
    x = rng.standard_normal((2, 96))
    q1, d1, s1 = Q8.quantize_q8_1(_bits(x))
    q2, d2, s2 = Q8.quantize_q8_1(_bits(x * 64.0))
    assert np.array_equal(q1, q2) and np.array_equal(d1 * 64, d2) and np.array_equal(s1 * 64, s2)


def _affine(rng, n, k, gs, bits=4):
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    codes, scales, biases = Q.quantize_affine(w, bits, gs)
    return codes, scales, biases


def _affine_u4(rng, n, k, gs):
    return _affine(rng, n, k, gs, 4)


def _q8_matvec(bits):
    return Q8.gemv_affine_u4_q8 if bits == 4 else Q8.gemv_affine_u8_q8


@pytest.mark.parametrize("bits", [4, 8])
def test_matvec_matches_dequantized_product(bits):
    """y equals W^ (oracle.gemv's dequantized weights) times x^ = d * q, up to
    the one fp32 rounding of s per block."""
    rng = _rng(7 + bits)
    for n, k, gs, bsz in [(37, 128, 64, 1), (16, 256, 32, 3), (9, 384, 128, 4)]:
        codes, scales, biases = _affine(rng, n, k, gs, bits)
        x = _bits(rng.standard_normal((bsz, k)))
        q, d, s = Q8.quantize_q8_1(x)
        y, a = _q8_matvec(bits)(codes, scales, biases, q, d, s, gs)
        w_hat = G.dequant_affine(codes, scales, biases, k, bits, gs)
        xhat = np.repeat(d.astype(np.float64), 32, axis=1) * q.astype(np.float64)
        y_ref = xhat @ w_hat.T
        bi = np.repeat(F.bf16_bits_to_f64(biases), gs, axis=1)
        # the s rounding contributes at most |bias| * |d * sum q| * 2^-24 per block
        slack = (np.abs(bi) @ np.abs(xhat).T).T * 2.0 ** -23 + 1e-12 * a
        assert np.all(np.abs(y - y_ref) <= slack), (n, k, gs, bsz)
        assert np.allclose(a, np.abs(xhat) @ np.abs(w_hat).T, rtol=1e-12)


@pytest.mark.parametrize("bits", [4, 8])
def test_matvec_integer_brute_force(bits):
    """x integer in [-127, 127] with a block maximum of 127: d = 1, q = x, s =
    sum x, and y is an exact rational sum computed term by term."""
    rng = _rng(3 + bits)
    n, k, gs = 5, 64, 32
    codes_u = rng.integers(0, 1 << bits, (n, k))
    codes = L.pack_u32(codes_u.astype(np.uint8), bits)
    scales = _bits(rng.uniform(-1, 1, (n, k // gs)))
    biases = _bits(rng.uniform(-1, 1, (n, k // gs)))
    xi = rng.integers(-127, 128, (1, k))
    xi[0, ::32] = 127
    q, d, s = Q8.quantize_q8_1(_bits(xi.astype(np.float64)))
    assert np.array_equal(q.astype(np.int64), xi) and np.all(d == 1)
    y, _ = _q8_matvec(bits)(codes, scales, biases, q, d, s, gs)
    sc = F.bf16_bits_to_f64(scales)
    bi = F.bf16_bits_to_f64(biases)
    for r in range(n):
        exact = Fraction(0)
        for c in range(k):
            g = c // gs
            exact += (Fraction(sc[r, g]) * int(codes_u[r, c]) + Fraction(bi[r, g])) * int(xi[0, c])
        assert abs(Fraction(y[0, r]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)


@pytest.mark.parametrize("bits", [4, 8])
def test_route_error_bound_against_bf16_product(bits):
    """The int8 route differs from the bf16 product by at most
    sum_k |W^| * d / 2 (each activation moves by at most half a step)."""
    rng = _rng(9 + bits)
    n, k, gs = 64, 512, 64
    codes, scales, biases = _affine(rng, n, k, gs, bits)
    x = _bits(rng.standard_normal((2, k)))
    q, d, s = Q8.quantize_q8_1(x)
    y, _ = _q8_matvec(bits)(codes, scales, biases, q, d, s, gs)
    y_bf16, _ = G.gemv_affine(codes, scales, biases, x, bits, gs)
    w_abs = np.abs(G.dequant_affine(codes, scales, biases, k, bits, gs))
    half_step = np.repeat(d.astype(np.float64), 32, axis=1) * (0.5 + 1e-5)
    bound = half_step @ w_abs.T
    assert np.all(np.abs(y - y_bf16) <= bound * (1 + 1e-9))
    # and the bound is not vacuous: the route is close to the bf16 product
    assert np.max(np.abs(y - y_bf16)) > 0
