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
import torch

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


def _f16_torch(vals):
    """float64 -> fp16 bits by torch's cast (round to nearest even): a library
    routine the oracle's numpy cast is checked against."""
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float64)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "q8_block_hand_example.json")))
    x = np.zeros(32 * len(g["x_blocks"]))
    for i, blk in enumerate(g["x_blocks"]):
        x[32 * i:32 * i + len(blk)] = blk
    bits = _bits(x)
    assert np.array_equal(F.bf16_bits_to_f64(bits), x), "the example's x must be exact in bf16"
    q, d, s = Q8.quantize_q8_1(bits[None, :])
    for i, blk in enumerate(g["q_blocks"]):
        want = np.zeros(32, dtype=np.int64)
        want[:len(blk)] = blk
        assert list(q[0, 32 * i:32 * (i + 1)].astype(np.int64)) == list(want), i
        assert int(d[0, i:i + 1].view(np.uint16)[0]) == int(g["d_fp16_bits"][i], 16), i
        assert int(s[0, i:i + 1].view(np.uint16)[0]) == int(g["s_fp16_bits"][i], 16), i
        assert int(q[0, 32 * i:32 * (i + 1)].astype(np.int64).sum()) == g["sum_q"][i]
    ds = Q8.pack_ds(d, s)
    assert ds.shape == (1, len(g["x_blocks"]), 2)
    words = ds.view(np.uint32)[..., 0]
    assert int(words[0, 0]) == (0x3A40 << 16) | 0x2000          # d low, s high


def test_pair_roundings_against_torch():
    """d and s are torch's fp16 rounding of amax / 127 and of d * sum(q)."""
    rng = _rng(13)
    x = _bits(rng.standard_normal((4, 32 * 64)) * np.exp(rng.uniform(-12, 6, (4, 64)).repeat(32, axis=1)))
    q, d, s = Q8.quantize_q8_1(x)
    xf = F.bf16_bits_to_f64(x).reshape(4, 64, 32)
    amax = np.max(np.abs(xf), axis=2)
    assert np.array_equal(d.view(np.uint16), _f16_torch(amax / 127.0))
    sq = q.astype(np.int64).reshape(4, 64, 32).sum(axis=2)
    assert np.array_equal(s.view(np.uint16), _f16_torch(d.astype(np.float64) * sq))


def test_block_invariants_random():
    rng = _rng(11)
    x = _bits(rng.standard_normal((3, 32 * 40)) * np.exp2(rng.uniform(-4, 8, (3, 1))))
    q, d, s = Q8.quantize_q8_1(x)
    xf = F.bf16_bits_to_f64(x).reshape(3, 40, 32)
    qb = q.astype(np.int64).reshape(3, 40, 32)
    df = d.astype(np.float64)
    amax = np.max(np.abs(xf), axis=2)
    assert np.all(df >= 2.0 ** -14), "these blocks keep d in the normal fp16 range"
    # d is amax / 127 to fp16 precision
    assert np.all(np.abs(df - amax / 127) <= 2.0 ** -11 * amax / 127)
    # the element of largest magnitude maps to +-127 (|amax / d - 127| < 0.1)
    assert np.all(np.max(np.abs(qb), axis=2) == 127)
    # every code is within half a step of x / d: no clamping with a normal d
    err = np.abs(xf - df[:, :, None] * qb)
    assert np.all(err <= df[:, :, None] * 0.5)
    # signs agree where the code is not zero
    assert np.all((qb == 0) | (np.sign(qb) == np.sign(xf)))
    # s is d times the code sum, to fp16 precision
    assert np.all(np.abs(s.astype(np.float64) - df * qb.sum(axis=2)) <= 2.0 ** -11 * np.abs(df * qb.sum(axis=2)))


def test_degenerate_blocks():
    # an all-zero row quantizes to zero codes and zero pairs
    q, d, s = Q8.quantize_q8_1(np.zeros((1, 64), dtype=np.uint16))
    assert not q.any() and not d.view(np.uint16).any() and not s.view(np.uint16).any()
    # a block of equal values maps every one to 127
    q, d, s = Q8.quantize_q8_1(_bits(np.full(32, -0.375))[None, :])
    assert np.all(q == -127)
    assert s.view(np.uint16)[0, 0] == _f16_torch([d.astype(np.float64)[0, 0] * (-127 * 32)])[0]
    # scaling x by a power of two scales d and s and keeps the codes (d normal)
    rng = _rng(5)
    x = rng.standard_normal((2, 96))
    q1, d1, s1 = Q8.quantize_q8_1(_bits(x))
    q2, d2, s2 = Q8.quantize_q8_1(_bits(x * 64.0))
    assert np.array_equal(q1, q2)
    assert np.array_equal(d1.astype(np.float64) * 64, d2.astype(np.float64))
    assert np.array_equal(s1.astype(np.float64) * 64, s2.astype(np.float64))
    # a block whose amax / 127 underflows fp16 to zero quantizes to zeros
    q, d, s = Q8.quantize_q8_1(_bits(np.full(32, 2.0 ** -27))[None, :])
    assert not q.any() and not d.view(np.uint16).any() and not s.view(np.uint16).any()


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
    the one fp16 rounding of s per block."""
    rng = _rng(7 + bits)
    for n, k, gs, bsz in [(37, 128, 64, 1), (16, 256, 32, 3), (9, 384, 128, 4)]:
        codes, scales, biases = _affine(rng, n, k, gs, bits)
        x = _bits(rng.standard_normal((bsz, k)))
        q, d, s = Q8.quantize_q8_1(x)
        y, a = _q8_matvec(bits)(codes, scales, biases, q, d, s, gs)
        w_hat = G.dequant_affine(codes, scales, biases, k, bits, gs)
        xhat = np.repeat(d.astype(np.float64), 32, axis=1) * q.astype(np.float64)
        y_ref = xhat @ w_hat.T
        # the fp16 rounding of s moves each block's bias term by at most
        # |bias| * (2^-11 * |d * sum q| + 2^-25)
        nblk = k // 32
        b_blk = np.abs(F.bf16_bits_to_f64(biases))[:, np.arange(nblk) * 32 // gs]        # [n, nblk]
        dsum = np.abs(d.astype(np.float64) * q.astype(np.int64).reshape(bsz, nblk, 32).sum(axis=2))
        slack = (2.0 ** -11 * dsum + 2.0 ** -25) @ b_blk.T + 1e-12 * a
        assert np.all(np.abs(y - y_ref) <= slack), (n, k, gs, bsz)
        assert np.allclose(a, np.abs(xhat) @ np.abs(w_hat).T, rtol=1e-12)


@pytest.mark.parametrize("bits", [4, 8])
def test_matvec_integer_brute_force(bits):
    """x integer with a block maximum of 127: d = 1, q = x, s = sum x (exact in
    fp16 below 2048), and y is an exact rational sum computed term by term."""
    rng = _rng(3 + bits)
    n, k, gs = 5, 64, 32
    codes_u = rng.integers(0, 1 << bits, (n, k))
    codes = L.pack_u32(codes_u.astype(np.uint8), bits)
    scales = _bits(rng.uniform(-1, 1, (n, k // gs)))
    biases = _bits(rng.uniform(-1, 1, (n, k // gs)))
    xi = rng.integers(-60, 61, (1, k))          # |block sum| < 2048: s exact in fp16
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
    sum_k |W^| * d / 2 (each activation moves by at most half a step) plus the
    fp16 rounding of s times the bias."""
    rng = _rng(9 + bits)
    n, k, gs = 64, 512, 64
    codes, scales, biases = _affine(rng, n, k, gs, bits)
    x = _bits(rng.standard_normal((2, k)))
    q, d, s = Q8.quantize_q8_1(x)
    y, _ = _q8_matvec(bits)(codes, scales, biases, q, d, s, gs)
    y_bf16, _ = G.gemv_affine(codes, scales, biases, x, bits, gs)
    w_abs = np.abs(G.dequant_affine(codes, scales, biases, k, bits, gs))
    half_step = np.repeat(d.astype(np.float64), 32, axis=1) * 0.5
    nblk = k // 32
    b_blk = np.abs(F.bf16_bits_to_f64(biases))[:, np.arange(nblk) * 32 // gs]
    dsum = np.abs(d.astype(np.float64) * q.astype(np.int64).reshape(2, nblk, 32).sum(axis=2))
    bound = half_step @ w_abs.T + (2.0 ** -11 * dsum + 2.0 ** -25) @ b_blk.T
    assert np.all(np.abs(y - y_bf16) <= bound * (1 + 1e-9))
    # and the bound is not vacuous: the route is close to the bf16 product
    assert np.max(np.abs(y - y_bf16)) > 0
