"""Pins for the oracle's dequantize-then-FP64-dot matvec (CPU only).

* Exact rational brute force on tiny shapes: every dequantized weight and every
  bf16 activation is a dyadic rational, so y can be computed exactly with
  ``fractions.Fraction``.  The brute force reads the packed bytes/words one
  element at a time with its own loops and decodes each code from its bit
  fields, so a wrong nibble order, group index, sign, dropped bias or
  transposed operand in the oracle fails here.  The oracle's float64 result
  must lie within the float64 summation bound K * 2**-53 * A of the exact one.
* One-hot activations, the integer special case and a closed-form constant
  matrix pin exact values.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import gemv as G

TWO = Fraction(2)


def _bf16(bits):
    """Exact value of a bf16 pattern from its fields (independent of numpy views)."""
    bits = int(bits)
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 0xFF, "no inf/nan in these fixtures"
    if e == 0:
        v = Fraction(m, 128) * TWO ** -126
    else:
        v = (1 + Fraction(m, 128)) * TWO ** (e - 127)
    return -v if s else v


def _e2m1(c):
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    v = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * TWO ** (e - 1)
    return -v if s else v


def _e4m3(c):
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    assert not (e == 15 and m == 7)
    v = Fraction(m, 8) * TWO ** -6 if e == 0 else (1 + Fraction(m, 8)) * TWO ** (e - 7)
    return -v if s else v


def _f32(v):
    return Fraction(float(np.float32(v)))


def _exact_y(wfun, x_bits, n, k):
    b = x_bits.shape[0]
    y = [[Fraction(0)] * n for _ in range(b)]
    a = [[Fraction(0)] * n for _ in range(b)]
    for bi in range(b):
        xs = [_bf16(x_bits[bi, kk]) for kk in range(k)]
        for nn in range(n):
            acc = Fraction(0)
            mass = Fraction(0)
            for kk in range(k):
                t = wfun(nn, kk) * xs[kk]
                acc += t
                mass += abs(t)
            y[bi][nn] = acc
            a[bi][nn] = mass
    return y, a


def _check(y, a, y_ex, a_ex, k):
    for bi in range(len(y_ex)):
        for nn in range(len(y_ex[0])):
            bound = Fraction(k + 2) * TWO ** -53 * a_ex[bi][nn]
            assert abs(Fraction(float(y[bi, nn])) - y_ex[bi][nn]) <= bound, (bi, nn)
            assert abs(Fraction(float(a[bi, nn])) - a_ex[bi][nn]) <= bound, (bi, nn)


def _rand_bf16(rng, shape, lo=-3.0, hi=3.0):
    import torch
    v = rng.uniform(lo, hi, shape).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n,k,gs,b", [(3, 64, 32, 1), (5, 128, 64, 2), (2, 256, 128, 3), (4, 32, 32, 4)])
def test_fp4_against_exact_brute_force(n, k, gs, b):
    rng = np.random.default_rng(n * 100 + k + gs)
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = _rand_bf16(rng, (n, k // gs), 0.001, 0.1)
    x = _rand_bf16(rng, (b, k))

    def w(nn, kk):
        byte = int(packed[nn, kk // 2])
        code = (byte >> 4) if kk % 2 else (byte & 0xF)
        return _bf16(scales[nn, kk // gs]) * _e2m1(code)

    y, a = G.gemv_fp4_e2m1(packed, scales, x, gs)
    _check(y, a, *_exact_y(w, x, n, k), k)


@pytest.mark.parametrize("bits,n,k,gs,b", [(4, 3, 64, 64, 1), (8, 3, 128, 64, 2),
                                           (4, 2, 256, 32, 1), (8, 2, 64, 128 // 2, 3)])
def test_affine_against_exact_brute_force(bits, n, k, gs, b):
    rng = np.random.default_rng(bits * 1000 + n + k)
    per = 32 // bits
    packed = rng.integers(0, 2 ** 32, (n, k // per), dtype=np.uint64).astype(np.uint32)
    scales = _rand_bf16(rng, (n, k // gs), 0.001, 0.05)
    biases = _rand_bf16(rng, (n, k // gs), -0.5, 0.5)
    x = _rand_bf16(rng, (b, k))

    def w(nn, kk):
        word = int(packed[nn, kk // per])
        q = (word >> (bits * (kk % per))) & ((1 << bits) - 1)
        g = kk // gs
        return _bf16(scales[nn, g]) * q + _bf16(biases[nn, g])

    y, a = G.gemv_affine(packed, scales, biases, x, bits, gs)
    _check(y, a, *_exact_y(w, x, n, k), k)


@pytest.mark.parametrize("n,k,b", [(3, 48, 1), (4, 16, 4), (2, 96, 2)])
def test_fp8_against_exact_brute_force(n, k, b):
    rng = np.random.default_rng(n * 7 + k)
    codes = rng.integers(0, 256, (n, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes in this fixture
    row_scale = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    x = _rand_bf16(rng, (b, k))

    def w(nn, kk):
        return _f32(row_scale[nn]) * _e4m3(int(codes[nn, kk]))

    y, a = G.gemv_fp8_e4m3(codes, row_scale, x)
    _check(y, a, *_exact_y(w, x, n, k), k)


def _one_hot_bf16(k, j):
    x = np.zeros((1, k), dtype=np.uint16)
    x[0, j] = 0x3F80                                # 1.0
    return x


def test_fp4_one_hot_reads_column_exactly():
    rng = np.random.default_rng(11)
    n, k, gs = 6, 128, 32
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = _rand_bf16(rng, (n, k // gs), 0.01, 1.0)
    w_hat = G.dequant_fp4_e2m1(packed, scales, k, gs)
    for j in (0, 1, 31, 32, 63, 127):
        y, _ = G.gemv_fp4_e2m1(packed, scales, _one_hot_bf16(k, j), gs)
        assert np.array_equal(y[0], w_hat[:, j])


def test_affine_integer_special_case_is_integer_matvec():
    # s = 1, b = 0 and small-integer x: y is an exact integer matvec
    rng = np.random.default_rng(12)
    for bits in (4, 8):
        n, k, gs = 5, 256, 64
        q = rng.integers(0, 1 << bits, (n, k))
        from oracle.layout import pack_u32
        packed = pack_u32(q.astype(np.uint8), bits)
        ones = np.full((n, k // gs), 0x3F80, dtype=np.uint16)
        zeros = np.zeros((n, k // gs), dtype=np.uint16)
        xi = rng.integers(-8, 9, (2, k))
        import torch
        xb = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        y, a = G.gemv_affine(packed, ones, zeros, xb, bits, gs)
        assert np.array_equal(y, (xi @ q.T).astype(np.float64))
        assert np.array_equal(a, (np.abs(xi) @ q.T).astype(np.float64))


def test_fp4_constant_matrix_closed_form():
    # every code = c, every scale = s, x = ones: y = K * s * E2M1(c)
    n, k, gs = 4, 96, 32
    for c, val in [(1, 0.5), (7, 6.0), (13, -3.0), (8, -0.0)]:
        packed = np.full((n, k // 2), c | (c << 4), dtype=np.uint8)
        scales = np.full((n, k // gs), 0x3E80, dtype=np.uint16)    # 0.25
        x = np.full((1, k), 0x3F80, dtype=np.uint16)
        y, a = G.gemv_fp4_e2m1(packed, scales, x, gs)
        assert np.all(y == k * 0.25 * val)
        assert np.all(a == k * 0.25 * abs(val))


def test_batch_rows_are_independent():
    rng = np.random.default_rng(13)
    n, k = 7, 64
    codes = rng.integers(0, 0x7E, (n, k), dtype=np.uint8)
    rs = rng.uniform(0.01, 1, n).astype(np.float32)
    x = _rand_bf16(rng, (4, k))
    y4, a4 = G.gemv_fp8_e4m3(codes, rs, x)
    for b in range(4):
        y1, a1 = G.gemv_fp8_e4m3(codes, rs, x[b:b + 1])
        assert np.array_equal(y1[0], y4[b]) and np.array_equal(a1[0], a4[b])


def test_row_blocking_does_not_change_result(monkeypatch):
    rng = np.random.default_rng(14)
    n, k, gs = 37, 64, 32
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = _rand_bf16(rng, (n, k // gs), 0.01, 1.0)
    x = _rand_bf16(rng, (1, k))
    y_full, _ = G.gemv_fp4_e2m1(packed, scales, x, gs)
    monkeypatch.setattr(G, "ROW_BLOCK", 5)
    y_blk, _ = G.gemv_fp4_e2m1(packed, scales, x, gs)
    assert np.array_equal(y_full, y_blk)


def test_shape_mismatch_raises():
    with pytest.raises(ValueError):
        G.gemv_fp4_e2m1(np.zeros((2, 16), np.uint8), np.zeros((2, 2), np.uint16),
                        np.zeros((1, 32), np.uint16), 32)
    with pytest.raises(ValueError):
        G.gemv_fp8_e4m3(np.zeros((2, 16), np.uint8), np.zeros(2, np.float32),
                        np.zeros((1, 15), np.uint16))
