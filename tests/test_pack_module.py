"""The library's host pack module (C++) against the oracle (CPU only).

Quantizers, packers and layout sizes are integer/byte work: bit-exact.
"""

import numpy as np
import pytest

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import layout as L
from oracle import quantize as Q


def _edge_weights(n, k, seed):
    w = synth.uniform_f32((n, k), -1.0, 1.0, seed) * np.float32(0.05)
    w[0, :] = 0.0                                  # all-zero groups
    w[1, :32] = np.float32(1e-41)                  # subnormal inputs -> zero/subnormal scales
    w[2, :] = np.float32(3e38) * np.sign(w[2, :])  # huge values
    w[3, :64] = np.float32(0.125)                  # constant group (affine s = 0)
    # exact FP4 tie points against scale 1/6 * 6 = 1: absmax 6 -> s = 1
    ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0], np.float32)
    w[4, :ties.size] = ties
    return w


@pytest.mark.parametrize("gs", [32, 64, 128])
def test_fp4_quantizer_matches_oracle(gs):
    for w in (synth.weights(1, 512, 512), _edge_weights(8, 256, gs)):
        c1, s1 = q.qg_quantize_fp4_e2m1(w, gs)
        c2, s2 = Q.quantize_fp4_e2m1(w, gs)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 64), (4, 32), (8, 128)])
def test_affine_quantizer_matches_oracle(bits, gs):
    for w in (synth.weights(5, 512, 512), _edge_weights(8, 256, bits + gs)):
        a = q.qg_quantize_affine(w, bits, gs)
        b = Q.quantize_affine(w, bits, gs)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


def test_fp8_quantizer_matches_oracle():
    for w in (synth.weights(9, 512, 640), _edge_weights(8, 256, 3)):
        a = q.qg_quantize_fp8_e4m3_rowwise(w)
        b = Q.quantize_fp8_e4m3_rowwise(w)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_ties_match_oracle():
    # row absmax 448 -> s = 1 exactly; then every E4M3 midpoint is an exact tie
    from oracle.formats import E4M3_TABLE
    t = E4M3_TABLE[:127]
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    w = np.zeros((2, 256), np.float32)
    w[:, 0] = 448.0
    w[0, 1:1 + mids.size] = mids
    w[1, 1:1 + mids.size] = -mids
    a = q.qg_quantize_fp8_e4m3_rowwise(w)
    b = Q.quantize_fp8_e4m3_rowwise(w)
    assert a[1][0] == 1.0
    assert np.array_equal(a[0], b[0])


def test_pack_unpack_match_oracle_layout():
    rng = np.random.default_rng(1)
    c4 = rng.integers(0, 16, (6, 64), dtype=np.uint8)
    assert np.array_equal(q.qg_pack_nibbles(c4).reshape(6, 32), L.pack_nibbles(c4))
    assert np.array_equal(q.qg_unpack_nibbles(L.pack_nibbles(c4), c4.size).reshape(6, 64), c4)
    for bits in (4, 8):
        c = rng.integers(0, 1 << bits, (6, 64), dtype=np.uint8)
        assert np.array_equal(q.qg_pack_u32(c, bits).reshape(6, -1), L.pack_u32(c, bits))
        assert np.array_equal(q.qg_unpack_u32(L.pack_u32(c, bits), c.size, bits).reshape(6, 64), c)


def test_bytes_closed_forms():
    for n, k in [(30720, 3840), (3840, 15360), (1, 32)]:
        assert q.qg_bytes_fp4(n, k, 32) == n * k // 2 + n * (k // 32) * 2
        if k % 64 == 0:
            assert q.qg_bytes_affine(n, k, 4, 64) == n * k // 2 + n * (k // 64) * 4
            assert q.qg_bytes_affine(n, k, 8, 64) == n * k + n * (k // 64) * 4
        else:
            assert q.qg_bytes_affine(n, k, 4, 64) == -1
        assert q.qg_bytes_fp8(n, k) == n * k + 4 * n
    # the packed arrays the oracle quantizer returns have exactly these sizes
    w = synth.weights(2, 64, 256)
    c, s = Q.quantize_fp4_e2m1(w, 32)
    assert c.nbytes + s.nbytes == q.qg_bytes_fp4(64, 256, 32)
    c, s, b = Q.quantize_affine(w, 8, 64)
    assert c.nbytes + s.nbytes + b.nbytes == q.qg_bytes_affine(64, 256, 8, 64)
    assert q.qg_bytes_fp4(4, 48, 32) == -1 and q.qg_bytes_affine(4, 64, 3, 64) == -1


def test_pack_module_errors():
    with pytest.raises(q.QgError) as e:
        q.qg_quantize_fp4_e2m1(np.zeros((2, 48), np.float32), 32)
    assert e.value.name == "QG_ERR_BAD_GROUP_SIZE"
    bad = np.zeros((2, 64), np.float32)
    bad[1, 5] = np.nan
    for fn in (lambda: q.qg_quantize_fp4_e2m1(bad, 32), lambda: q.qg_quantize_affine(bad, 4, 64),
               lambda: q.qg_quantize_fp8_e4m3_rowwise(bad)):
        with pytest.raises(q.QgError) as e:
            fn()
        assert e.value.name == "QG_ERR_BAD_VALUE"
    with pytest.raises(q.QgError) as e:
        q.qg_quantize_affine(np.zeros((2, 64), np.float32), 3, 64)
    assert e.value.name == "QG_ERR_BAD_BITS"
    with pytest.raises(q.QgError) as e:
        q.qg_pack_nibbles(np.array([1, 16], np.uint8))
    assert e.value.name == "QG_ERR_BAD_VALUE"


def test_q4k_quantizer_and_repack_match_oracle():
    """The library's two-level quantizer writes the oracle's storage records
    bit for bit, and its repack the oracle's device layout."""
    from oracle import superblock as SB
    golden = np.zeros((1, 256), np.float32)
    golden[0, :32] = np.arange(32) % 16 / 4.0
    for w in (synth.weights(11, 300, 768), _edge_weights(8, 512, 7), golden,
              (synth.weights(12, 64, 256) * np.float32(1e-3))):   # fp16-subnormal d
        rec = q.qg_quantize_q4k(w)
        ref = SB.quantize_q4k(w)
        assert np.array_equal(rec, ref)
        for u, v in zip(q.qg_repack_q4k(rec), SB.repack_q4k(ref)):
            assert u.dtype == v.dtype and np.array_equal(u, v)
    assert q.qg_bytes_q4k(15360, 3840) == SB.bytes_device(15360, 3840)
    assert q.qg_bytes_q4k_records(15360, 3840) == SB.bytes_storage(15360, 3840)
    assert q.qg_bytes_q4k(8, 100) == -1 and q.qg_bytes_q4k_records(8, 100) == -1
    with pytest.raises(q.QgError):
        q.qg_quantize_q4k(np.zeros((2, 128), np.float32))          # k not a multiple of 256
