"""The int8 activation route for affine 4-bit and 8-bit weights on the GPU,
through the C ABI (qg_quantize_q8_1, qgemv_affine_u{4,8}_q8 and their fused
forms), against oracle.q8.

* The quantizer's codes and fp16 {d, s} pairs are the decisions of exact
  arithmetic on both sides (float64 in the oracle, correctly rounded fp32
  quotients on the GPU): compared bit for bit.
* The matvec gets the oracle's own quantized activations (never the GPU's)
  and meets the parity criterion against the float64 block sum.
* End to end (GPU quantize, then GPU matvec) equals the matvec on the
  oracle's blocks bitwise, since the blocks are equal.
* The full-size affine shapes run in the launch configuration the bench
  times, checked on a seeded sample of rows.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import formats as F
from oracle import quantize as Q
from oracle import q8 as Q8
from tests import parity
from tests.gpu_util import dev, host_y, log, out_tensor, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _x_blocks(seed, batch, k):
    """N(0, 1) activations with a per-block magnitude spread over 2^-14..2^6
    (the small blocks have fp16-subnormal d), some all-zero blocks, a block
    whose d underflows to zero, and a block whose quotients land on .5 ties."""
    rng = np.random.default_rng([0, 55, seed, batch, k])
    x = rng.standard_normal((batch, k)).astype(np.float32)
    x *= np.repeat(np.exp2(rng.integers(-14, 7, (batch, k // 32))), 32, axis=1).astype(np.float32)
    nb = k // 32
    if nb > 2:
        x[:, 32:64] = 0.0                                      # an all-zero block
        # ties: amax = 127/64 gives d = 2^-6 exactly, and x = (2m+1)/128
        # (exact in bf16) gives x / d = m + 1/2, rounded to the even neighbour
        x[0, 64] = 127.0 / 64.0
        x[0, 65:96] = (2.0 * (np.arange(31) - 15) + 1.0) / 128.0
    if nb > 3:
        x[-1, 96:128] = 2.0 ** -27                             # amax / 127 below fp16: d = 0
    return F.f64_to_bf16_bits(x.astype(np.float64))


def _ds(d_ref, s_ref):
    """The oracle's pairs in the library's layout (fp16 bits, d then s)."""
    return Q8.pack_ds(d_ref, s_ref)


def _gpu_quantize(x_bits):
    xq, ds = q.qg_quantize_q8_1(dev(x_bits))
    torch.cuda.synchronize()
    return xq.cpu().numpy(), ds.cpu().numpy()


@pytest.mark.parametrize("batch,k", [(1, 32), (1, 96), (3, 3840), (4, 4096), (2, 15360), (4, 15360)])
def test_quantize_bitwise(batch, k):
    log("q8 quantize batch=%d k=%d" % (batch, k))
    x = _x_blocks(1, batch, k)
    xq, ds = _gpu_quantize(x)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    assert np.array_equal(xq, q_ref)
    assert np.array_equal(ds.view(np.uint16), _ds(d_ref, s_ref))


def _weights(seed, n, k, gs, bits=4):
    w = synth.weights(300 + seed, n, k)
    return Q.quantize_affine(w, bits, gs)


def _fns(bits):
    if bits == 4:
        return q.qgemv_affine_u4_q8, q.qgemv_affine_u4_q8_fused
    return q.qgemv_affine_u8_q8, q.qgemv_affine_u8_q8_fused


def _matvec(arrays, xq, ds, n, gs, bf16=False, bits=4):
    y = out_tensor(xq.shape[0], n, bf16)
    _fns(bits)[0](dev(arrays[0]), dev(arrays[1]), dev(arrays[2]), dev(xq), dev(ds), y, gs)
    return host_y(y)


@pytest.mark.parametrize("n,k,gs,batch", [
    (1, 32, 32, 1), (37, 128, 64, 1), (250, 3840, 64, 4), (129, 4096, 128, 3),
    (300, 15360, 64, 2), (64, 15360, 32, 4), (1000, 512, 64, 1),
    # at least 4 rows per wave: 4-row tiles (8200, 9001: ragged)
    (8200, 512, 64, 3), (9001, 256, 32, 4), (8200, 256, 64, 1), (9001, 512, 128, 2),
])
@pytest.mark.parametrize("bits", [4, 8])
def test_matvec_parity(bits, n, k, gs, batch):
    log("q8 matvec u%d n=%d k=%d gs=%d batch=%d" % (bits, n, k, gs, batch))
    arrays = _weights(n + k, n, k, gs, bits)
    x = _x_blocks(2, batch, k)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    ds = _ds(d_ref, s_ref)
    y = _matvec(arrays, q_ref, ds, n, gs, bits=bits)
    y_ref, a_ref = Q8.gemv_affine_q8(arrays[0], arrays[1], arrays[2], q_ref, d_ref, s_ref, bits, gs)
    parity.assert_parity(y, y_ref, a_ref, "u%d q8 n=%d k=%d" % (bits, n, k))
    # bf16 output is the rounding of the same sums
    yb = _matvec(arrays, q_ref, ds, n, gs, bf16=True, bits=bits)
    yf = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, yf)


def test_end_to_end_equals_oracle_blocks():
    n, k, gs, batch = 513, 3840, 64, 4
    log("q8 end to end n=%d k=%d batch=%d" % (n, k, batch))
    arrays = _weights(9, n, k, gs)
    x = _x_blocks(3, batch, k)
    dargs = [dev(a) for a in arrays]
    xq, ds = q.qg_quantize_q8_1(dev(x))
    y = out_tensor(batch, n)
    q.qgemv_affine_u4_q8(dargs[0], dargs[1], dargs[2], xq, ds, y, gs)
    y_gpu = host_y(y)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    y_blocks = _matvec(arrays, q_ref, _ds(d_ref, s_ref), n, gs)
    assert np.array_equal(y_gpu, y_blocks)
    y_ref, a_ref = Q8.gemv_affine_u4_q8(arrays[0], arrays[1], arrays[2], q_ref, d_ref, s_ref, gs)
    parity.assert_parity(y_gpu, y_ref, a_ref, "u4 q8 end to end")


@pytest.mark.parametrize("n,k,gs,batch", [
    (1, 32, 32, 1), (37, 128, 64, 2), (513, 3840, 64, 4), (129, 4096, 128, 3), (300, 15360, 64, 1),
    (64, 15360, 32, 4), (1000, 8192, 64, 1), (8200, 512, 64, 3), (9001, 1024, 128, 4), (8200, 256, 32, 1),
    (9001, 512, 64, 2),
])
@pytest.mark.parametrize("bits", [4, 8])
def test_fused_equals_separate_bitwise(bits, n, k, gs, batch):
    """The in-kernel quantization stages the same blocks as qg_quantize_q8_1,
    so the fused call returns the two-launch result bit for bit."""
    log("q8 fused u%d n=%d k=%d gs=%d batch=%d" % (bits, n, k, gs, batch))
    arrays = _weights(7 * n + k, n, k, gs, bits)
    sep, fused = _fns(bits)
    x = _x_blocks(5, batch, k)
    dargs = [dev(a) for a in arrays]
    xd = dev(x)
    xq, ds = q.qg_quantize_q8_1(xd)
    y_sep = out_tensor(batch, n)
    sep(dargs[0], dargs[1], dargs[2], xq, ds, y_sep, gs)
    y_fused = out_tensor(batch, n)
    fused(dargs[0], dargs[1], dargs[2], xd, y_fused, gs)
    a, b = host_y(y_sep), host_y(y_fused)
    assert np.array_equal(a, b)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    y_ref, a_ref = Q8.gemv_affine_q8(arrays[0], arrays[1], arrays[2], q_ref, d_ref, s_ref, bits, gs)
    parity.assert_parity(b, y_ref, a_ref, "u%d q8 fused n=%d k=%d" % (bits, n, k))


@pytest.mark.parametrize("bits", [4, 8])
def test_all_codes_and_zero_blocks(bits):
    """Uniform random code words (every code value) and an activation with
    all-zero blocks: the zero blocks add nothing, bias terms included."""
    n, k, gs = 96, 1024, 64
    log("q8 uniform codes u%d n=%d k=%d" % (bits, n, k))
    codes = synth.uniform_words((n, k * bits // 32), 21)
    scales = synth.uniform_bf16((n, k // gs), -0.05, 0.05, 22)
    biases = synth.uniform_bf16((n, k // gs), -0.05, 0.05, 23)
    x = _x_blocks(4, 2, k)
    x[1, :] = 0
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    y = _matvec((codes, scales, biases), q_ref, _ds(d_ref, s_ref), n, gs, bits=bits)
    y_ref, a_ref = Q8.gemv_affine_q8(codes, scales, biases, q_ref, d_ref, s_ref, bits, gs)
    parity.assert_parity(y, y_ref, a_ref, "u%d q8 uniform codes" % bits)
    assert np.all(y[1] == 0)


def test_errors_leave_y_untouched():
    n, k, gs = 8, 64, 64
    arrays = [dev(a) for a in _weights(1, n, k, gs)]
    xq = torch.zeros((1, k), dtype=torch.int8, device="cuda:0")
    ds = torch.zeros((1, k // 32, 2), dtype=torch.int16, device="cuda:0")
    y = out_tensor(1, n, fill=7.0)
    lib = q.lib()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())   # noqa: E731
    s = ctypes.c_void_p(0)
    assert lib.qgemv_affine_u4_q8(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xq), p(ds), p(y),
                                  n, 48, gs, 1, 0, s) != 0                       # k not a block multiple
    assert lib.qgemv_affine_u4_q8(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xq), p(ds), p(y),
                                  n, k, 48, 1, 0, s) != 0                        # bad group size
    assert lib.qgemv_affine_u4_q8(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xq), p(ds), p(y),
                                  n, k, gs, 5, 0, s) != 0                        # batch 5
    assert lib.qgemv_affine_u4_q8(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xq), p(ds), p(y),
                                  n, 65536 * 2, gs, 1, 0, s) != 0                # beyond the LDS staging
    assert lib.qg_quantize_q8_1(p(xq), 48, 1, p(xq), p(ds), s) != 0
    assert lib.qgemv_affine_u8_q8(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xq), p(ds), p(y),
                                  n, k, gs, 5, 0, s) != 0                        # batch 5
    xb = torch.zeros((1, k), dtype=torch.bfloat16, device="cuda:0")
    assert lib.qgemv_affine_u8_q8_fused(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xb), p(y),
                                        n, 48, gs, 1, 0, s) != 0                 # k not a block multiple
    assert lib.qgemv_affine_u4_q8_fused(p(arrays[0]), p(arrays[1]), p(arrays[2]), p(xb), p(y),
                                        n, k, gs, 0, 0, s) != 0                  # batch 0
    assert lib.qgemv_affine_u4_q8_fused(p(arrays[0]), p(arrays[1]), p(arrays[2]), None, p(y),
                                        n, k, gs, 1, 0, s) != 0                  # null x
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("name", ["mlp_up", "mlp_down"])
@pytest.mark.parametrize("bits", [4, 8])
def test_full_size_sampled(bits, name, batch):
    sid, n, k = synth.shape(name)
    gs = 64
    log("q8 full-size u%d %s [%d x %d] batch=%d" % (bits, name, n, k, batch))
    w = synth.weights(sid, n, k)
    arrays = q.qg_quantize_affine(w, bits, gs)
    sep = _fns(bits)[0]
    del w
    x = synth.activations(sid, batch, k)
    dargs = [dev(a) for a in arrays]
    xq, ds = q.qg_quantize_q8_1(dev(x))
    y = out_tensor(batch, n)
    sep(dargs[0], dargs[1], dargs[2], xq, ds, y, gs)
    y1 = host_y(y)
    y2t = out_tensor(batch, n)
    sep(dargs[0], dargs[1], dargs[2], xq, ds, y2t, gs)
    y2 = host_y(y2t)
    assert np.isfinite(y1).all() and np.array_equal(y1, y2)
    rows = synth.sample_rows(n, 192, seed=sid)
    ora = Q.quantize_affine(synth.weight_rows(sid, n, k, rows), bits, gs)
    for a_lib, a_ora in zip(arrays, ora):
        assert np.array_equal(a_lib[rows], a_ora)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    y_ref, a_ref = Q8.gemv_affine_q8(ora[0], ora[1], ora[2], q_ref, d_ref, s_ref, bits, gs)
    r = parity.assert_parity(y1[:, rows], y_ref, a_ref, "u%d q8 %s" % (bits, name))
    log("q8 full-size u%d %s: %r" % (bits, name, r))


@pytest.mark.parametrize("bits", [4, 8])
def test_largest_staged_k(bits):
    """batch 4 at the largest k whose int8 blocks fit the 128 KiB staging
    (4 * k * 1.125 bytes: k = 29120 with groups of 32), plain and fused, and
    the next block multiple is refused before any launch."""
    n, k, gs, batch = 70, 29120, 32, 4
    log("q8 largest k u%d n=%d k=%d batch=%d" % (bits, n, k, batch))
    arrays = _weights(11 + bits, n, k, gs, bits)
    x = _x_blocks(6, batch, k)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    y_ref, a_ref = Q8.gemv_affine_q8(arrays[0], arrays[1], arrays[2], q_ref, d_ref, s_ref, bits, gs)
    sep, fused = _fns(bits)
    dargs = [dev(a) for a in arrays]
    y = out_tensor(batch, n)
    sep(dargs[0], dargs[1], dargs[2], dev(q_ref), dev(_ds(d_ref, s_ref)), y, gs)
    parity.assert_parity(host_y(y), y_ref, a_ref, "u%d q8 largest k" % bits)
    yf = out_tensor(batch, n)
    fused(dargs[0], dargs[1], dargs[2], dev(x), yf, gs)
    parity.assert_parity(host_y(yf), y_ref, a_ref, "u%d q8 fused largest k" % bits)
    # k + 32 no longer fits: QG_ERR_TOO_LARGE, y untouched
    k2 = k + 32
    arrays2 = [dev(a) for a in _weights(12 + bits, n, k2, gs, bits)]
    y2 = out_tensor(batch, n, fill=3.0)
    with pytest.raises(q.QgError) as err:
        fused(arrays2[0], arrays2[1], arrays2[2], dev(_x_blocks(7, batch, k2)), y2, gs)
    assert err.value.status == 9
    torch.cuda.synchronize()
    assert torch.all(y2 == 3.0)


def test_quantize_long_rows_bitwise():
    """The standalone quantizer has no staging limit: 4 rows of 2^18."""
    batch, k = 4, 1 << 18
    log("q8 quantize long rows batch=%d k=%d" % (batch, k))
    x = _x_blocks(8, batch, k)
    xq, ds = _gpu_quantize(x)
    q_ref, d_ref, s_ref = Q8.quantize_q8_1(x)
    assert np.array_equal(xq, q_ref)
    assert np.array_equal(ds.view(np.uint16), _ds(d_ref, s_ref))
