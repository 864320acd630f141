"""The two-level super-block 4-bit matvec on the GPU, through the C ABI
(qgemv_q4k and its plan and fused-norm forms), against oracle.superblock.

The library quantizes the seeded weights to storage records (checked bit for
bit against the oracle's records) and repacks them to the device layout; the
GPU computes y from that layout, the oracle from the records.  Cases: ragged
row counts, every batch size, split-K rows (k = 15360), the LDS kernel (rows
too long for the K segments, and sub-block arrays not 4-byte aligned),
launch plans and batch rows bitwise, bf16 output, the fused norm, and the
full-size 15360 x 3840 / 3840 x 15360 matrices on every row.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import formats as F
from oracle import norm as N
from oracle import superblock as SB
from tests import parity
from tests.gpu_util import dev, host_y, log, out_tensor, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _matrix(seed, n, k):
    w = synth.weights(500 + seed % 113, n, k)
    rec = q.qg_quantize_q4k(w)
    assert np.array_equal(rec, SB.quantize_q4k(w)), "library and oracle records differ"
    return rec, [dev(a) for a in q.qg_repack_q4k(rec)]


def _run(dargs, x, n, plan=None, bf16=False, gamma=None, eps=0.0):
    x = np.atleast_2d(x)
    y = out_tensor(x.shape[0], n, bf16)
    q.qgemv_q4k(dargs[0], dargs[1], dargs[2], dev(x), y, plan=plan,
                gamma=None if gamma is None else dev(gamma), eps=eps)
    return host_y(y)


@pytest.mark.parametrize("n,k,batch", [
    (1, 256, 1), (7, 512, 2), (33, 3840, 1), (100, 4096, 3), (65, 3840, 4), (300, 15360, 1),
    (129, 14336, 4), (50, 33024, 2), (17, 65536, 4),
])
def test_q4k_parity(n, k, batch):
    log("q4k n=%d k=%d batch=%d" % (n, k, batch))
    rec, dargs = _matrix(n + k, n, k)
    x = synth.activations(600 + n % 37, batch, k)
    y = _run(dargs, x, n)
    y_ref, a_ref = SB.gemv_q4k(rec, x)
    r = parity.assert_parity(y, y_ref, a_ref, "q4k n=%d k=%d" % (n, k))
    log("   %r" % r)
    if batch == 2:
        for b in (0, 1):
            assert np.array_equal(_run(dargs, x[b:b + 1], n)[0], y[b]), b
    if batch == 4:
        # batch 3-4 share the matrix blocks' order (where x fits their LDS)
        assert np.array_equal(_run(dargs, x[:3], n), y[:3])
    yb = _run(dargs, x, n, bf16=True)
    assert np.array_equal(yb, F.f64_to_bf16_bits(y.astype(np.float64)))


def test_q4k_one_hot_columns_exact():
    """x = e_k returns column k of W^ exactly (one product, exact in fp32)."""
    n, k = 70, 768
    rec, dargs = _matrix(3, n, k)
    w = SB.dequant_q4k(rec)
    for col in (0, 31, 32, 255, 256, 767):
        x = np.zeros((1, k))
        x[0, col] = 1.0
        y = _run(dargs, F.f64_to_bf16_bits(x), n)
        assert np.array_equal(y[0].astype(np.float64), w[:, col]), col


PLANS = [None, {"rows_per_tile": 1}, {"rows_per_tile": 4, "waves_per_block": 1, "blocks": 3},
         {"rows_per_tile": 2, "waves_per_block": 5, "blocks": 7}, {"waves_per_block": 8, "blocks": 30000}]


@pytest.mark.parametrize("k,batch", [(3840, 2), (15360, 2), (3840, 4)])
def test_q4k_bitwise_across_plans(k, batch):
    n = 1001
    rec, dargs = _matrix(k, n, k)
    x = synth.activations(700, batch, k)
    ys = []
    for plan in PLANS:
        log("q4k plan k=%d %s" % (k, plan))
        ys.append(_run(dargs, x, n, plan=plan))
    for plan, y in zip(PLANS[1:], ys[1:]):
        assert np.array_equal(y, ys[0]), plan
    y_ref, a_ref = SB.gemv_q4k(rec, x)
    parity.assert_parity(ys[0], y_ref, a_ref)


def test_q4k_unaligned_sub_block_array():
    """A sub-block array that is only 2-byte aligned takes the LDS kernel
    (one parameter load per lane): another order of additions, same bound."""
    n, k = 90, 3840
    rec, dargs = _matrix(5, n, k)
    sub = dargs[1]
    buf = torch.zeros(sub.numel() + 1, dtype=torch.int16, device=sub.device)
    odd = buf[1:].view(sub.shape)
    odd.copy_(sub)
    assert odd.data_ptr() % 4 == 2
    x = synth.activations(701, 3, k)
    log("q4k 2-byte aligned sub-block array")
    y = out_tensor(3, n)
    q.qgemv_q4k(dargs[0], odd, dargs[2], dev(x), y)
    y_ref, a_ref = SB.gemv_q4k(rec, x)
    parity.assert_parity(host_y(y), y_ref, a_ref)


def test_q4k_fused_norm_equals_plain_on_normalized_x():
    n, k = 400, 3840
    rec, dargs = _matrix(6, n, k)
    x = synth.activations(702, 2, k)
    gamma = F.f64_to_bf16_bits(np.random.default_rng(7).uniform(0.5, 1.5, k))
    log("q4k fused norm n=%d k=%d" % (n, k))
    y = _run(dargs, x, n, gamma=gamma, eps=1e-5)
    xg = q.qg_rmsnorm_bf16(dev(x), dev(gamma), 1e-5)
    torch.cuda.synchronize()
    xg = xg.cpu().numpy().view(np.uint16)
    assert np.array_equal(y, _run(dargs, xg, n))
    y_ref, a_ref = SB.gemv_q4k(rec, N.rmsnorm_bf16(x, gamma, 1e-5))
    # the normalized x may differ in a few bf16 roundings (midpoint ambiguity):
    # the plain call above is already bitwise, so only the magnitude is checked
    assert np.allclose(y, y_ref, rtol=1e-2, atol=1e-2 * np.max(np.abs(y_ref)))


@pytest.mark.parametrize("name,batch", [("mlp_up", 1), ("mlp_down", 1), ("mlp_up", 4)])
def test_q4k_full_size_all_rows(name, batch):
    sid, n, k = synth.shape(name)
    log("q4k full-size %s [%d x %d]: generating" % (name, n, k))
    w = synth.weights(sid, n, k)
    rec = q.qg_quantize_q4k(w)
    rows = synth.sample_rows(n, 128, seed=sid)
    assert np.array_equal(rec[rows], SB.quantize_q4k(synth.weight_rows(sid, n, k, rows)))
    del w
    dargs = [dev(a) for a in q.qg_repack_q4k(rec)]
    x = synth.activations(sid, batch, k)
    log("q4k full-size %s batch %d: launching" % (name, batch))
    y1 = _run(dargs, x, n)
    assert np.array_equal(_run(dargs, x, n), y1), "second launch differs"
    del dargs
    torch.cuda.empty_cache()
    log("q4k full-size %s: oracle on all %d rows" % (name, n))
    y_ref, a_ref = SB.gemv_q4k(rec, x)
    r = parity.assert_parity(y1, y_ref, a_ref, "q4k %s batch %d all rows" % (name, batch))
    log("q4k full-size %s batch %d: %r" % (name, batch, r))
