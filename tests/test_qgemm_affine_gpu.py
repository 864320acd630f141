"""GPU parity of the affine 4-bit small-batch GEMM (qgemm_affine_u4: more
than four activation rows, codes decoded in registers and fed to bf16 MFMA,
each group folded as s * sum(q x) + b * sum(x)) against the oracle's float64
matvec of every activation row (oracle.gemv.gemv_affine, bits = 4).

Beyond parity (tests/parity.py's bar):
* each activation row's output is bitwise what that row alone gives (m = 1)
  and what any other m gives, across the activation-row blocks of 16, 32 and
  64 per workgroup, the one-wave K slices and the streaming kernel that takes
  up to 16 rows with x in LDS; repeated launches are bitwise identical;
* bf16 output is the RNE of the f32 output;
* nothing outside y[m, n] is written;
* the bias term alone (zero scales) and the scale term alone (zero biases)
  each meet the bar.
Shapes span ragged row tiles, ragged token tiles, a partial last K chunk, k
below one chunk, every group size and every K-slice count.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import formats as F
from oracle import gemv as G
from tests import parity
from tests.gpu_util import dev, host_y, log, out_tensor, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(n, k, gs, m, seed):
    w = synth.weights(800 + seed % 50, n, k)
    codes, scales, biases = q.qg_quantize_affine(w, 4, gs)
    x = synth.activations(800 + seed % 50, m, k)
    return codes, scales, biases, x


def _run(arrays, x, gs, bf16=False):
    m, n = x.shape[0], arrays[0].shape[0]
    y = out_tensor(m, n, bf16)
    q.qgemm_affine_u4(dev(arrays[0]), dev(arrays[1]), dev(arrays[2]), dev(x), y, gs)
    return host_y(y)


CASES = [
    (1, 64, 64, 5), (64, 256, 32, 16), (100, 3840, 64, 16), (1000, 4224, 64, 17), (130, 128, 32, 33),
    (77, 15360, 128, 64), (200, 3840, 64, 65), (33, 512, 64, 100), (300, 4096, 128, 8), (64, 2048, 32, 130),
    (9000, 512, 64, 20), (9000, 768, 128, 40), (33000, 256, 64, 40), (33000, 512, 32, 70),
    # up to 16 rows with x in LDS (the streaming kernel): group parameters
    # loaded one by one (66 groups, not a multiple of 4), long rows
    (1000, 4224, 64, 9), (50, 15360, 32, 6), (4100, 3840, 128, 16),
]


@pytest.mark.parametrize("n,k,gs,m", CASES)
def test_qgemm_affine_parity(n, k, gs, m):
    log("qgemm u4 n=%d k=%d gs=%d m=%d" % (n, k, gs, m))
    arrays = _inputs(n, k, gs, m, n + k + m)
    x = arrays[3]
    y = _run(arrays[:3], x, gs)
    y_ref, a_ref = G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 4, gs)
    r = parity.assert_parity(y, y_ref, a_ref, "qgemm u4 n=%d k=%d m=%d" % (n, k, m))
    log("   %r" % r)


@pytest.mark.parametrize("n,k,gs,m", [(150, 3840, 64, 37), (70, 4224, 128, 70), (9000, 1024, 64, 35),
                                      (33000, 512, 32, 70), (4200, 8192, 64, 16), (10300, 8448, 32, 8)])
def test_qgemm_affine_rows_alone_repeat_and_bf16(n, k, gs, m):
    arrays = _inputs(n, k, gs, m, 11)
    x = arrays[3]
    log("qgemm u4 rows alone n=%d k=%d m=%d" % (n, k, m))
    y = _run(arrays[:3], x, gs)
    for i in (0, 1, m // 2, m - 1):
        assert np.array_equal(_run(arrays[:3], x[i:i + 1], gs)[0], y[i]), i
    # another m (other activation-row blocks per workgroup) gives the same rows
    for m2 in (3, 17, 33, 65):
        if m2 < m:
            assert np.array_equal(_run(arrays[:3], x[:m2], gs), y[:m2]), m2
    for _ in range(2):
        assert np.array_equal(_run(arrays[:3], x, gs), y)
    yb = _run(arrays[:3], x, gs, bf16=True)
    assert np.array_equal(yb, F.f64_to_bf16_bits(y.astype(np.float64)))


@pytest.mark.parametrize("m", [21, 70])
def test_qgemm_affine_writes_only_y(m):
    n, k, gs = 130, 1024, 64
    arrays = _inputs(n, k, gs, m, 4)
    x = arrays[3]
    log("qgemm u4 guard bands m=%d" % m)
    guard = 4096
    buf = torch.full((m * n + 2 * guard,), -7.0, dtype=torch.float32, device="cuda:0")
    y = buf[guard:guard + m * n].view(m, n)
    q.qgemm_affine_u4(dev(arrays[0]), dev(arrays[1]), dev(arrays[2]), dev(x), y, gs)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == -7.0) and np.all(host[guard + m * n:] == -7.0)
    y_ref, a_ref = G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 4, gs)
    parity.assert_parity(host[guard:guard + m * n].reshape(m, n), y_ref, a_ref)


def test_qgemm_affine_terms_alone():
    """Zero scales leave the bias term b * sum(x) alone; zero biases leave the
    scale term alone: each meets the bar on its own."""
    n, k, gs, m = 200, 2048, 64, 24
    codes, scales, biases, x = _inputs(n, k, gs, m, 5)
    zero = np.zeros_like(scales)
    for s_, b_ in ((zero, biases), (scales, zero)):
        y = _run((codes, s_, b_), x, gs)
        y_ref, a_ref = G.gemv_affine(codes, s_, b_, x, 4, gs)
        parity.assert_parity(y, y_ref, a_ref)


def test_qgemm_affine_full_size_mlp_up():
    """15360 x 3840 (g64) at 64 activation rows: every output against the
    oracle, and a second launch bitwise."""
    sid, n, k = synth.shape("mlp_up")
    gs, m = 64, 64
    log("qgemm u4 full-size mlp_up m=%d: generating" % m)
    w = synth.weights(sid, n, k)
    arrays = q.qg_quantize_affine(w, 4, gs)
    del w
    x = synth.activations(sid + 7, m, k)
    y = _run(arrays, x, gs)
    assert np.array_equal(_run(arrays, x, gs), y)
    log("qgemm u4 full-size mlp_up: oracle")
    y_ref, a_ref = G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 4, gs)
    r = parity.assert_parity(y, y_ref, a_ref, "qgemm u4 mlp_up m=%d" % m)
    log("qgemm u4 full-size mlp_up m=%d: %r" % (m, r))
