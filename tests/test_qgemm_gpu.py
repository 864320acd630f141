"""GPU parity of the small-batch GEMM (qgemm_fp4_e2m1: more than four
activation rows, weights decoded in registers and fed to bf16 MFMA) against
the oracle's float64 matvec of every activation row.

The GEMM sums each scale group's products in fp32 inside the MFMA and scales
the group sum once; the bar is the matvec's (tests/parity.py): 1e-3 relative,
guarded against cancellation.  Beyond parity:
* each activation row's output is bitwise what that row alone gives (m = 1),
  and repeated launches are bitwise identical;
* bf16 output is the RNE of the f32 output;
* nothing outside y[m, n] is written.
Shapes span ragged row tiles (n % 64), ragged token tiles (m % 16, m % 64),
a partial last K chunk (k % 256), k below one chunk, every group size, and
more activation rows than one workgroup takes (m > 64).
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
    w = synth.weights(500 + seed % 50, n, k)
    codes, scales = q.qg_quantize_fp4_e2m1(w, gs)
    x = synth.activations(500 + seed % 50, m, k)
    return codes, scales, x


def _run(codes, scales, x, gs, bf16=False):
    m, n = x.shape[0], codes.shape[0]
    y = out_tensor(m, n, bf16)
    q.qgemm_fp4_e2m1(dev(codes), dev(scales), dev(x), y, gs)
    return host_y(y)


# The workgroup splits K into 4, 2 or 1 slices by n (at most 4096, 10240, or
# more rows) and by the number of 256-wide chunks; every split is covered.
CASES = [
    (1, 32, 32, 5), (64, 256, 32, 16), (100, 3840, 32, 16), (1000, 4224, 64, 17), (130, 96, 32, 33),
    (77, 15360, 128, 64), (200, 3840, 32, 65), (33, 512, 64, 100), (300, 4096, 128, 8), (64, 2048, 32, 130),
    (100, 512, 32, 16), (9000, 512, 32, 20), (9000, 768, 128, 40), (33000, 256, 64, 40), (33000, 512, 32, 70),
]


@pytest.mark.parametrize("n,k,gs,m", CASES)
def test_qgemm_parity(n, k, gs, m):
    seed = n + k + m
    log("qgemm fp4 n=%d k=%d gs=%d m=%d" % (n, k, gs, m))
    codes, scales, x = _inputs(n, k, gs, m, seed)
    y = _run(codes, scales, x, gs)
    y_ref, a_ref = G.gemv_fp4_e2m1(codes, scales, x, gs)
    parity.assert_parity(y, y_ref, a_ref, "qgemm n=%d k=%d m=%d" % (n, k, m))


# the last two take one wave per K slice (16-row workgroups: few row tiles,
# x too large for the streaming kernel at m rows) with 2 and 1 K slices; their
# single rows run on the streaming kernel
@pytest.mark.parametrize("n,k,gs,m", [(150, 3840, 32, 37), (70, 4224, 128, 70), (9000, 1024, 64, 35),
                                      (33000, 512, 32, 70), (4200, 8192, 32, 16), (10300, 8448, 32, 8)])
def test_qgemm_rows_alone_repeat_and_bf16(n, k, gs, m):
    codes, scales, x = _inputs(n, k, gs, m, 9)
    log("qgemm rows alone n=%d k=%d m=%d" % (n, k, m))
    y = _run(codes, scales, x, gs)
    for i in (0, 1, m // 2, m - 1):
        assert np.array_equal(_run(codes, scales, x[i:i + 1], gs)[0], y[i]), i
    for _ in range(3):
        assert np.array_equal(_run(codes, scales, x, gs), y)
    y16 = _run(codes, scales, x, gs, bf16=True)
    assert np.array_equal(y16, F.f64_to_bf16_bits(y.astype(np.float64)))


@pytest.mark.parametrize("m", [21, 13])           # the general kernel, the streaming one
def test_qgemm_writes_only_y(m):
    n, k, gs = 90, 1024, 32
    codes, scales, x = _inputs(n, k, gs, m, 4)
    log("qgemm canaries n=%d k=%d m=%d" % (n, k, m))
    pad = 4096
    buf = torch.full((pad + m * n + pad,), 7.25, dtype=torch.float32, device="cuda:0")
    y = buf[pad:pad + m * n].view(m, n)
    q.qgemm_fp4_e2m1(dev(codes), dev(scales), dev(x), y, gs)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 7.25) and np.all(host[pad + m * n:] == 7.25)
    y_ref, a_ref = G.gemv_fp4_e2m1(codes, scales, x, gs)
    parity.assert_parity(host[pad:pad + m * n].reshape(m, n), y_ref, a_ref)


def test_qgemm_zero_scales_give_zero_rows():
    n, k, gs, m = 48, 512, 32, 9
    codes, scales, x = _inputs(n, k, gs, m, 5)
    scales = scales.copy()
    scales[::3] = 0
    y = _run(codes, scales, x, gs)
    assert np.all(y[:, ::3] == 0)


@pytest.mark.parametrize("n,k,gs", [(2000, 3840, 32), (130, 4096, 64), (20000, 1024, 128)])
def test_qgemm_small_m_kernel_matches_general_kernel_bitwise(n, k, gs):
    """Up to 16 activation rows whose x fits in LDS take the streaming kernel;
    17 rows take the general one.  Both add a row's terms in the same order."""
    codes, scales, x = _inputs(n, k, gs, 17, 11)
    log("qgemm small-m vs general n=%d k=%d gs=%d" % (n, k, gs))
    y17 = _run(codes, scales, x, gs)
    y16 = _run(codes, scales, x[:16], gs)
    assert np.array_equal(y16, y17[:16])
    y_ref, a_ref = G.gemv_fp4_e2m1(codes, scales, x, gs)
    parity.assert_parity(y17, y_ref, a_ref, "qgemm n=%d k=%d m=17" % (n, k))
