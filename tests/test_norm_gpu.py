"""GPU parity of the fused RMSNorm variants (y = W . RMSNorm(x) in one launch)
and of the standalone norm, against the oracle (oracle.norm, then
oracle.gemv).

The GPU evaluates x * r * gamma in fp32 (r from an fp32 sum of squares) and
rounds to bf16; the oracle evaluates it in float64.  Where the exact value
lies within the fp32 error of a bf16 rounding midpoint the two may pick the
two different neighbours.  The fp32 error is bounded by the arithmetic: the
sum of squares has at most 8 + 6 + k/512 roundings of positive terms, then a
division, an addition, a square root and a reciprocal, then two products, so
|error| <= (22 + k/1024 + 7) * 2^-24 relative.  AMBIG = 64 * 2^-24 (plus the
k term) covers it twice over.  So:

* the standalone norm equals the oracle's bf16 values bit for bit, except at
  elements within AMBIG of a midpoint, where it may hold the other neighbour;
* the fused result equals, bit for bit, the plain entry point fed the
  standalone norm's output (the same arithmetic in the same order);
* the fused result meets the parity bar against the oracle widened by what
  the ambiguous elements can move it: sum_k |W^[n,k]| * |other_k - x~_k|
  over the ambiguous k;
* every format, split-K, the LDS kernel; bitwise the same for every launch
  shape and for each batch row alone (r is summed in an order fixed by k);
* argument errors.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import formats as F
from oracle import gemv as G
from oracle import norm as N
from oracle import quantize as Q
from tests import parity
from tests.gpu_util import dev, host_y, log, out_tensor, require_gpu, run


def host_bits(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _quantize(fmt, w, gs):
    if fmt == "fp4":
        return Q.quantize_fp4_e2m1(w, gs)
    if fmt in ("u4", "u8"):
        return Q.quantize_affine(w, 4 if fmt == "u4" else 8, gs)
    return Q.quantize_fp8_e4m3_rowwise(w)


def _oracle(fmt, arrays, x, gs):
    if fmt == "fp4":
        return G.gemv_fp4_e2m1(arrays[0], arrays[1], x, gs)
    if fmt in ("u4", "u8"):
        return G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 4 if fmt == "u4" else 8, gs)
    return G.gemv_fp8_e4m3(arrays[0], arrays[1], x)


def _gamma(k, seed):
    rng = np.random.default_rng(seed)
    return F.f64_to_bf16_bits(rng.uniform(0.5, 1.5, k))


def _dequant(fmt, arrays, k, gs):
    if fmt == "fp4":
        return G.dequant_fp4_e2m1(arrays[0], arrays[1], k, gs)
    if fmt in ("u4", "u8"):
        return G.dequant_affine(arrays[0], arrays[1], arrays[2], k, 4 if fmt == "u4" else 8, gs)
    return G.dequant_fp8_e4m3(arrays[0], arrays[1])


def _ambiguous(x, gamma, eps):
    """(mask, other_bits): elements whose exact normalized value lies within
    the fp32 error bound of a bf16 rounding midpoint, and the neighbour on
    the other side of that midpoint."""
    k = x.shape[-1]
    v = N.rmsnorm_f64(x, gamma, eps)
    rne = F.f64_to_bf16_bits(v)
    rv = F.bf16_bits_to_f64(rne)
    toward = np.where(np.abs(v) > np.abs(rv), 1, -1)           # step away from or toward zero
    other = (rne.astype(np.int32) + toward).astype(np.uint16)
    ov = F.bf16_bits_to_f64(other)
    mid = (rv + ov) / 2
    bound = (64 + k / 1024) * 2.0 ** -24
    mask = (np.abs(v - mid) <= bound * np.abs(v)) & (rv != 0) & (np.sign(ov) == np.sign(rv))
    return mask, other


def run_norm(fmt, arrays, x, gamma, eps, n, gs=None, plan=None, bf16=False):
    x = np.atleast_2d(x)
    y = out_tensor(x.shape[0], n, bf16)
    xd, gd = dev(x), dev(gamma)
    if fmt == "fp4":
        q.qgemv_fp4_e2m1_rmsnorm(dev(arrays[0]), dev(arrays[1]), xd, gd, eps, y, gs, plan=plan)
    elif fmt == "u4":
        q.qgemv_affine_u4_rmsnorm(dev(arrays[0]), dev(arrays[1]), dev(arrays[2]), xd, gd, eps, y, gs, plan=plan)
    elif fmt == "u8":
        q.qgemv_affine_u8_rmsnorm(dev(arrays[0]), dev(arrays[1]), dev(arrays[2]), xd, gd, eps, y, gs, plan=plan)
    else:
        q.qgemv_fp8_e4m3_rmsnorm(dev(arrays[0]), dev(arrays[1]), xd, gd, eps, y, plan=plan)
    return host_y(y)


CASES = [
    ("fp4", 1000, 3840, 32, 1), ("fp4", 700, 3840, 32, 4), ("fp4", 300, 15360, 32, 2),
    ("u4", 900, 4096, 64, 1), ("u4", 250, 15360, 64, 3), ("u8", 800, 3840, 64, 2),
    ("u8", 120, 14336, 64, 1), ("fp8", 1500, 3840, None, 1), ("fp8", 600, 3840, None, 4),
    ("fp4", 90, 3872, 32, 2),          # the LDS kernel
    ("fp8", 333, 5120, None, 3),       # the matrix-core kernel, rows of several steps
    ("fp4", 200, 15360, 32, 4),        # matrix blocks, gamma in LDS beside 120 KiB of x
    ("u4", 260, 15360, 64, 4),         # matrix blocks, gamma read from memory (no room in LDS)
]


@pytest.mark.parametrize("fmt,n,k,gs,batch", CASES)
def test_fused_norm_parity(fmt, n, k, gs, batch):
    seed = n + k + batch
    log("norm %s n=%d k=%d gs=%s batch=%d" % (fmt, n, k, gs, batch))
    w = synth.weights(300 + seed % 97, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(300 + seed % 97, batch, k)
    gamma = _gamma(k, seed)
    eps = 1e-6
    y = run_norm(fmt, arrays, x, gamma, eps, n, gs)

    # the standalone norm: the oracle's bits except at ambiguous elements
    xg = host_bits(q.qg_rmsnorm_bf16(dev(x), dev(gamma), eps))
    xn = N.rmsnorm_bf16(x, gamma, eps)
    amb, other = _ambiguous(x, gamma, eps)
    diff = xg != xn
    assert np.all(amb[diff]) and np.array_equal(xg[diff], other[diff]), \
        "%d non-ambiguous mismatches" % int(np.sum(diff & ~amb))
    log("   %d of %d normalized values ambiguous, %d rounded the other way" % (amb.sum(), amb.size, diff.sum()))

    # the fused result is the plain matvec of the GPU's normalized x
    y_plain = run(fmt, arrays, xg, n, gs=gs)
    assert np.array_equal(y, y_plain)

    # against the oracle, widened by what the ambiguous elements can move
    y_ref, a_ref = _oracle(fmt, arrays, xn, gs)
    dx = np.where(amb, np.abs(F.bf16_bits_to_f64(other) - F.bf16_bits_to_f64(xn)), 0.0)
    extra = dx @ np.abs(_dequant(fmt, arrays, k, gs)).T               # [B, N]
    err = np.abs(y.astype(np.float64) - y_ref)
    bar = 1e-3 * np.maximum(np.abs(y_ref), 2.0 ** -12 * a_ref) + extra
    assert np.all(err <= bar), "max excess %g" % float(np.max(err - bar))
    if not amb.any():
        parity.assert_parity(y, y_ref, a_ref, "%s fused norm n=%d k=%d" % (fmt, n, k))


def _exact_tie_inputs(k, seed):
    """x, gamma, eps for which every fp32 step of the norm is exact: x has four
    significant bits (its squares and their sums stay far inside fp32's 24),
    eps tops the mean square up to exactly 4, so r = 1/2; gamma has seven
    significant bits, so x * r * gamma is exact in fp32 and many values sit
    exactly on a bf16 rounding midpoint."""
    rng = np.random.default_rng(seed)
    xv = rng.choice([-1.0, 1.0], k) * (8 + rng.integers(0, 8, k)) / 8.0 * 2.0 ** rng.integers(-1, 1, k)
    gv = (64 + rng.integers(0, 64, k)) / 64.0 * 2.0 ** rng.integers(-1, 1, k)
    x = F.f64_to_bf16_bits(xv)[None, :]
    gamma = F.f64_to_bf16_bits(gv)
    assert np.array_equal(F.bf16_bits_to_f64(x[0]), xv) and np.array_equal(F.bf16_bits_to_f64(gamma), gv)
    mean_sq = float(np.sum(xv * xv)) / k
    eps = 4.0 - mean_sq
    assert eps >= 0.0 and np.float32(eps) == eps
    return x, gamma, float(eps)


@pytest.mark.parametrize("k", [3840, 15360])
def test_norm_rounds_exact_midpoints_to_even(k):
    """With every fp32 step exact (r = 1/2 exactly, exact products), the GPU's
    rounding to bf16 is the only rounding: the standalone and the fused norm
    must give the oracle's round-to-nearest-even bits everywhere, including
    the values that sit exactly on a midpoint (rounded both up and down)."""
    x, gamma, eps = _exact_tie_inputs(k, 11 + k)
    log("norm exact midpoints k=%d" % k)
    v = N.rmsnorm_f64(x, gamma, eps)
    ref = N.rmsnorm_bf16(x, gamma, eps)
    rv = F.bf16_bits_to_f64(ref)
    # midpoints: the exact value is half way between its bf16 neighbours
    up = (ref.astype(np.int32) + 1).astype(np.uint16)
    dn = (ref.astype(np.int32) - 1).astype(np.uint16)
    on_mid = (np.abs(v - (rv + F.bf16_bits_to_f64(up)) / 2) == 0) | (np.abs(v - (rv + F.bf16_bits_to_f64(dn)) / 2) == 0)
    rounded_up = on_mid & (np.abs(rv) > np.abs(v))
    rounded_dn = on_mid & (np.abs(rv) < np.abs(v))
    assert rounded_up.sum() > 50 and rounded_dn.sum() > 50, (rounded_up.sum(), rounded_dn.sum())
    got = host_bits(q.qg_rmsnorm_bf16(dev(x), dev(gamma), eps))
    assert np.array_equal(got, ref), "%d of %d values differ" % (int(np.sum(got != ref)), k)
    # the fused call on these inputs equals the plain call on them
    n, gs = 96, 32
    arrays = Q.quantize_fp4_e2m1(synth.weights(41, n, k), gs)
    y = run_norm("fp4", arrays, x, gamma, eps, n, gs)
    assert np.array_equal(y, run("fp4", arrays, got, n, gs=gs))


@pytest.mark.parametrize("k", [8, 3840, 8200, 16384, 20480])
def test_standalone_norm_kept_and_reread_rows(k):
    """Rows whose x and gamma fit in LDS beside the sums (k up to 16352) are
    read once; longer rows are read again to normalize.  Both: the oracle's
    bits except at ambiguous elements, each batch row as it is alone, and the
    same in place (out = x).  k = 8 is one unit; 8200 ends in a ragged group."""
    log("standalone norm k=%d" % k)
    x = synth.activations(400 + k % 89, 3, k)
    gamma = _gamma(k, k)
    eps = 1e-6
    xg = host_bits(q.qg_rmsnorm_bf16(dev(x), dev(gamma), eps))
    xn = N.rmsnorm_bf16(x, gamma, eps)
    amb, other = _ambiguous(x, gamma, eps)
    diff = xg != xn
    assert np.all(amb[diff]) and np.array_equal(xg[diff], other[diff]), \
        "%d non-ambiguous mismatches" % int(np.sum(diff & ~amb))
    for b in range(3):
        assert np.array_equal(host_bits(q.qg_rmsnorm_bf16(dev(x[b:b + 1]), dev(gamma), eps))[0], xg[b]), b
    xd = dev(x)
    q.qg_rmsnorm_bf16(xd, dev(gamma), eps, xd)
    assert np.array_equal(host_bits(xd), xg)


def test_fused_norm_equals_plain_on_a_reread_row():
    """k = 20480: the standalone norm reads x twice, the fused one keeps it in
    LDS; the two still agree bit for bit."""
    n, k, gs = 700, 20480, 32
    arrays = _quantize("fp4", synth.weights(36, n, k), gs)
    x = synth.activations(36, 1, k)
    gamma = _gamma(k, 9)
    y = run_norm("fp4", arrays, x, gamma, 1e-6, n, gs)
    xg = host_bits(q.qg_rmsnorm_bf16(dev(x), dev(gamma), 1e-6))
    assert np.array_equal(y, run("fp4", arrays, xg, n, gs=gs))


PLANS = [None, {"rows_per_tile": 1}, {"rows_per_tile": 4, "waves_per_block": 1, "blocks": 3},
         {"rows_per_tile": 2, "waves_per_block": 5, "blocks": 7}, {"waves_per_block": 2, "blocks": 1000}]


@pytest.mark.parametrize("fmt,k,gs", [("fp4", 3840, 32), ("u8", 4096, 64), ("fp8", 3840, None)])
def test_fused_norm_bitwise_across_plans_and_batch(fmt, k, gs):
    n = 1001
    w = synth.weights(31, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(31, 4, k)
    gamma = _gamma(k, 5)
    ys = []
    for plan in PLANS:
        log("norm plan %s %s" % (fmt, plan))
        ys.append(run_norm(fmt, arrays, x, gamma, 1e-5, n, gs, plan=plan))
    for plan, y in zip(PLANS[1:], ys[1:]):
        assert np.array_equal(y, ys[0]), plan
    if fmt not in ("fp8", "fp4"):
        for b in range(4):
            y1 = run_norm(fmt, arrays, x[b:b + 1], gamma, 1e-5, n, gs)
            assert np.array_equal(y1[0], ys[0][b]), b
    else:
        # FP8 and FP4 sum on the vector unit below 3 activation rows and on
        # the matrix cores from 3 on: bitwise inside each group of batch sizes
        y2 = run_norm(fmt, arrays, x[:2], gamma, 1e-5, n, gs)
        for b in range(2):
            y1 = run_norm(fmt, arrays, x[b:b + 1], gamma, 1e-5, n, gs)
            assert np.array_equal(y1[0], y2[b]), b
        y3 = run_norm(fmt, arrays, x[:3], gamma, 1e-5, n, gs)
        assert np.array_equal(y3, ys[0][:3])
    y16 = run_norm(fmt, arrays, x, gamma, 1e-5, n, gs, bf16=True)
    assert np.array_equal(y16, F.f64_to_bf16_bits(ys[0].astype(np.float64)))


def test_fused_norm_does_not_touch_x_and_handles_a_zero_row():
    n, k, gs = 500, 4096, 32
    w = synth.weights(33, n, k)
    arrays = _quantize("fp4", w, gs)
    x = synth.activations(33, 2, k)
    x[1] = 0                                   # a zero row: r = 1/sqrt(eps), output 0
    gamma = _gamma(k, 6)
    xd = dev(x)
    before = xd.clone()
    y = out_tensor(2, n)
    q.qgemv_fp4_e2m1_rmsnorm(dev(arrays[0]), dev(arrays[1]), xd, dev(gamma), 1e-5, y, gs)
    yh = host_y(y)
    assert torch.equal(xd, before)
    assert np.all(yh[1] == 0)
    y_ref, a_ref = _oracle("fp4", arrays, N.rmsnorm_bf16(x, gamma, 1e-5), gs)
    parity.assert_parity(yh, y_ref, a_ref)


def test_fused_norm_beyond_lds():
    """u8 at batch 4 and k = 15360: x and gamma ((4 + 1) * k * 2 bytes) exceed
    128 KiB of LDS, so the LDS kernel takes the call (another order of
    additions): it meets the widened parity bar; batch 3 still fits and stays
    bitwise the plain call on the separately normalized x."""
    n, k, gs = 64, 15360, 64
    fmt = "u8"
    arrays = _quantize(fmt, synth.weights(35, n, k), gs)
    x = synth.activations(35, 4, k)
    gamma = _gamma(k, 8)
    eps = 1e-5
    log("norm beyond LDS u8 n=%d k=%d batch=4" % (n, k))
    y4 = run_norm(fmt, arrays, x, gamma, eps, n, gs)
    xn = N.rmsnorm_bf16(x, gamma, eps)
    amb, other = _ambiguous(x, gamma, eps)
    y_ref, a_ref = _oracle(fmt, arrays, xn, gs)
    dx = np.where(amb, np.abs(F.bf16_bits_to_f64(other) - F.bf16_bits_to_f64(xn)), 0.0)
    extra = dx @ np.abs(_dequant(fmt, arrays, k, gs)).T
    bar = 1e-3 * np.maximum(np.abs(y_ref), 2.0 ** -12 * a_ref) + extra
    assert np.all(np.abs(y4.astype(np.float64) - y_ref) <= bar)
    y3 = run_norm(fmt, arrays, x[:3], gamma, eps, n, gs)
    xg = host_bits(q.qg_rmsnorm_bf16(dev(x[:3]), dev(gamma), eps))
    assert np.array_equal(y3, run(fmt, arrays, xg, n, gs=gs))


def test_fused_norm_argument_errors():
    n, k, gs = 64, 512, 32
    arrays = _quantize("fp4", synth.weights(34, n, k), gs)
    c, s = dev(arrays[0]), dev(arrays[1])
    x = dev(synth.activations(34, 1, k))
    g = dev(_gamma(k, 7))
    y = out_tensor(1, n)
    for eps, code in ((-1.0, 8), (float("nan"), 8), (float("inf"), 8)):
        with pytest.raises(q.QgError) as e:
            q.qgemv_fp4_e2m1_rmsnorm(c, s, x, g, eps, y, gs)
        assert e.value.status == code
    buf = torch.zeros(k + 1, dtype=torch.int16, device="cuda:0")
    with pytest.raises(q.QgError) as e:
        q.qgemv_fp4_e2m1_rmsnorm(c, s, x, buf[1:], 1e-5, y, gs)      # 2-byte aligned gamma
    assert e.value.status == 4
    with pytest.raises(ValueError):
        q.qgemv_fp4_e2m1_rmsnorm(c, s, x, g[:-8], 1e-5, y, gs)       # wrong length
