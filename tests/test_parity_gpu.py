"""GPU parity of the HIP path against the oracle, at sizes the oracle finishes
in seconds: several tiles, partial passes and ragged row tails, every batch
size, every group size, both output types, explicit launch shapes, and the
degenerate cases.  Every call goes through the C ABI (the binding only
marshals arguments).

Bars (the guarded 1e-3 relative criterion is in tests/parity.py):
  * general inputs: parity with the float64 oracle;
  * one-hot activations, the code tables and integer-valued cases: bitwise
    (each output is one exactly rounded product or an exact integer sum);
  * batch rows, launch shapes and repeated launches: bitwise identical;
  * bf16 output: bitwise the round-to-nearest-even of the f32 output.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import formats as F
from oracle import gemv as G
from oracle import quantize as Q
from tests import parity
from tests.gpu_util import dev, host_y, log, out_tensor, require_gpu, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _quantize(fmt, w, gs=None):
    """Codes from the library's pack module, checked bit-exact against the oracle's."""
    if fmt == "fp4":
        lib, ora = q.qg_quantize_fp4_e2m1(w, gs), Q.quantize_fp4_e2m1(w, gs)
    elif fmt in ("u4", "u8"):
        bits = 4 if fmt == "u4" else 8
        lib, ora = q.qg_quantize_affine(w, bits, gs), Q.quantize_affine(w, bits, gs)
    else:
        lib, ora = q.qg_quantize_fp8_e4m3_rowwise(w), Q.quantize_fp8_e4m3_rowwise(w)
    for a, b in zip(lib, ora):
        assert np.array_equal(a, b)
    return ora


def _oracle(fmt, arrays, x, gs=None):
    if fmt == "fp4":
        return G.gemv_fp4_e2m1(arrays[0], arrays[1], x, gs)
    if fmt == "u4":
        return G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 4, gs)
    if fmt == "u8":
        return G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 8, gs)
    return G.gemv_fp8_e4m3(arrays[0], arrays[1], x)


def _case(fmt, n, k, gs, batch, seed, plan=None):
    log("%s n=%d k=%d gs=%s batch=%d seed=%d plan=%s" % (fmt, n, k, gs, batch, seed, plan))
    w = synth.weights(100 + seed, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(100 + seed, batch, k)
    y = run(fmt, arrays, x, n, gs=gs, plan=plan)
    y_ref, a_ref = _oracle(fmt, arrays, x, gs)
    parity.assert_parity(y, y_ref, a_ref, "%s n=%d k=%d" % (fmt, n, k))
    return arrays, x, y


# ---------------------------------------------------------------- configs

def test_tiny_fp4_config():
    """Tiny FP4-E2M1 GEMV: W [256, 512], group 32, bf16 absmax scales, seed 0."""
    w, x = synth.tiny_fp4_inputs()
    arrays = _quantize("fp4", w, 32)
    log("tiny fp4 256x512")
    y = run("fp4", arrays, x, 256, gs=32)
    y_ref, a_ref = G.gemv_fp4_e2m1(arrays[0], arrays[1], x, 32)
    r = parity.assert_parity(y, y_ref, a_ref, "tiny")
    log("tiny fp4 parity %r" % r)


@pytest.mark.parametrize("n,k,gs,batch", [
    (1, 32, 32, 1), (7, 64, 32, 2), (33, 3840, 32, 1), (100, 512, 128, 3),
    (65, 4224, 64, 4), (300, 15360, 32, 1), (129, 2048, 32, 4), (5, 8192, 128, 2),
])
def test_fp4_shapes(n, k, gs, batch):
    _case("fp4", n, k, gs, batch, seed=n + k)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n,k,gs,batch", [
    (1, 64, 64, 1), (9, 128, 32, 2), (40, 3840, 64, 1), (77, 4096, 64, 3),
    (31, 15360, 64, 1), (64, 14336, 128, 4), (3, 1088, 64, 2),
])
def test_affine_shapes(bits, n, k, gs, batch):
    fmt = "u4" if bits == 4 else "u8"
    _case(fmt, n, k, gs, batch, seed=bits * 1000 + n + k)


WPC = {"fp4": 32, "u4": 32, "u8": 16, "fp8": 16}      # weights per 16-byte chunk


@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("fmt,gs,k", [("fp4", 32, 65536), ("u4", 64, 65536), ("u8", 64, 32768),
                                      ("fp8", None, 65536), ("u8", 32, 16416), ("fp4", 128, 40960)])
def test_long_rows_each_format(fmt, gs, k, batch):
    """Rows too long for the row kernel's K segments whose activations do not
    fit in LDS either (the LDS kernel then reads them with each step) meet the
    parity bar on a ragged row count; a batch row gives the bits it gives alone."""
    n = 70
    arrays, x, y = _case(fmt, n, k, gs, batch, seed=7 * batch + k % 97)
    if batch > 1:
        for b in (0, batch - 1):
            assert np.array_equal(run(fmt, arrays, x[b:b + 1], n, gs=gs)[0], y[b])


@pytest.mark.parametrize("batch", [3, 4])
def test_u8_long_rows_batch_3_4(batch):
    """u8 at k = 15360 holds 4 * 960 * 64 bytes of fp32 activation pieces per
    batch row: beyond LDS at batch 3-4 for the LDS kernel, so the row kernel's
    K segments take it, with x in registers; bitwise equal to batch 1 rows."""
    n, k, gs = 300, 15360, 64
    arrays, x, y = _case("u8", n, k, gs, batch, seed=31 + batch)
    for b in range(batch):
        assert np.array_equal(run("u8", arrays, x[b:b + 1], n, gs=gs)[0], y[b]), b


@pytest.mark.parametrize("n,k,batch", [
    (1, 16, 1), (8, 48, 2), (50, 3840, 4), (257, 1040, 1), (19, 4096, 3), (2, 15360, 1),
    # matrix-core path (batch 3, 4): a single row, a ragged last pass, rows of
    # several steps with a ragged tail, a row count off the 4-row tiles
    (1, 16, 3), (7, 272, 4), (1003, 4112, 3), (4097, 1024, 4), (30, 9984, 4),
])
def test_fp8_shapes(n, k, batch):
    _case("fp8", n, k, None, batch, seed=n * 7 + k)


# ---------------------------------------------------------------- code tables

def _one_hot(k, col, batch=1):
    x = np.zeros((batch, k), np.uint16)
    x[:, col] = 0x3F80
    return x


def test_fp4_all_codes_bitwise():
    """Row c holds code c in every position; x one-hot on an even and an odd column."""
    n, k = 16, 64
    codes = np.array([[c | (c << 4)] * (k // 2) for c in range(16)], np.uint8)
    scales = np.full((n, k // 32), 0x3F80, np.uint16)            # scale 1
    for col in (0, 1, 62, 63):
        log("fp4 code table col=%d" % col)
        y = run("fp4", (codes, scales), _one_hot(k, col), n, gs=32)
        assert np.array_equal(y[0].astype(np.float64), F.E2M1_TABLE), (col, y)


def test_fp8_all_codes_bitwise():
    n, k = 256, 32
    codes = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k, axis=1)
    rs = np.ones(n, np.float32)
    for col in (0, 5, 31):
        log("fp8 code table col=%d" % col)
        y = run("fp8", (codes, rs), _one_hot(k, col), n)
        want = F.E4M3_TABLE
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(y[0]), nan)
        assert np.array_equal(y[0][~nan].astype(np.float64), want[~nan])


@pytest.mark.parametrize("bits", [4, 8])
def test_affine_all_codes_bitwise(bits):
    n, k, per = 1 << bits, 128, 32 // bits
    levels = np.arange(n, dtype=np.uint32)
    word = np.zeros(n, np.uint32)
    for j in range(per):
        word |= levels << (bits * j)
    codes = np.repeat(word[:, None], k // per, axis=1)
    scales = np.full((n, 2), 0x3F80, np.uint16)                  # s = 1
    biases = np.zeros((n, 2), np.uint16)                         # b = 0
    for col in (0, 1, 2, 3, 5, 7, 127):
        log("u%d code table col=%d" % (bits, col))
        y = run("u4" if bits == 4 else "u8", (codes, scales, biases), _one_hot(k, col), n, gs=64)
        assert np.array_equal(y[0], levels.astype(np.float32)), (col, y[0][:20])


# ---------------------------------------------------------------- exact cases

@pytest.mark.parametrize("fmt,gs", [("fp4", 32), ("fp4", 128), ("u4", 64), ("u8", 64), ("fp8", None)])
def test_one_hot_reads_one_column_bitwise(fmt, gs):
    n, k = 70, 4096
    w = synth.weights(7, n, k)
    arrays = _quantize(fmt, w, gs)
    if fmt == "fp4":
        w_hat = G.dequant_fp4_e2m1(arrays[0], arrays[1], k, gs)
    elif fmt in ("u4", "u8"):
        w_hat = G.dequant_affine(arrays[0], arrays[1], arrays[2], k, 4 if fmt == "u4" else 8, gs)
    else:
        w_hat = G.dequant_fp8_e4m3(arrays[0], arrays[1])
    for col in (0, 1, 31, 32, 2047, 4095):
        log("one-hot %s col=%d" % (fmt, col))
        y = run(fmt, arrays, _one_hot(k, col), n, gs=gs)
        # one product (plus the bias for affine), rounded once to f32
        assert np.array_equal(y[0], w_hat[:, col].astype(np.float32)), (fmt, col)


@pytest.mark.parametrize("bits", [4, 8])
def test_affine_integer_case_bitwise(bits):
    """s = 1, b = 0 and small-integer x: y is an exact integer matvec."""
    n, k, gs = 96, 3840, 64
    per = 32 // bits
    rng = np.random.default_rng(bits)
    codes = synth.uniform_words((n, k // per), bits)
    scales = np.full((n, k // gs), 0x3F80, np.uint16)
    biases = np.zeros((n, k // gs), np.uint16)
    xi = rng.integers(-4, 5, (2, k))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    log("affine integer case bits=%d" % bits)
    y = run("u4" if bits == 4 else "u8", (codes, scales, biases), x, n, gs=gs)
    from oracle.layout import unpack_u32
    qmat = unpack_u32(codes, k, bits).astype(np.int64)
    want = xi @ qmat.T
    assert np.abs(want).max() < 2 ** 24
    assert np.array_equal(y, want.astype(np.float32))


# ---------------------------------------------------------------- uniform random codes

@pytest.mark.parametrize("fmt", ["fp4", "u4", "u8", "fp8"])
def test_uniform_random_codes(fmt):
    """Every code value (not just those a Gaussian quantizes to) against the oracle."""
    n, k, gs, batch = 200, 2560, 64, 2
    if fmt == "fp4":
        arrays = (synth.uniform_bytes((n, k // 2), 1), synth.uniform_bf16((n, k // gs), 1e-3, 0.1, 1))
    elif fmt in ("u4", "u8"):
        per = 8 if fmt == "u4" else 4
        arrays = (synth.uniform_words((n, k // per), 2), synth.uniform_bf16((n, k // gs), 1e-4, 1e-2, 2),
                  synth.uniform_bf16((n, k // gs), -0.2, 0.2, 3))
    else:
        c = synth.uniform_bytes((n, k), 4)
        c[(c & 0x7F) == 0x7F] = 0x7E                               # no NaN codes here
        arrays = (c, synth.uniform_f32(n, 1e-4, 1e-2, 4))
    x = synth.uniform_bf16((batch, k), -2.0, 2.0, 5)
    log("uniform codes %s" % fmt)
    y = run(fmt, arrays, x, n, gs=gs)
    y_ref, a_ref = _oracle(fmt, arrays, x, gs)
    parity.assert_parity(y, y_ref, a_ref, fmt)


def test_fp8_nan_code_gives_nan_row():
    n, k = 6, 64
    codes = np.full((n, k), 0x38, np.uint8)                        # 1.0
    codes[2, 17] = 0x7F
    codes[4, 0] = 0xFF
    x = synth.uniform_bf16((1, k), 0.5, 1.0, 6)
    log("fp8 nan row")
    y = run("fp8", (codes, np.ones(n, np.float32)), x, n)
    assert np.isnan(y[0, 2]) and np.isnan(y[0, 4])
    assert np.isfinite(y[0, [0, 1, 3, 5]]).all()


def test_zero_scale_rows_give_zero():
    n, k = 9, 256
    w = synth.weights(8, n, k)
    w[3] = 0.0
    arrays = _quantize("fp4", w, 32)
    log("zero row fp4")
    y = run("fp4", arrays, synth.activations(8, 1, k), n, gs=32)
    assert y[0, 3] == 0.0


# ---------------------------------------------------------------- bitwise consistency

# formats whose batch 3-4 runs on the matrix blocks (for rows whose x fits
# their LDS): another order of additions than batch 1-2
MATRIX_FROM_3 = {"fp4", "u4", "fp8"}


@pytest.mark.parametrize("fmt,gs,k", [("fp4", 32, 3840), ("u4", 64, 4096), ("u8", 64, 3840), ("fp8", None, 3840),
                                      ("fp4", 64, 15360), ("u4", 128, 14336)])
def test_batch_rows_match_single_calls_bitwise(fmt, gs, k):
    n = 515
    w = synth.weights(9, n, k)
    arrays = _quantize(fmt, w, gs)
    x4 = synth.activations(9, 4, k)
    log("batch consistency %s k=%d" % (fmt, k))
    y4 = run(fmt, arrays, x4, n, gs=gs)
    ys = {bsz: run(fmt, arrays, x4[:bsz], n, gs=gs) for bsz in (1, 2, 3)}
    ys[4] = y4
    singles = [run(fmt, arrays, x4[b:b + 1], n, gs=gs)[0] for b in range(4)]
    if fmt not in MATRIX_FROM_3:
        for b in range(4):
            assert np.array_equal(singles[b], y4[b]), (fmt, b)
        for bsz in (2, 3):
            assert np.array_equal(ys[bsz], y4[:bsz])
    else:
        # the vector unit below 3 activation rows, the matrix cores from 3
        # on: bitwise inside each group, and both groups within the parity
        # bound of the exact result
        for b in range(2):
            assert np.array_equal(singles[b], ys[2][b]), b
        assert np.array_equal(ys[3], y4[:3])
        y_ref, a_ref = _oracle(fmt, arrays, x4, gs)
        parity.assert_parity(y4, y_ref, a_ref)
        parity.assert_parity(np.stack(singles), y_ref, a_ref)


PLANS = [None, {"rows_per_tile": 1}, {"rows_per_tile": 2}, {"rows_per_tile": 4},
         {"rows_per_tile": 4, "waves_per_block": 1, "blocks": 3},
         {"rows_per_tile": 2, "waves_per_block": 8, "blocks": 5},
         {"rows_per_tile": 1, "waves_per_block": 2, "blocks": 1000},
         {"waves_per_block": 3, "blocks": 7}]


@pytest.mark.parametrize("fmt,gs,k,batch", [("fp4", 32, 3840, 2), ("u4", 64, 15360, 2), ("u8", 128, 1024, 2),
                                            ("fp8", None, 2048, 2), ("fp8", None, 3840, 4), ("fp8", None, 5120, 3),
                                            ("fp4", 32, 3840, 4), ("u4", 64, 4096, 3), ("fp4", 128, 15360, 3)])
def test_launch_shapes_bitwise_identical(fmt, gs, k, batch):
    n = 1001
    w = synth.weights(10, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(10, batch, k)
    ys = []
    for plan in PLANS:
        log("plan %s %s" % (fmt, plan))
        ys.append(run(fmt, arrays, x, n, gs=gs, plan=plan))
    y_ref, a_ref = _oracle(fmt, arrays, x, gs)
    parity.assert_parity(ys[0], y_ref, a_ref)
    for y in ys[1:]:
        assert np.array_equal(y, ys[0])


def test_repeated_launches_bitwise_identical():
    n, k = 4000, 3840
    w = synth.weights(11, n, k)
    codes, scales = _quantize("fp4", w, 32)
    cd, sd = dev(codes), dev(scales)
    xd = dev(synth.activations(11, 1, k))
    outs = []
    for _ in range(3):
        y = out_tensor(1, n)
        q.qgemv_fp4_e2m1(cd, sd, xd, y, 32)
        outs.append(host_y(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("fmt,gs", [("fp4", 32), ("u4", 64), ("u8", 64), ("fp8", None)])
def test_bf16_output_is_rne_of_f32_output(fmt, gs):
    n, k = 333, 1024
    w = synth.weights(12, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(12, 3, k)
    log("bf16 out %s" % fmt)
    y32 = run(fmt, arrays, x, n, gs=gs)
    y16 = run(fmt, arrays, x, n, gs=gs, bf16=True)
    assert np.array_equal(y16, F.f64_to_bf16_bits(y32.astype(np.float64)))


# ---------------------------------------------------------------- poisoning

GUARD = 4096


def _guarded(a, fill_byte):
    """Device buffer with GUARD bytes of `fill_byte` before and after `a`."""
    raw = np.ascontiguousarray(a).view(np.uint8).ravel()
    buf = np.full(raw.size + 2 * GUARD, fill_byte, np.uint8)
    buf[GUARD:GUARD + raw.size] = raw
    d = torch.from_numpy(buf).to("cuda:0")
    return d, d[GUARD:GUARD + raw.size]


@pytest.mark.parametrize("fmt,gs,batch", [("fp4", 64, 2), ("u4", 64, 2), ("u8", 32, 2), ("fp8", None, 2),
                                          ("fp8", None, 4)])
def test_poisoned_neighbours_are_never_read_or_written(fmt, gs, batch):
    """NaN in every byte around the inputs; y pre-filled with NaN and fenced by
    canaries.  FP8 at batch 4 runs on the matrix-core kernel."""
    n, k = 123, 3904 if fmt != "fp8" else 3856
    w = synth.weights(13, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(13, batch, k)
    # bf16 NaN is 0x7FC0 -> bytes C0 7F; 0xFF bytes are NaN for bf16 and f32
    # and the E4M3 NaN code; for packed 4-bit codes 0xFF is a valid code (-6),
    # which a stray read would still turn into a parity failure
    dev_arrays = []
    for a in arrays:
        full, view = _guarded(a, 0xFF)
        dt = {np.uint8: torch.uint8, np.uint16: torch.int16, np.uint32: torch.int32,
              np.float32: torch.float32}[a.dtype.type]
        dev_arrays.append((full, view.view(dt).view(a.shape)))
    xfull, xv = _guarded(x, 0xFF)
    xv = xv.view(torch.int16).view(batch, k)
    yfull = torch.full(((batch * n * 4) + 2 * GUARD,), 0xAB, dtype=torch.uint8, device="cuda:0")
    yv = yfull[GUARD:GUARD + batch * n * 4].view(torch.float32).view(batch, n)
    yv.fill_(float("nan"))
    log("poison %s batch=%d" % (fmt, batch))
    views = [v for _, v in dev_arrays]
    if fmt == "fp4":
        q.qgemv_fp4_e2m1(views[0], views[1], xv, yv, gs)
    elif fmt == "u4":
        q.qgemv_affine_u4(views[0], views[1], views[2], xv, yv, gs)
    elif fmt == "u8":
        q.qgemv_affine_u8(views[0], views[1], views[2], xv, yv, gs)
    else:
        q.qgemv_fp8_e4m3(views[0], views[1], xv, yv)
    y = host_y(yv)
    assert np.isfinite(y).all(), "unwritten or poisoned outputs"
    yb = yfull.cpu().numpy()
    assert (yb[:GUARD] == 0xAB).all() and (yb[-GUARD:] == 0xAB).all(), "write outside y"
    y_ref, a_ref = _oracle(fmt, arrays, x, gs)
    parity.assert_parity(y, y_ref, a_ref)


# ---------------------------------------------------------------- kernel paths

@pytest.mark.parametrize("fmt,n,k,gs,batch", [
    # rows cut into 2, 4 or 8 K segments (split-K inside a workgroup)
    ("fp4", 129, 15360, 32, 1), ("fp4", 67, 15360, 32, 2), ("fp4", 40, 8192, 64, 4),
    ("u4", 100, 14336, 64, 1), ("u4", 33, 15360, 64, 3), ("u8", 77, 15360, 64, 1),
    ("u8", 50, 3840, 64, 2), ("u8", 9, 14336, 64, 1), ("fp8", 70, 15360, None, 4),
    ("fp8", 300, 8192, None, 1),
])
def test_split_k_shapes(fmt, n, k, gs, batch):
    _case(fmt, n, k, gs, batch, seed=n * 31 + k + batch)


@pytest.mark.parametrize("fmt,n,k,gs,batch", [
    # shapes the register kernel does not take: odd group counts per row or
    # segment, a chunk count no power-of-two segment count divides
    ("fp4", 90, 3872, 32, 1), ("u4", 45, 3904, 64, 2), ("u8", 61, 3904, 32, 1),
    ("fp8", 80, 4112, None, 3),
])
def test_lds_kernel_shapes(fmt, n, k, gs, batch):
    _case(fmt, n, k, gs, batch, seed=n * 17 + k)


def test_two_byte_aligned_scales_take_the_lds_kernel():
    """Scales that are only 2-byte aligned are legal; results must not change."""
    n, k, gs = 150, 3840, 32
    w = synth.weights(14, n, k)
    codes, scales = _quantize("fp4", w, gs)
    x = synth.activations(14, 2, k)
    y_ref, a_ref = G.gemv_fp4_e2m1(codes, scales, x, gs)
    y_aligned = run("fp4", (codes, scales), x, n, gs=gs)
    buf = torch.zeros(scales.size + 1, dtype=torch.int16, device="cuda:0")
    buf[1:] = torch.from_numpy(scales.view(np.int16).ravel()).to("cuda:0")
    s_odd = buf[1:].view(n, k // gs)
    assert s_odd.data_ptr() % 4 == 2
    y = out_tensor(2, n)
    log("fp4 2-byte aligned scales")
    q.qgemv_fp4_e2m1(dev(codes), s_odd, dev(x), y, gs)
    y2 = host_y(y)
    parity.assert_parity(y2, y_ref, a_ref)
    parity.assert_parity(y_aligned, y_ref, a_ref)


@pytest.mark.parametrize("fmt,gs,k", [("fp4", 32, 15360), ("u8", 64, 15360), ("u4", 64, 14336)])
def test_split_k_batch_and_bf16(fmt, gs, k):
    n = 200
    w = synth.weights(15, n, k)
    arrays = _quantize(fmt, w, gs)
    x4 = synth.activations(15, 4, k)
    bmax = 4
    log("split-K batch/bf16 %s k=%d batch<=%d" % (fmt, k, bmax))
    yb = run(fmt, arrays, x4[:bmax], n, gs=gs)
    # batch rows alone give their bits inside the vector group (1-2) and,
    # for the formats that take the matrix blocks from 3 on, inside 3-4
    y2 = run(fmt, arrays, x4[:2], n, gs=gs)
    for b in range(2):
        assert np.array_equal(run(fmt, arrays, x4[b:b + 1], n, gs=gs)[0], y2[b])
    if fmt in MATRIX_FROM_3:
        assert np.array_equal(run(fmt, arrays, x4[:3], n, gs=gs), yb[:3])
    else:
        assert np.array_equal(y2, yb[:2])
    y16 = run(fmt, arrays, x4[:bmax], n, gs=gs, bf16=True)
    assert np.array_equal(y16, F.f64_to_bf16_bits(yb.astype(np.float64)))
    y_ref, a_ref = _oracle(fmt, arrays, x4[:bmax], gs)
    parity.assert_parity(yb, y_ref, a_ref)


# ---------------------------------------------------------------- tile sharing

# Launch shapes that exercise how a workgroup hands out its tiles: chunks of
# many tiles with a ragged last chunk, wave counts that are not powers of two,
# one workgroup for every row, and more workgroups than rows (most get none).
SHARING_PLANS = [
    None,
    {"rows_per_tile": 1, "waves_per_block": 8, "blocks": 4},
    {"rows_per_tile": 2, "waves_per_block": 5, "blocks": 3},
    {"rows_per_tile": 4, "waves_per_block": 6, "blocks": 11},
    {"rows_per_tile": 2, "waves_per_block": 4, "blocks": 1},
    {"rows_per_tile": 1, "waves_per_block": 8, "blocks": 30000},
]


@pytest.mark.parametrize("fmt,n,k,gs,batch", [
    ("fp4", 20011, 512, 32, 1),       # x staged, one K segment
    ("fp8", 20011, 1024, None, 2),
    ("u4", 3001, 8192, 64, 1),        # two K segments, several waves per segment
    ("u8", 3001, 4096, 64, 2),
    ("fp4", 5003, 3840, 32, 3),       # x not staged (registers): one chunk per wave
])
def test_shared_tiles_bitwise_across_plans(fmt, n, k, gs, batch):
    """Each row segment is streamed by exactly one wave, whichever wave takes
    it: the result meets the oracle and is bitwise the same for every launch
    shape (the sums do not depend on which wave computed them)."""
    w = synth.weights(16, n, k)
    arrays = _quantize(fmt, w, gs)
    x = synth.activations(16, batch, k)
    ys = []
    for plan in SHARING_PLANS:
        log("shared tiles %s n=%d k=%d batch=%d plan %s" % (fmt, n, k, batch, plan))
        ys.append(run(fmt, arrays, x, n, gs=gs, plan=plan))
    y_ref, a_ref = _oracle(fmt, arrays, x, gs)
    parity.assert_parity(ys[0], y_ref, a_ref, "%s n=%d k=%d" % (fmt, n, k))
    for plan, y in zip(SHARING_PLANS[1:], ys[1:]):
        assert np.array_equal(y, ys[0]), plan


def test_fp8_plan_query_by_batch():
    """The plan the library reports for FP8: one-row tiles on the vector
    kernel at batch 1 and 2, 4-row tiles on the matrix-core kernel at 3 and
    4, one workgroup per compute unit for the lm_head, fewer for few rows."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for batch in (1, 2, 3, 4):
        p = q.qg_plan_query(q.QG_FMT_FP8_E4M3, 262144, 3840, batch)
        assert p["rows_per_tile"] == (1 if batch < 3 else 4), (batch, p)
        assert p["waves_per_block"] == 8 and p["blocks"] == cus, (batch, p)
    p = q.qg_plan_query(q.QG_FMT_FP8_E4M3, 40, 3840, 4)      # 10 tiles of 4 rows: 2 workgroups of 8 waves
    assert p["rows_per_tile"] == 4 and p["blocks"] == 2, p


def test_stale_hip_error_is_not_this_calls():
    """An error an earlier, unrelated HIP call left in the thread (here an
    invalid hipSetDevice) is neither reported as the next matvec's launch
    failure nor cleared: the library takes each launch's own status, and the
    error stays for its owner to read."""
    import ctypes
    with open("/proc/self/maps") as f:
        path = next(line.split()[-1] for line in f if "libamdhip64" in line)
    hip = ctypes.CDLL(path)
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    n, k, gs = 64, 512, 32
    w, x = synth.weights(41, n, k), synth.activations(41, 1, k)
    arrays = _quantize("fp4", w, gs)
    y_ref, a_ref = _oracle("fp4", arrays, x, gs)
    codes, scales, xd = dev(arrays[0]), dev(arrays[1]), dev(x)
    y = out_tensor(1, n)
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0
    log("stale HIP error before a launch")
    stale = hip.hipSetDevice(4096)                     # leaves an error behind
    assert stale != 0
    p = lambda t: ctypes.c_void_p(t.data_ptr())        # noqa: E731
    st = q.lib().qgemv_fp4_e2m1(p(codes), p(scales), p(xd), p(y), n, k, gs, 1, 0, None)
    left = hip.hipGetLastError()                       # read (and clear) it before torch runs again
    assert st == 0, q.qg_status_string(st)
    assert left == stale
    parity.assert_parity(host_y(y), y_ref, a_ref, "after a stale error")
