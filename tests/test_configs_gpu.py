"""The full-size workloads on the GPU, in the launch configuration the bench
times (the plain entry points).

For each matrix the library quantizes the seeded fp32 weights and the GPU
computes every output.  The oracle independently re-quantizes a seeded sample
of rows from the same seeded weights (checking the library's codes bit for
bit), then computes every output in float64 from the packed arrays (row
blocks of 4096 over a thread pool): every element of every config must meet
the parity criterion, and the report (maximum error, unguarded maximum,
elements that used the cancellation floor) is logged per config.  A second
launch must reproduce the outputs bitwise.

Workloads (weights ~ N(0, 0.02), x ~ N(0, 1) in bf16, batch 1 unless noted):
  FP4-E2M1 g32: Gemma-4-12B gate_up 30720x3840, qkv 8192x3840,
                o_proj 3840x4096, fc_down 3840x15360
  affine g64 4/8-bit: 15360x3840, 3840x15360, 14336x4096, 4096x14336
  FP8-E4M3 row scale: lm_head 262144x3840, batch 1 and 4
  batch 4 of FP4 gate_up / fc_down and u4 15360x3840 / 3840x15360
  one GPU's share at tensor-parallel degree 8: FP4 3840x3840, 1024x3840,
                3840x512, 3840x1920; FP8 32768x3840
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import block_quantized_weight_qgemv_amd as q
import synth
from oracle import gemv as G
from oracle import quantize as Q
from tests import parity
from tests.gpu_util import dev, host_y, log, out_tensor, require_gpu

pytestmark = pytest.mark.gpu

SAMPLE = 192


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _launch(fmt, dargs, xd, y, gs):
    if fmt == "fp4":
        q.qgemv_fp4_e2m1(dargs[0], dargs[1], xd, y, gs)
    elif fmt == "u4":
        q.qgemv_affine_u4(dargs[0], dargs[1], dargs[2], xd, y, gs)
    elif fmt == "u8":
        q.qgemv_affine_u8(dargs[0], dargs[1], dargs[2], xd, y, gs)
    else:
        q.qgemv_fp8_e4m3(dargs[0], dargs[1], xd, y)


def _oracle(fmt, arrays, x, gs):
    if fmt == "fp4":
        return G.gemv_fp4_e2m1(arrays[0], arrays[1], x, gs)
    if fmt in ("u4", "u8"):
        return G.gemv_affine(arrays[0], arrays[1], arrays[2], x, 4 if fmt == "u4" else 8, gs)
    return G.gemv_fp8_e4m3(arrays[0], arrays[1], x)


def _oracle_all_rows(fmt, arrays, x, gs, block=4096):
    """The float64 oracle on every row of the packed arrays, 4096-row blocks
    spread over the host cores (one BLAS thread per worker)."""
    n = arrays[0].shape[0]
    bounds = [(r, min(n, r + block)) for r in range(0, n, block)]
    workers = max(1, min(16, len(os.sched_getaffinity(0))))

    def one(b):
        return _oracle(fmt, [a[b[0]:b[1]] for a in arrays], x, gs)

    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(one, bounds))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def _full_size(fmt, name, batch=1, gs=None):
    sid, n, k = synth.shape(name)
    log("full-size %s %s [%d x %d] batch=%d: generating" % (fmt, name, n, k, batch))
    w = synth.weights(sid, n, k)
    if fmt == "fp4":
        arrays = q.qg_quantize_fp4_e2m1(w, gs)
    elif fmt in ("u4", "u8"):
        arrays = q.qg_quantize_affine(w, 4 if fmt == "u4" else 8, gs)
    else:
        arrays = q.qg_quantize_fp8_e4m3_rowwise(w)
    del w
    x = synth.activations(sid, batch, k)
    dargs = [dev(a) for a in arrays]
    xd = dev(x)
    log("full-size %s %s: launching" % (fmt, name))
    y = out_tensor(batch, n)
    _launch(fmt, dargs, xd, y, gs)
    y1 = host_y(y)
    y2t = out_tensor(batch, n)
    _launch(fmt, dargs, xd, y2t, gs)
    y2 = host_y(y2t)
    del dargs
    torch.cuda.empty_cache()
    assert np.isfinite(y1).all()
    assert np.array_equal(y1, y2), "second launch differs"

    # the oracle side: re-quantize the sampled rows from the seeded weights
    rows = synth.sample_rows(n, SAMPLE, seed=sid)
    w_rows = synth.weight_rows(sid, n, k, rows)
    if fmt == "fp4":
        ora = Q.quantize_fp4_e2m1(w_rows, gs)
        y_ref, a_ref = G.gemv_fp4_e2m1(ora[0], ora[1], x, gs)
    elif fmt in ("u4", "u8"):
        bits = 4 if fmt == "u4" else 8
        ora = Q.quantize_affine(w_rows, bits, gs)
        y_ref, a_ref = G.gemv_affine(ora[0], ora[1], ora[2], x, bits, gs)
    else:
        ora = Q.quantize_fp8_e4m3_rowwise(w_rows)
        y_ref, a_ref = G.gemv_fp8_e4m3(ora[0], ora[1], x)
    for a_lib, a_ora in zip(arrays, ora):
        assert np.array_equal(a_lib[rows], a_ora), "library and oracle codes differ"
    parity.assert_parity(y1[:, rows], y_ref, a_ref, "%s %s sampled" % (fmt, name))
    # every output element against the oracle on the library's packed arrays
    log("full-size %s %s: oracle on all %d rows" % (fmt, name, n))
    y_all, a_all = _oracle_all_rows(fmt, arrays, x, gs)
    r = parity.assert_parity(y1, y_all, a_all, "%s %s all rows" % (fmt, name))
    log("full-size %s %s batch=%d: %r" % (fmt, name, batch, r))


@pytest.mark.parametrize("name", ["gate_up", "qkv", "o_proj", "fc_down"])
def test_fp4_gemma_shapes(name):
    _full_size("fp4", name, gs=32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("name", ["mlp_up", "mlp_down", "llama_up", "llama_down"])
def test_affine_shapes(bits, name):
    _full_size("u4" if bits == 4 else "u8", name, gs=64)


@pytest.mark.parametrize("fmt,name,gs", [("fp4", "gate_up", 32), ("fp4", "fc_down", 32),
                                         ("u4", "mlp_up", 64), ("u4", "mlp_down", 64)])
def test_batch4_matrix_blocks(fmt, name, gs):
    """Batch 4 of the 4-bit formats (the 4x4x4 matrix-block kernel), every
    row of the full-size matrix against the oracle."""
    _full_size(fmt, name, batch=4, gs=gs)


@pytest.mark.parametrize("fmt,name,gs", [("fp4", "gate_up_tp8", 32), ("fp4", "qkv_tp8", 32),
                                         ("fp4", "o_proj_tp8", 32), ("fp4", "fc_down_tp8", 32),
                                         ("fp8", "lm_head_tp8", None)])
def test_tensor_parallel_shards(fmt, name, gs):
    """One GPU's share of the Gemma shapes and the lm_head at tensor-parallel
    degree 8 (the shapes the sharded layers hand each GPU), every row against
    the oracle."""
    _full_size(fmt, name, gs=gs)


@pytest.mark.parametrize("batch", [1, 4])
def test_fp8_lm_head(batch):
    _full_size("fp8", "lm_head", batch=batch)


@pytest.mark.parametrize("name,m", [("gate_up", 16), ("fc_down", 64)])
def test_fp4_gemm_gemma_shapes(name, m):
    """The small-batch GEMM at a benchmarked shape: gate_up at 16 activation
    rows (x staged once per workgroup) and fc_down at 64 (x staged chunk by
    chunk, K slices).  Sampled rows against the oracle; a second launch and
    a single activation row reproduce the bits."""
    sid, n, k = synth.shape(name)
    gs = 32
    log("full-size GEMM fp4 %s [%d x %d] m=%d: generating" % (name, n, k, m))
    w = synth.weights(sid, n, k)
    codes, scales = q.qg_quantize_fp4_e2m1(w, gs)
    del w
    x = synth.activations(sid + 7, m, k)
    dc, ds, xd = dev(codes), dev(scales), dev(x)
    log("full-size GEMM fp4 %s m=%d: launching" % (name, m))
    y = out_tensor(m, n)
    q.qgemm_fp4_e2m1(dc, ds, xd, y, gs)
    y1 = host_y(y)
    q.qgemm_fp4_e2m1(dc, ds, xd, y, gs)
    assert np.array_equal(host_y(y), y1), "second launch differs"
    y_one = out_tensor(1, n)
    q.qgemm_fp4_e2m1(dc, ds, dev(x[m - 1:m]), y_one, gs)
    assert np.array_equal(host_y(y_one)[0], y1[m - 1]), "single row differs"
    del dc, ds
    torch.cuda.empty_cache()
    assert np.isfinite(y1).all()
    rows = synth.sample_rows(n, SAMPLE, seed=sid)
    ora = Q.quantize_fp4_e2m1(synth.weight_rows(sid, n, k, rows), gs)
    assert np.array_equal(codes[rows], ora[0]) and np.array_equal(scales[rows], ora[1])
    y_ref, a_ref = G.gemv_fp4_e2m1(ora[0], ora[1], x, gs)
    parity.assert_parity(y1[:, rows], y_ref, a_ref, "GEMM %s m=%d sampled" % (name, m))
    log("full-size GEMM fp4 %s m=%d: oracle on all %d rows" % (name, m, n))
    y_all, a_all = _oracle_all_rows("fp4", [codes, scales], x, gs)
    r = parity.assert_parity(y1, y_all, a_all, "GEMM %s m=%d all rows" % (name, m))
    log("full-size GEMM fp4 %s m=%d: %r" % (name, m, r))
