"""A decode step captured in a HIP graph: every replay equals the eager launches
bitwise.

The step is the FP4 layer sequence (qkv, o_proj, gate_up, fc_down shapes,
scaled down) over three distinct layers, each matvec writing its own output.
The graph is replayed three times; between replays the outputs are cleared by
a fill kernel outside the graph and the program does eager work of its own,
so each replay has to write every output again.  The library records no
memset or allocation into the graph (Part 2 post, "Where it landed": a graph
decode step is one of the two ranked levers; the pages verify graph replay
bit-identical to direct launch).
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_qgemv_amd as q
import synth
from tests.gpu_util import dev, log, require_gpu

pytestmark = pytest.mark.gpu

SHAPES = [("qkv", 1024, 3840), ("o_proj", 480, 4096), ("gate_up", 3840, 3840), ("fc_down", 480, 15360)]
LAYERS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_graph_replay_matches_eager_bitwise():
    mats = []
    for li in range(LAYERS):
        for si, (name, n, k) in enumerate(SHAPES):
            w = synth.weights(200 + si, n, k, layer=li)
            codes, scales = q.qg_quantize_fp4_e2m1(w, 32)
            x = synth.activations(200 + si, 1, k)
            y = torch.empty((1, n), dtype=torch.float32, device="cuda:0")
            mats.append((name, dev(codes), dev(scales), dev(x), y))

    def step():
        for name, c, s, x, y in mats:
            q.qgemv_fp4_e2m1(c, s, x, y, 32)

    log("graph: eager step")
    step()
    torch.cuda.synchronize()
    eager = [m[4].cpu().numpy().copy() for m in mats]
    assert all(np.isfinite(e).all() for e in eager)

    log("graph: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                               # warm the launch path on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    scratch = torch.randn(1 << 20, device="cuda:0")
    for rep in range(3):
        for m in mats:
            m[4].zero_()                     # a fill kernel, outside the graph
        scratch.mul_(1.0001).add_(0.5)        # eager work between replays
        torch.cuda.synchronize()
        log("graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for (name, *_, y), e in zip(mats, eager):
            assert np.array_equal(y.cpu().numpy(), e), (rep, name)


def test_graph_replay_with_norms_matches_eager_bitwise():
    """The pre-norm decode step (an RMSNorm before qkv and before gate_up) in
    one graph, twice: with the norm fused into those matvecs, and with
    separate norm launches writing the normalized x that plain matvecs read.
    Every replay equals the eager launches bitwise, and the fused outputs
    equal the separate ones."""
    rng = np.random.default_rng(11)
    normed = {"qkv", "gate_up"}
    mats = []
    for li in range(LAYERS):
        for si, (name, n, k) in enumerate(SHAPES):
            w = synth.weights(210 + si, n, k, layer=li)
            codes, scales = q.qg_quantize_fp4_e2m1(w, 32)
            x = dev(synth.activations(210 + si + 7 * li, 1, k))
            g16 = torch.from_numpy(rng.uniform(0.5, 1.5, k).astype(np.float32)).to("cuda:0").to(torch.bfloat16)
            y_f = torch.empty((1, n), dtype=torch.float32, device="cuda:0")
            y_s = torch.empty((1, n), dtype=torch.float32, device="cuda:0")
            mats.append((name, dev(codes), dev(scales), x, g16, torch.empty_like(x), y_f, y_s))

    def step():
        for name, c, s, x, g, xn, y_f, y_s in mats:
            if name in normed:
                q.qgemv_fp4_e2m1_rmsnorm(c, s, x, g, 1e-6, y_f, 32)
                q.qg_rmsnorm_bf16(x, g, 1e-6, xn)
                q.qgemv_fp4_e2m1(c, s, xn, y_s, 32)
            else:
                q.qgemv_fp4_e2m1(c, s, x, y_f, 32)
                q.qgemv_fp4_e2m1(c, s, x, y_s, 32)

    log("graph+norm: eager step")
    step()
    torch.cuda.synchronize()
    eager = [(m[6].cpu().numpy().copy(), m[7].cpu().numpy().copy()) for m in mats]
    for (name, *_), (f, s) in zip(mats, eager):
        assert np.isfinite(f).all() and np.array_equal(f, s), name

    log("graph+norm: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    scratch = torch.randn(1 << 20, device="cuda:0")
    for rep in range(3):
        for m in mats:
            m[5].zero_()
            m[6].zero_()
            m[7].zero_()
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        log("graph+norm: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for (name, *_, y_f, y_s), (f, s) in zip(mats, eager):
            assert np.array_equal(y_f.cpu().numpy(), f), (rep, name, "fused")
            assert np.array_equal(y_s.cpu().numpy(), s), (rep, name, "separate")


def test_graph_replay_int8_route_matches_eager_bitwise():
    """The int8 activation route in one graph: a quantize launch whose blocks
    feed two matvecs (as one x feeds gate and up), and the fused launch,
    over affine u4 shapes at batch 1 and 4.  Every replay equals the eager
    launches bitwise (the quantized blocks and pairs included)."""
    cases = []
    for ci, (n, k, b) in enumerate([(1024, 3840, 1), (480, 15360, 4), (768, 4096, 4)]):
        w1 = synth.weights(230 + ci, n, k)
        w2 = synth.weights(240 + ci, n, k)
        a1 = [dev(a) for a in q.qg_quantize_affine(w1, 4, 64)]
        a2 = [dev(a) for a in q.qg_quantize_affine(w2, 4, 64)]
        x = dev(synth.activations(230 + ci, b, k))
        xq = torch.empty((b, k), dtype=torch.int8, device="cuda:0")
        ds = torch.empty((b, k // 32, 2), dtype=torch.int16, device="cuda:0")
        ys = [torch.empty((b, n), dtype=torch.float32, device="cuda:0") for _ in range(3)]
        cases.append((a1, a2, x, xq, ds, ys))

    def step():
        for a1, a2, x, xq, ds, ys in cases:
            q.qg_quantize_q8_1(x, xq, ds)
            q.qgemv_affine_u4_q8(a1[0], a1[1], a1[2], xq, ds, ys[0], 64)
            q.qgemv_affine_u4_q8(a2[0], a2[1], a2[2], xq, ds, ys[1], 64)
            q.qgemv_affine_u4_q8_fused(a1[0], a1[1], a1[2], x, ys[2], 64)

    def outputs():
        return [[t.cpu().numpy().copy() for t in (xq, ds, *ys)] for _, _, _, xq, ds, ys in cases]

    log("graph int8: eager step")
    step()
    torch.cuda.synchronize()
    eager = outputs()
    for e in eager:
        assert np.isfinite(e[3]).all() and np.array_equal(e[2], e[4])   # fused equals two launches

    log("graph int8: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    scratch = torch.randn(1 << 20, device="cuda:0")
    for rep in range(3):
        for _, _, _, xq, ds, ys in cases:
            xq.zero_()
            ds.zero_()
            for t in ys:
                t.zero_()
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        log("graph int8: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for ci, (got, want) in enumerate(zip(outputs(), eager)):
            for j, (a, b) in enumerate(zip(got, want)):
                assert np.array_equal(a, b), (rep, ci, j)


def test_graph_replay_matrix_blocks_q4k_and_gemm_match_eager_bitwise():
    """The other kernels in one captured step: FP4 and u4 at batch 3 and 4
    (the 4x4x4 matrix-block kernel, split-K partials in LDS), the two-level
    format at batch 1 and 4, and the affine GEMM at 24 rows.  Three replays,
    each after the outputs were cleared outside the graph, equal the eager
    step bitwise."""
    calls = []
    for bi, batch in enumerate((3, 4)):
        w = synth.weights(230 + bi, 512, 3840)
        codes, scales = q.qg_quantize_fp4_e2m1(w, 32)
        x = dev(synth.activations(230 + bi, batch, 3840))
        y = torch.empty((batch, 512), dtype=torch.float32, device="cuda:0")
        c, s = dev(codes), dev(scales)
        calls.append((lambda c=c, s=s, x=x, y=y: q.qgemv_fp4_e2m1(c, s, x, y, 32), y))
        wa = synth.weights(240 + bi, 300, 15360)
        a = [dev(t) for t in q.qg_quantize_affine(wa, 4, 64)]
        xa = dev(synth.activations(240 + bi, batch, 15360))
        ya = torch.empty((batch, 300), dtype=torch.float32, device="cuda:0")
        calls.append((lambda a=a, x=xa, y=ya: q.qgemv_affine_u4(a[0], a[1], a[2], x, y, 64), ya))
    for batch in (1, 4):
        wq = synth.weights(250 + batch, 700, 3840)
        dq = [dev(t) for t in q.qg_repack_q4k(q.qg_quantize_q4k(wq))]
        xq = dev(synth.activations(250 + batch, batch, 3840))
        yq = torch.empty((batch, 700), dtype=torch.float32, device="cuda:0")
        calls.append((lambda d=dq, x=xq, y=yq: q.qgemv_q4k(d[0], d[1], d[2], x, y), yq))
    wg = synth.weights(260, 1000, 4096)
    ag = [dev(t) for t in q.qg_quantize_affine(wg, 4, 64)]
    xg = dev(synth.activations(260, 24, 4096))
    yg = torch.empty((24, 1000), dtype=torch.float32, device="cuda:0")
    calls.append((lambda a=ag, x=xg, y=yg: q.qgemm_affine_u4(a[0], a[1], a[2], x, y, 64), yg))

    def step():
        for fn, _ in calls:
            fn()

    log("graph (matrix blocks, two-level, GEMM): eager step")
    step()
    torch.cuda.synchronize()
    eager = [y.cpu().numpy().copy() for _, y in calls]
    assert all(np.isfinite(e).all() for e in eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.randn(1 << 20, device="cuda:0")
    for rep in range(3):
        for _, y in calls:
            y.zero_()
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        log("graph (matrix blocks, two-level, GEMM): replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for i, ((_, y), e) in enumerate(zip(calls, eager)):
            assert np.array_equal(y.cpu().numpy(), e), (rep, i)
