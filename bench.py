#!/usr/bin/env python3
"""Benchmark of the MI355X block-quantized weight matvec.

Default workload (one JSON line on stdout): the Gemma-4-12B-shaped FP4-E2M1
gate_up matvec, W [30720, 3840] with group-32 bf16 scales, x bf16, batch 1,
fp32 output.  One step is one full matvec over one weight matrix; the weights
rotate over >= 1 GiB of distinct device copies so that every step streams its
weights from HBM rather than from the 256 MB Infinity Cache, as the distinct
layers of a decode token do.  Inputs are resident in HBM before timing starts.

  value          algorithmic bytes of the K timed steps / elapsed time (GB/s)
  ms_per_step    elapsed time / K (HIP events on the launch stream)
  roofline       the same kernel duration against the 8 TB/s HBM peak;
                 traffic from rocprofv3 FETCH_SIZE / WRITE_SIZE when known
  cpu_baseline   the float64 oracle on the host cores, on the same workload

Algorithmic bytes of one FP4 g32 matvec: N*K/2 codes + N*K/32*2 scales +
B*K*2 activations + B*N*4 outputs (66,485,760 B for gate_up).

Other modes: --sweep times every workload shape (plain entry points) and the
48-layer FP4 decode step, writing a table to stderr and JSON to --out;
--calibrate-copy times a plain device copy (the reference kernel for the
rocprofv3 byte counters); --plan R,W,B overrides the launch shape.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
METRIC = "quantized GEMV HBM GB/s & % of 8 TB/s peak; µs per Gemma-12B-shaped matvec"
ROT_BYTES = 1 << 30
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_quantized_weight_qgemv_amd", "csrc")
KERNEL_SOURCES = ["qgemv_common.hpp", "qgemv_formats.hpp", "qgemv_kernels.hpp", "qgemv_launch.hpp", "qgemv_api.hip",
                  "qgemv_fp4.hip"]
# rocprofv3 FETCH_SIZE / WRITE_SIZE of the default workload, each scaled by
# what the counter reads for a plain copy of known size; written by
# --summarize-pmc and only used while the kernel sources are unchanged
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp4_gate_up_30720x3840_traffic.json")
COPY_BYTES = 512 << 20


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic():
    """Scaled HBM bytes per launch from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ workloads

def algorithmic_bytes(fmt, n, k, batch, gs):
    import block_quantized_weight_qgemv_amd as q
    if fmt == "fp4":
        w = q.qg_bytes_fp4(n, k, gs)
    elif fmt == "q4k":
        w = q.qg_bytes_q4k(n, k)
    elif fmt in ("u4", "u8", "u4q8", "u4q8mv", "u4q8f", "u8q8", "u8q8f"):
        w = q.qg_bytes_affine(n, k, 8 if fmt.startswith("u8") else 4, gs)
    else:
        w = q.qg_bytes_fp8(n, k)
    return w + batch * k * 2 + batch * n * 4


def quantize(fmt, w, gs):
    import block_quantized_weight_qgemv_amd as q
    if fmt == "fp4":
        return q.qg_quantize_fp4_e2m1(w, gs)
    if fmt == "q4k":
        return q.qg_repack_q4k(q.qg_quantize_q4k(w))
    if fmt in ("u4", "u8", "u4q8", "u4q8mv", "u4q8f", "u8q8", "u8q8f"):
        return q.qg_quantize_affine(w, 8 if fmt.startswith("u8") else 4, gs)
    return q.qg_quantize_fp8_e4m3_rowwise(w)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda:0")


class Workload:
    """Device-resident copies of one quantized matrix and a launch closure."""

    def __init__(self, fmt, shape_name, batch=1, gs=None, copies=None, plan=None, keep_host=False):
        import torch
        import synth
        import block_quantized_weight_qgemv_amd as q
        self.q = q
        self.fmt, self.name, self.batch, self.gs, self.plan = fmt, shape_name, batch, gs, plan
        sid, n, k = synth.shape(shape_name)
        self.n, self.k = n, k
        w = synth.weights(sid, n, k)
        self.host = quantize(fmt, w, gs)
        del w
        self.x_host = synth.activations(sid, batch, k)
        self.bytes = algorithmic_bytes(fmt, n, k, batch, gs)
        wbytes = sum(a.nbytes for a in self.host)
        self.copies = copies or min(4096, max(1, math.ceil(ROT_BYTES / wbytes)))
        first = [to_dev(a) for a in self.host]
        self.dev = [first] + [[t.clone() for t in first] for _ in range(self.copies - 1)]
        if not keep_host:
            self.host = None
        self.x = to_dev(self.x_host)
        self.y = torch.empty((batch, n), dtype=torch.float32, device="cuda:0")
        if fmt in ("u4q8", "u4q8mv", "u8q8"):
            # int8 activation blocks: requantized every step ("u4q8", the whole
            # route) or once here ("u4q8mv", the matvec kernel alone)
            self.xq, self.ds = q.qg_quantize_q8_1(self.x)

    def launch(self, i):
        d = self.dev[i % self.copies]
        q = self.q
        if self.fmt == "fp4":
            q.qgemv_fp4_e2m1(d[0], d[1], self.x, self.y, self.gs, plan=self.plan)
        elif self.fmt == "u4":
            q.qgemv_affine_u4(d[0], d[1], d[2], self.x, self.y, self.gs, plan=self.plan)
        elif self.fmt == "q4k":
            q.qgemv_q4k(d[0], d[1], d[2], self.x, self.y, plan=self.plan)
        elif self.fmt == "u8":
            q.qgemv_affine_u8(d[0], d[1], d[2], self.x, self.y, self.gs, plan=self.plan)
        elif self.fmt == "u4q8f":
            q.qgemv_affine_u4_q8_fused(d[0], d[1], d[2], self.x, self.y, self.gs)
        elif self.fmt == "u8q8f":
            q.qgemv_affine_u8_q8_fused(d[0], d[1], d[2], self.x, self.y, self.gs)
        elif self.fmt == "u8q8":
            q.qg_quantize_q8_1(self.x, self.xq, self.ds)
            q.qgemv_affine_u8_q8(d[0], d[1], d[2], self.xq, self.ds, self.y, self.gs)
        elif self.fmt in ("u4q8", "u4q8mv"):
            if self.fmt == "u4q8":
                q.qg_quantize_q8_1(self.x, self.xq, self.ds)
            q.qgemv_affine_u4_q8(d[0], d[1], d[2], self.xq, self.ds, self.y, self.gs)
        else:
            q.qgemv_fp8_e4m3(d[0], d[1], self.x, self.y, plan=self.plan)

    def label(self):
        return "%s %s [%dx%d] B=%d" % (self.fmt, self.name, self.n, self.k, self.batch)


def time_steps(launch, steps, warmup, mode="graph"):
    """Run `warmup` untimed steps, then time exactly `steps` steps; returns ms."""
    import torch
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    if mode == "graph":
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                launch(warmup + i)
        g.replay()                       # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        start.record()
        g.replay()
        stop.record()
    else:
        start.record()
        for i in range(steps):
            launch(warmup + i)
        stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop)


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(wl, target_s=12.0):
    """The float64 oracle on the host cores over the same packed matrix.

    Row blocks of 2048 rows are spread over one worker thread per core of
    the process's CPU share (the cores it may run on, at most 16: the host
    share of one GPU on a shared node; BLAS pinned to one thread per worker);
    whole matvecs are repeated until about `target_s` seconds have passed.
    The host's core counts and the numpy/BLAS builds are recorded with the
    figure.
    """
    from concurrent.futures import ThreadPoolExecutor
    import numpy
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import gemv as G

    usable = len(os.sched_getaffinity(0))
    cores = min(16, usable)
    blas = [{k: d.get(k) for k in ("internal_api", "version", "threading_layer", "num_threads")}
            for d in threadpool_info() if d.get("user_api") == "blas"]
    arrays, x, n, gs = wl.host, wl.x_host, wl.n, wl.gs
    blocks = [(r, min(n, r + 2048)) for r in range(0, n, 2048)]

    def one(bounds):
        r0, r1 = bounds
        if wl.fmt == "fp4":
            return G.gemv_fp4_e2m1(arrays[0][r0:r1], arrays[1][r0:r1], x, gs)
        if wl.fmt in ("u4", "u8"):
            return G.gemv_affine(arrays[0][r0:r1], arrays[1][r0:r1], arrays[2][r0:r1], x,
                                 4 if wl.fmt == "u4" else 8, gs)
        return G.gemv_fp8_e4m3(arrays[0][r0:r1], arrays[1][r0:r1], x)

    passes = 0
    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(cores) as ex:
        while True:
            list(ex.map(one, blocks))
            passes += 1
            if time.perf_counter() - t0 >= target_s:
                break
    dt = time.perf_counter() - t0
    return {
        "value": round(wl.bytes * passes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d full %dx%d matvecs (same packed weights and x), float64 oracle, "
                  "%d threads over 2048-row blocks, %.1f s" % (passes, wl.n, wl.k, cores, dt),
        "host": {"os_cpu_count": os.cpu_count(), "usable_cpus": usable, "threads": cores,
                 "numpy": numpy.__version__, "blas": blas},
    }


# ------------------------------------------------------------------ modes

def parse_plan(s):
    if not s:
        return None
    r, w, b = (int(v) for v in s.split(","))
    return {"rows_per_tile": r, "waves_per_block": w, "blocks": b}


def run_default(args):
    import torch
    plan = parse_plan(args.plan)
    wl = Workload("fp4", "gate_up", batch=1, gs=32, plan=plan, keep_host=not args.no_cpu_baseline)
    log("bench: %s, %d weight copies (%.2f GB), %d warmup + %d timed steps, mode=%s"
        % (wl.label(), wl.copies, wl.copies * (wl.bytes / 1e9), args.warmup, args.steps, args.mode))
    ms = time_steps(wl.launch, args.steps, args.warmup, args.mode)
    ms_per_step = ms / args.steps
    gbs = wl.bytes / (ms_per_step * 1e-3) / 1e9
    log("bench: %.3f ms for %d steps -> %.2f us/step, %.1f GB/s (%.1f%% of 8 TB/s)"
        % (ms, args.steps, ms_per_step * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS))
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4_e2m1 weights, bf16 x, f32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the host, N(0,1) bf16 x)",
        "config": {
            "workload": "Gemma-4-12B FP4-E2M1 gate_up matvec W[30720x3840] group-32 bf16 scales, batch 1",
            "n": wl.n, "k": wl.k, "batch": 1, "group_size": 32,
            "us_per_matvec": round(ms_per_step * 1e3, 3),
            "algorithmic_bytes_per_step": wl.bytes,
            "weight_copies_rotated": wl.copies,
            "launch": args.mode,
            "plan": wl.q.qg_plan_query(wl.q.QG_FMT_FP4_E2M1, wl.n, wl.k, 1) if plan is None else plan,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out))


SWEEP = [
    ("fp4", "gate_up", 1, 32), ("fp4", "qkv", 1, 32), ("fp4", "o_proj", 1, 32), ("fp4", "fc_down", 1, 32),
    ("u4", "mlp_up", 1, 64), ("u4", "mlp_down", 1, 64), ("u4", "llama_up", 1, 64), ("u4", "llama_down", 1, 64),
    # the two-level super-block 4-bit format beside affine u4 g64 (pre-unpacked device layout)
    ("q4k", "mlp_up", 1, None), ("q4k", "mlp_down", 1, None), ("q4k", "llama_up", 1, None),
    ("q4k", "llama_down", 1, None), ("q4k", "mlp_up", 4, None),
    ("u8", "mlp_up", 1, 64), ("u8", "mlp_down", 1, 64), ("u8", "llama_up", 1, 64), ("u8", "llama_down", 1, 64),
    ("fp8", "lm_head", 1, None), ("fp8", "lm_head", 4, None), ("fp4", "tiny", 1, 32),
    # batch 2-4 (batch 3-4 of the 4-bit formats on the matrix blocks)
    ("fp4", "gate_up", 2, 32), ("fp4", "gate_up", 3, 32), ("fp4", "gate_up", 4, 32), ("fp4", "qkv", 4, 32),
    ("fp4", "o_proj", 4, 32), ("fp4", "fc_down", 4, 32), ("u4", "mlp_up", 3, 64),
    # the int8 activation route for u4 (quantize + matvec, and the matvec
    # alone) beside the bf16 route, at batch 1 and 4
    ("u4q8", "mlp_up", 1, 64), ("u4q8mv", "mlp_up", 1, 64), ("u4q8", "mlp_down", 1, 64),
    ("u4q8mv", "mlp_down", 1, 64), ("u4q8", "llama_up", 1, 64), ("u4q8", "llama_down", 1, 64),
    ("u4", "mlp_up", 4, 64), ("u4q8", "mlp_up", 4, 64), ("u4", "mlp_down", 4, 64), ("u4q8", "mlp_down", 4, 64),
    # quantization inside the matvec (one launch)
    ("u4q8f", "mlp_up", 1, 64), ("u4q8f", "mlp_down", 1, 64), ("u4q8f", "llama_up", 1, 64),
    ("u4q8f", "llama_down", 1, 64), ("u4q8f", "mlp_up", 4, 64), ("u4q8f", "mlp_down", 4, 64),
    ("u4", "mlp_up", 2, 64), ("u4q8f", "mlp_up", 2, 64),
    # the int8 route for 8-bit codes beside the bf16 route (whose fp32
    # activations at 3840x15360, batch 4, are read from memory with the
    # weights instead of staged in LDS)
    ("u8", "mlp_up", 4, 64), ("u8", "mlp_down", 4, 64), ("q4k", "mlp_down", 4, None),
    ("u8q8", "mlp_up", 1, 64), ("u8q8", "mlp_down", 1, 64), ("u8q8", "mlp_up", 4, 64), ("u8q8", "mlp_down", 4, 64),
    ("u8q8f", "mlp_up", 1, 64), ("u8q8f", "mlp_down", 1, 64), ("u8q8f", "mlp_up", 4, 64),
    ("u8q8f", "mlp_down", 4, 64),
    # one GPU's share of the Gemma shapes and the lm_head at tensor-parallel
    # degree 8 (rows split for gate_up, qkv and the lm_head; K for o_proj and
    # fc_down)
    ("fp4", "gate_up_tp8", 1, 32), ("fp4", "qkv_tp8", 1, 32), ("fp4", "o_proj_tp8", 1, 32),
    ("fp4", "fc_down_tp8", 1, 32), ("fp8", "lm_head_tp8", 1, None),
]


def timed_steps(launch, mode, target_ms=25.0):
    """Steps for a timed region of about target_ms: the first launches of a
    short region run at lower clocks (a 200-launch region of the 30720x3840
    FP4 matvec times about 8% slower per launch than a 2000-launch one)."""
    est = time_steps(launch, 20, 5, mode) / 20
    return int(min(4000, max(50, target_ms / max(est, 1e-4))))


def run_sweep(args):
    import torch
    rows = []
    only = set(args.only.split(",")) if args.only else None
    for fmt, name, batch, gs in SWEEP:
        if only and name not in only and "%s:%s" % (fmt, name) not in only \
                and "%s:%s:%d" % (fmt, name, batch) not in only:
            continue
        wl = Workload(fmt, name, batch=batch, gs=gs, plan=parse_plan(args.plan))
        steps = args.sweep_steps or timed_steps(wl.launch, args.mode)
        ms = time_steps(wl.launch, steps, max(1, steps // 10), args.mode)
        us = ms / steps * 1e3
        gbs = wl.bytes / (us * 1e-6) / 1e9
        row = {"fmt": fmt, "shape": name, "n": wl.n, "k": wl.k, "batch": batch, "group_size": gs,
               "bytes": wl.bytes, "copies": wl.copies, "us": round(us, 3), "GBps": round(gbs, 1),
               "frac_8TBps": round(gbs / HBM_PEAK_GBS, 4)}
        rows.append(row)
        log("%-42s %9.2f us  %8.1f GB/s  %5.1f%%" % (wl.label(), us, gbs, 100 * gbs / HBM_PEAK_GBS))
        del wl
        torch.cuda.empty_cache()
    if not only or "qgemm" in only:
        rows.extend(run_qgemm_sweep(args))
    if not only or "step48" in only:
        step = run_decode_step(args)
        per_shape = {r["shape"]: r["us"] for r in rows
                     if r["fmt"] == "fp4" and r.get("kernel") != "qgemm" and r.get("batch") == 1}
        if all(s in per_shape for s in ("qkv", "o_proj", "gate_up", "fc_down")):
            # the step beside 48 x the sum of the per-shape times measured alone
            step["sum_of_shapes_us"] = round(48 * sum(per_shape[s] for s in ("qkv", "o_proj", "gate_up", "fc_down")), 2)
            log("%-42s %9.2f us  (48 x the four per-shape times above)" % ("fp4 48 x (qkv+o_proj+gate_up+fc_down)",
                                                                           step["sum_of_shapes_us"]))
        rows.append(step)
    if args.out:
        with open(args.out, "w") as f:
            json.dump(rows, f, indent=1)


def run_qgemm_sweep(args):
    """The small-batch GEMMs (qgemm_fp4_e2m1 on the Gemma-4-12B FP4 shapes,
    qgemm_affine_u4 on 15360x3840 and 3840x15360 g64) at m = 8 .. 128
    activation rows: algorithmic bytes (weights + parameters once, x, y) per
    launch and MFMA rate, beside the same work done by ceil(m/4) launches of
    the batch-4 matvec (which re-reads the weights each time)."""
    import torch
    import block_quantized_weight_qgemv_amd as q
    import synth
    rows = []
    for fmt, name in (("fp4", "gate_up"), ("fp4", "qkv"), ("fp4", "fc_down"), ("u4", "mlp_up"), ("u4", "mlp_down")):
        gs = 32 if fmt == "fp4" else 64
        wl = Workload(fmt, name, batch=4, gs=gs)
        wbytes = q.qg_bytes_fp4(wl.n, wl.k, gs) if fmt == "fp4" else q.qg_bytes_affine(wl.n, wl.k, 4, gs)
        sid = synth.shape(name)[0]
        for m in (8, 16, 32, 64, 128):
            x = to_dev(synth.activations(sid, m, wl.k))
            y = torch.empty((m, wl.n), dtype=torch.float32, device="cuda:0")

            def gemm(i):
                d = wl.dev[i % wl.copies]
                if fmt == "fp4":
                    q.qgemm_fp4_e2m1(d[0], d[1], x, y, gs)
                else:
                    q.qgemm_affine_u4(d[0], d[1], d[2], x, y, gs)

            steps = timed_steps(gemm, args.mode)
            us = time_steps(gemm, steps, max(1, steps // 10), args.mode) / steps * 1e3
            nbytes = wbytes + m * wl.k * 2 + m * wl.n * 4
            gbs = nbytes / (us * 1e-6) / 1e9
            tflops = 2.0 * m * wl.n * wl.k / (us * 1e-6) / 1e12
            calls = (m + 3) // 4

            def matvecs(i):
                for j in range(calls):
                    wl.launch(i * calls + j)

            msteps = max(10, timed_steps(matvecs, args.mode) // 2)
            us_mv = time_steps(matvecs, msteps, max(1, msteps // 10), args.mode) / msteps * 1e3
            rows.append({"fmt": fmt, "shape": name, "kernel": "qgemm", "n": wl.n, "k": wl.k, "m": m,
                         "bytes": nbytes, "us": round(us, 3), "GBps": round(gbs, 1),
                         "frac_8TBps": round(gbs / HBM_PEAK_GBS, 4), "mfma_TFLOPs": round(tflops, 1),
                         "matvec_b4_x%d_us" % calls: round(us_mv, 3)})
            log("%-42s %9.2f us  %8.1f GB/s  %5.1f%%  %6.1f TFLOP/s  (%d batch-4 matvecs: %.2f us)"
                % ("qgemm %s %s [%dx%d] m=%d" % (fmt, name, wl.n, wl.k, m), us, gbs, 100 * gbs / HBM_PEAK_GBS,
                   tflops, calls, us_mv))
            del x, y
        del wl
        torch.cuda.empty_cache()
    return rows


def run_decode_step(args, layers=48):
    """The FP4 decode step: qkv, o_proj, gate_up, fc_down for 48 distinct layers.

    Also the step with an RMSNorm before qkv and before gate_up (the two norms
    of a pre-norm decoder layer), once fused into those matvecs and once as
    separate norm launches (the same norm arithmetic) ahead of plain matvecs."""
    import torch
    import block_quantized_weight_qgemv_amd as q
    shapes = ["qkv", "o_proj", "gate_up", "fc_down"]
    wls = [Workload("fp4", s, batch=1, gs=32, copies=layers) for s in shapes]
    total = sum(w.bytes for w in wls) * layers
    per_step = layers * len(shapes)
    reps = 10                     # decode steps per timed region (~15 ms)

    def timed(launch, n_launch):
        ms_runs = [time_steps(launch, per_step * reps, per_step * 2, args.mode) / reps for _ in range(3)]
        ms = float(np.median(ms_runs))
        gbs = total / (ms * 1e-3) / 1e9
        return ms, gbs

    def launch(i):
        layer = i // len(shapes)
        wls[i % len(shapes)].launch(layer)

    ms, gbs = timed(launch, per_step)
    log("%-42s %9.2f us  %8.1f GB/s  %5.1f%%  (192 launches per step; 10 steps per region, median of 3)"
        % ("fp4 48-layer decode step", ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS))
    row = {"fmt": "fp4", "shape": "decode_step_48_layers", "bytes": total, "launches": per_step,
           "us": round(ms * 1e3, 2), "GBps": round(gbs, 1), "frac_8TBps": round(gbs / HBM_PEAK_GBS, 4)}

    # with the two RMSNorms per layer
    normed = {0: 3840, 2: 3840}           # shape index -> k (qkv and gate_up read the normed stream)
    rng = np.random.default_rng(7)
    gammas = {si: torch.from_numpy(rng.uniform(0.5, 1.5, k).astype(np.float32)).to("cuda:0").to(torch.bfloat16)
              for si, k in normed.items()}
    xn = {si: torch.empty_like(wls[si].x) for si in normed}

    def launch_fused(i):
        layer, si = i // len(shapes), i % len(shapes)
        w = wls[si]
        if si in normed:
            d = w.dev[layer % w.copies]
            q.qgemv_fp4_e2m1_rmsnorm(d[0], d[1], w.x, gammas[si], 1e-6, w.y, 32)
        else:
            w.launch(layer)

    def launch_separate(i):
        layer, si = i // len(shapes), i % len(shapes)
        w = wls[si]
        if si in normed:
            d = w.dev[layer % w.copies]
            q.qg_rmsnorm_bf16(w.x, gammas[si], 1e-6, xn[si])
            q.qgemv_fp4_e2m1(d[0], d[1], xn[si], w.y, 32)
        else:
            w.launch(layer)

    for name, fn, n_launch, key in (("fused", launch_fused, per_step, "norm_fused_us"),
                                    ("separate", launch_separate, per_step + 2 * layers, "norm_separate_us")):
        ms_n, gbs_n = timed(fn, n_launch)
        row[key] = round(ms_n * 1e3, 2)
        log("%-42s %9.2f us  %8.1f GB/s  %5.1f%%  (%d launches per step)"
            % ("fp4 48-layer step + 96 RMSNorms, %s" % name, ms_n * 1e3, gbs_n, 100 * gbs_n / HBM_PEAK_GBS, n_launch))
    del wls
    torch.cuda.empty_cache()
    return row


def run_probe(args):
    """Achievable HBM read bandwidth: the stream probe over a 2 GiB buffer, and
    over 64 MiB windows rotating through it (the size of one matvec)."""
    import torch
    import block_quantized_weight_qgemv_amd as q
    total = 2 << 30
    buf = torch.empty(total, dtype=torch.uint8, device="cuda:0").fill_(7)
    rows = []
    for window in (total, 64 << 20):
        nwin = total // window
        best = {}
        for pattern in (3, 4, 5):
            for unroll in (4, 8, 16):
                for tpb in (256, 512):
                    for waves_per_cu in (8, 16, 32):
                        blocks = 256 * waves_per_cu * 64 // tpb
                        out = torch.empty(blocks * tpb, dtype=torch.int32, device="cuda:0")
                        views = [buf[i * window:(i + 1) * window] for i in range(nwin)]
                        launch = lambda i: q.qg_stream_probe(views[i % nwin], pattern, unroll, blocks, tpb, out)
                        steps = 10 if window == total else 64
                        ms = time_steps(launch, steps, 2, "graph") / steps
                        gbs = window / (ms * 1e-3) / 1e9
                        rows.append({"window": window, "pattern": pattern, "unroll": unroll, "threads": tpb,
                                     "blocks": blocks, "us": round(ms * 1e3, 2), "GBps": round(gbs, 1)})
                        if gbs > best.get(pattern, (0,))[0]:
                            best[pattern] = (gbs, unroll, tpb, blocks, ms * 1e3)
        for pattern, b in sorted(best.items()):
            log("probe window=%5d MiB pattern=%d best: %.1f GB/s (%.1f%% of 8 TB/s) %.2f us unroll=%d tpb=%d blocks=%d"
                % (window >> 20, pattern, b[0], 100 * b[0] / HBM_PEAK_GBS, b[4], b[1], b[2], b[3]))
    if args.out:
        with open(args.out, "w") as f:
            json.dump(rows, f, indent=1)


def run_probe_sizes(args):
    """The stream probe at each sweep workload's algorithmic byte count
    (windows of that size rotating through 2 GiB, so the Infinity Cache cannot
    serve them; best of a few launch shapes), beside the workload's own time
    in the same session: how close each launch gets to a plain read of its
    bytes, launch overhead and ramp included for both."""
    import torch
    import block_quantized_weight_qgemv_amd as q
    total = 2 << 30
    buf = torch.empty(total, dtype=torch.uint8, device="cuda:0").fill_(7)
    rows = []
    for fmt, name, batch, gs in SWEEP:
        if fmt == "fp4" and name == "tiny":
            continue
        wl = Workload(fmt, name, batch=batch, gs=gs)
        steps = timed_steps(wl.launch, args.mode)
        us = time_steps(wl.launch, steps, max(1, steps // 10), args.mode) / steps * 1e3
        nbytes = wl.bytes
        del wl
        torch.cuda.empty_cache()
        window = (nbytes + 15) // 16 * 16
        nwin = max(1, total // window)
        views = [buf[i * window:(i + 1) * window] for i in range(nwin)]
        best = None
        for pattern in (4, 5):
            for unroll in (8, 16):
                for waves_per_cu in (8, 16):
                    tpb = 512
                    blocks = 256 * waves_per_cu * 64 // tpb
                    out = torch.empty(blocks * tpb, dtype=torch.int32, device="cuda:0")
                    launch = lambda i: q.qg_stream_probe(views[i % nwin], pattern, unroll, blocks, tpb, out)
                    ps = timed_steps(launch, args.mode)
                    pus = time_steps(launch, ps, max(1, ps // 10), args.mode) / ps * 1e3
                    if best is None or pus < best[0]:
                        best = (pus, pattern, unroll, blocks)
        row = {"fmt": fmt, "shape": name, "batch": batch, "bytes": nbytes, "us": round(us, 3),
               "probe_us": round(best[0], 3), "probe_config": {"pattern": best[1], "unroll": best[2],
                                                              "blocks": best[3], "threads": 512},
               "us_over_probe": round(us / best[0], 3)}
        rows.append(row)
        log("%-4s %-10s B=%d %11d B  matvec %8.2f us  read stream %8.2f us  ratio %.3f  (%.1f%% / %.1f%% of 8 TB/s)"
            % (fmt, name, batch, nbytes, us, best[0], us / best[0],
               100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 100 * nbytes / (best[0] * 1e-6) / 1e9 / HBM_PEAK_GBS))
    if args.out:
        with open(args.out, "w") as f:
            json.dump(rows, f, indent=1)


def _pmc_median(run_dir, counter, kernel_substr):
    import csv
    import glob
    import statistics
    vals = []
    for path in glob.glob(os.path.join(run_dir, "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no %s values for kernels matching %r in %s" % (counter, kernel_substr, run_dir))
    return statistics.median(vals), len(vals)


def run_summarize_pmc(args):
    """FETCH_SIZE and WRITE_SIZE per matvec launch, scaled by the counters of a
    plain copy of COPY_BYTES (read COPY_BYTES, wrote COPY_BYTES)."""
    fetch_dir, write_dir, copy_fetch_dir, copy_write_dir = args.summarize_pmc
    k_fetch, n1 = _pmc_median(fetch_dir, "FETCH_SIZE", args.pmc_kernel)
    k_write, n2 = _pmc_median(write_dir, "WRITE_SIZE", args.pmc_kernel)
    c_fetch, _ = _pmc_median(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    c_write, _ = _pmc_median(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    f_scale = COPY_BYTES / (c_fetch * 1024.0)
    w_scale = COPY_BYTES / (c_write * 1024.0)
    fetch_b = k_fetch * 1024.0 * f_scale
    write_b = k_write * 1024.0 * w_scale
    default = args.pmc_workload == ""
    out = {
        "workload": "FP4-E2M1 gate_up W[30720x3840] group 32, batch 1 (bench.py default)" if default
        else args.pmc_workload,
        "kernel": args.pmc_kernel,
        "kernel_source_sha256": kernel_source_hash(),
        "fetch_size_kib_median": k_fetch, "write_size_kib_median": k_write, "dispatches": [n1, n2],
        "copy_bytes": COPY_BYTES, "copy_fetch_size_kib": c_fetch, "copy_write_size_kib": c_write,
        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
        "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
        "hbm_read_bytes_per_launch": int(round(fetch_b)),
        "hbm_write_bytes_per_launch": int(round(write_b)),
        "algorithmic_bytes_per_launch": algorithmic_bytes("fp4", 30720, 3840, 1, 32) if default
        else int(args.pmc_bytes),
        "commands": args.commands or "",
    }
    with open(args.out or TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    log(json.dumps(out, indent=1))


BUSY_FILE = os.path.join(ROOT, "profiles", "fp4_gate_up_30720x3840_busy.json")
BUSY_COUNTERS = ["VALUBusy", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE", "TA_BUSY_avr", "SQ_INSTS_VALU",
                 "SQ_INSTS_VMEM_RD", "SQ_WAVES", "SQ_WAVE_CYCLES"]


def run_summarize_busy(args):
    """VALU busy against memory-unit (TA) busy for the matvec kernel, from one
    rocprofv3 --pmc run with BUSY_COUNTERS (medians over dispatches).

    VALUBusy is rocprofv3's derived counter: 100 * sum(SQ_ACTIVE_INST_VALU) /
    CU_NUM / max(GRBM_GUI_ACTIVE) (SQ_ACTIVE_INST_VALU counts quad-cycles).
    rocprofv3 reports GRBM_GUI_ACTIVE summed over the 8 XCDs, so one XCD's
    active cycles are GRBM_GUI_ACTIVE / 8; memory-unit busy is TA_BUSY_avr
    (busy cycles averaged over the TA instances, one per CU) over that."""
    run_dir = args.summarize_busy
    med = {}
    for c in BUSY_COUNTERS:
        med[c], n = _pmc_median(run_dir, c, args.pmc_kernel)
    gui_per_xcd = med["GRBM_GUI_ACTIVE"] / 8.0
    default = args.pmc_workload == ""
    out = {
        "workload": "FP4-E2M1 gate_up W[30720x3840] group 32, batch 1 (bench.py default)" if default
        else args.pmc_workload,
        "kernel": args.pmc_kernel,
        "kernel_source_sha256": kernel_source_hash(),
        "dispatches": n,
        "counters_median": med,
        "valu_busy_pct": round(med["VALUBusy"], 2),
        "mem_unit_busy_pct": round(100.0 * med["TA_BUSY_avr"] / gui_per_xcd, 2),
        "gpu_active_cycles_per_xcd": gui_per_xcd,
        "valu_insts_per_wave": round(med["SQ_INSTS_VALU"] / med["SQ_WAVES"], 1),
        "vmem_read_insts_per_wave": round(med["SQ_INSTS_VMEM_RD"] / med["SQ_WAVES"], 1),
        "commands": args.commands or "",
    }
    with open(args.out or BUSY_FILE, "w") as f:
        json.dump(out, f, indent=1)
    log(json.dumps(out, indent=1))


def run_summarize_trace(args):
    """Short text summary of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    run_dir = args.summarize_trace
    lines = ["# rocprofv3 kernel-trace summary", "# command: %s" % (args.commands or "?"), ""]
    for path in sorted(glob.glob(os.path.join(run_dir, "*kernel_stats.csv"))):
        rows = list(csv.DictReader(open(path)))
        lines.append("%-70s %7s %12s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct"))
        for r in rows:
            name = r.get("Name", "")[:70]
            lines.append("%-70s %7s %12.3f %12.3f %12.3f %12.2f" % (
                name, r.get("Calls", ""), float(r.get("AverageNs", 0)) / 1e3, float(r.get("MinNs", 0)) / 1e3,
                float(r.get("MaxNs", 0)) / 1e3, float(r.get("Percentage", 0))))
    for path in sorted(glob.glob(os.path.join(run_dir, "*kernel_trace.csv"))):
        import statistics
        durs = {}
        for r in csv.DictReader(open(path)):
            durs.setdefault(r["Kernel_Name"][:70], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines.append("")
        lines.append("%-70s %7s %10s %10s %10s" % ("kernel (per-dispatch durations)", "n", "median_us", "p10_us", "p90_us"))
        for k, v in durs.items():
            v = sorted(v)
            lines.append("%-70s %7d %10.3f %10.3f %10.3f" % (k, len(v), statistics.median(v),
                                                          v[len(v) // 10], v[(len(v) * 9) // 10]))
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def run_calibrate_copy(args):
    """A plain device copy of known size, for scaling the rocprofv3 byte counters."""
    import torch
    nbytes = COPY_BYTES
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("calibrate: copied %d bytes 3 times (each copy reads %d and writes %d bytes)" % (nbytes, nbytes, nbytes))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--mode", choices=["graph", "stream"], default="graph")
    ap.add_argument("--plan", default="", help="rows_per_tile,waves_per_block,blocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--only", default="", help="with --sweep: comma list of shape names, fmt:shape or fmt:shape:batch")
    ap.add_argument("--sweep-steps", type=int, default=0,
                    help="with --sweep: this many timed steps per workload (default: about 25 ms of them)")
    ap.add_argument("--out", default="")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--probe", action="store_true", help="stream-probe read bandwidth sweep")
    ap.add_argument("--probe-sizes", action="store_true",
                    help="stream probe at each sweep workload's byte count, beside the workload")
    ap.add_argument("--summarize-pmc", nargs=4, metavar="DIR",
                    help="fetch, write, copy-fetch and copy-write rocprofv3 --pmc output dirs")
    ap.add_argument("--pmc-kernel", default="qgemv", help="with --summarize-pmc: kernel name substring")
    ap.add_argument("--pmc-workload", default="", help="with --summarize-pmc: workload label (default: the bench line's)")
    ap.add_argument("--pmc-bytes", default="0", help="with --summarize-pmc and --pmc-workload: algorithmic bytes")
    ap.add_argument("--summarize-trace", metavar="DIR", help="rocprofv3 --kernel-trace --stats output dir")
    ap.add_argument("--summarize-busy", metavar="DIR",
                    help="rocprofv3 --pmc output dir holding BUSY_COUNTERS (VALU and memory-unit busy)")
    ap.add_argument("--commands", default="", help="with --summarize-*: the commands that made the data")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        run_summarize_pmc(args)
        return 0
    if args.summarize_trace:
        run_summarize_trace(args)
        return 0
    if args.summarize_busy:
        run_summarize_busy(args)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py runs on one GPU only: this matvec library has no multi-GPU path "
                         "(rows would shard across GPUs with no exchange between them)\n")
        return 2
    import torch
    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a HIP device\n")
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        run_calibrate_copy(args)
    elif args.probe:
        run_probe(args)
    elif args.probe_sizes:
        run_probe_sizes(args)
    elif args.sweep:
        run_sweep(args)
    else:
        run_default(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
