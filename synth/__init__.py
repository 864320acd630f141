"""Seeded synthetic inputs for the quantized matvec: fp32 weights and bf16 activations.

This module is shared by the tests, ``bench.py`` and ``smoke()``: it is the only
code that both the oracle side and the library side receive data from.  It
holds none of the method's arithmetic (no quantization, packing, decoding or
dot products): it only draws random numbers and rounds activations to bf16
with torch's own conversion.

The pages measure on real checkpoints (Gemma-4-12B FP4, gemma-4-12b and
Llama-3.1-8B MLX 4/8-bit) that are not available here; these Gaussian inputs
with the pages' shapes stand in for them.

Recipes
  tiny FP4 (256 x 512):  rng = default_rng(0);
                         W = rng.normal(0, 0.02, (256, 512)).astype(float32);
                         x = rng.normal(0, 1, 512) rounded to bf16.
  every other shape:     row block j (4096 rows) of layer L of shape S is
                         default_rng([0, S, L, j]).standard_normal(dtype=float32) * 0.02;
                         activations are default_rng([0, S, 1, 1000 + B])
                         .standard_normal((B, K)) rounded to bf16.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

BLOCK_ROWS = 4096
WEIGHT_STD = np.float32(0.02)

#: named matvec shapes [N, K] with the stable id used in their seeds
SHAPES = {
    "tiny":          (0, 256, 512),
    "gate_up":       (1, 30720, 3840),     # Gemma-4-12B fused gate+up, FP4
    "qkv":           (2, 8192, 3840),      # Gemma-4-12B local-layer qkv
    "o_proj":        (3, 3840, 4096),
    "fc_down":       (4, 3840, 15360),
    "mlp_up":        (5, 15360, 3840),     # Gemma-4-12B gate or up alone (affine)
    "mlp_down":      (6, 3840, 15360),
    "llama_up":      (7, 14336, 4096),     # Llama-3.1-8B gate/up
    "llama_down":    (8, 4096, 14336),
    "lm_head":       (9, 262144, 3840),    # 262K vocab x hidden 3840
    # one GPU's share at tensor-parallel degree 8: column-parallel layers
    # split their rows, row-parallel layers (o_proj, fc_down) their K
    "gate_up_tp8":   (10, 3840, 3840),
    "qkv_tp8":       (11, 1024, 3840),
    "o_proj_tp8":    (12, 3840, 512),
    "fc_down_tp8":   (13, 3840, 1920),
    "lm_head_tp8":   (14, 32768, 3840),
}


def shape(name):
    """(shape_id, N, K) of a named shape."""
    return SHAPES[name]


def _bf16_bits(x_f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def tiny_fp4_inputs():
    """The tiny FP4 case exactly as specified: (W fp32 [256, 512], x bf16 bits [1, 512])."""
    rng = np.random.default_rng(0)
    w = rng.normal(0, 0.02, (256, 512)).astype(np.float32)
    x = rng.normal(0, 1, 512).astype(np.float32)
    return w, _bf16_bits(x)[None, :]


def _block(shape_id, layer, j, n, k):
    rows = min(BLOCK_ROWS, n - j * BLOCK_ROWS)
    rng = np.random.default_rng([0, shape_id, layer, j])
    w = rng.standard_normal((rows, k), dtype=np.float32)
    w *= WEIGHT_STD
    return w


def weights(shape_id, n, k, layer=0, threads=None):
    """fp32 [N, K] weights ~ N(0, 0.02), generated in independent 4096-row blocks."""
    out = np.empty((n, k), dtype=np.float32)
    nblk = (n + BLOCK_ROWS - 1) // BLOCK_ROWS

    def fill(j):
        out[j * BLOCK_ROWS:(j + 1) * BLOCK_ROWS] = _block(shape_id, layer, j, n, k)

    threads = threads or min(16, os.cpu_count() or 1, nblk)
    if threads <= 1:
        for j in range(nblk):
            fill(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def weight_rows(shape_id, n, k, rows, layer=0):
    """The same values as ``weights(...)[rows]`` without building the whole matrix."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, k), dtype=np.float32)
    for j in np.unique(rows // BLOCK_ROWS):
        blk = _block(shape_id, layer, int(j), n, k)
        sel = np.nonzero(rows // BLOCK_ROWS == j)[0]
        out[sel] = blk[rows[sel] - j * BLOCK_ROWS]
    return out


def activations(shape_id, batch, k):
    """bf16 bits uint16 [B, K], x ~ N(0, 1) rounded to bf16."""
    rng = np.random.default_rng([0, shape_id, 1, 1000 + batch])
    x = rng.standard_normal((batch, k), dtype=np.float32)
    return _bf16_bits(x)


def sample_rows(n, count, seed=0):
    """A seeded, sorted sample of row indices that always includes both ends."""
    rng = np.random.default_rng([0, 99, seed, n])
    pick = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]).astype(np.int64))


def uniform_bytes(shape, seed):
    """Uniform random bytes (every code value of a format, for decode coverage)."""
    return np.random.default_rng([0, 77, seed]).integers(0, 256, shape, dtype=np.uint8)


def uniform_words(shape, seed):
    """Uniform random uint32 words."""
    r = np.random.default_rng([0, 78, seed]).integers(0, 2 ** 32, shape, dtype=np.uint64)
    return r.astype(np.uint32)


def uniform_bf16(shape, lo, hi, seed):
    """bf16 bits of uniform(lo, hi) values."""
    v = np.random.default_rng([0, 79, seed]).uniform(lo, hi, shape).astype(np.float32)
    return _bf16_bits(v)


def uniform_f32(shape, lo, hi, seed):
    return np.random.default_rng([0, 80, seed]).uniform(lo, hi, shape).astype(np.float32)
