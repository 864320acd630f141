"""Offline quantizers (the host-side step before the matvec).  Test infrastructure.

The quantizers decide which codes the matvec consumes, not whether the matvec
is right: the oracle and the GPU read the same codes.  They are here so the
oracle can rebuild, independently of the library's C++ pack module, the exact
codes that a seeded fp32 weight matrix must produce; the tests compare the two
bit for bit.

All arithmetic is float64 on exact inputs, with one rounding per operation,
in this order (the C++ pack module has to do the same operations):

FP4-E2M1, group absmax (Part 2 post, "The assumption that failed the
profiler"; the page gives per-group scales but not their derivation: this
module reads them as absmax/6, the scale that maps the group's largest
magnitude onto E2M1's largest value):
    s  = bf16_rne(absmax_g / 6)
    c  = e2m1_rne(w / s)          (saturating at 6; s == 0 -> every code 0)

Affine min-max, group 64 (#683, "Step 2 result": scale and bias rounded to
bf16 *before* q is computed, "self-consistent triples"):
    s  = bf16_rne((max_g - min_g) / (2**bits - 1))
    b  = bf16_rne(min_g)
    q  = clamp(rint((w - b) / s), 0, 2**bits - 1)     (rint: half to even;
                                                        s == 0 -> q = 0)

FP8-E4M3, one fp32 scale per row (the page: "one FMA per byte with no
dequant", a row scale applied once):
    s_n = fl32(absmax_n / 448)    (binary32 division)
    c   = e4m3_rne(w / s_n)       (saturating at 448; s_n == 0 -> code 0)

The sign bit of an FP code is set iff w < 0.
"""

import numpy as np

from .formats import (bf16_bits_to_f64, f64_to_bf16_bits, e2m1_rne_codes,
                      e4m3_rne_codes)
from .layout import pack_nibbles, pack_u32

_BLOCK_ROWS = 64        # bounds the float64 temporaries


def _check_w(w, group_size=None):
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise ValueError("weights must be a 2-D float32 array")
    if not np.isfinite(w).all():
        raise ValueError("weights must be finite")
    if group_size is not None and (group_size <= 0 or w.shape[1] % group_size):
        raise ValueError("K=%d is not a multiple of group_size=%r" % (w.shape[1], group_size))
    return w


def quantize_fp4_e2m1(w, group_size):
    """fp32 [N, K] -> (codes uint8 [N, K/2], scales bf16 bits uint16 [N, K/gs])."""
    w = _check_w(w, group_size)
    n, k = w.shape
    ng = k // group_size
    codes = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, ng), dtype=np.uint16)
    for r0 in range(0, n, _BLOCK_ROWS):
        g = w[r0:r0 + _BLOCK_ROWS].astype(np.float64).reshape(-1, ng, group_size)
        absmax = np.abs(g).max(axis=-1)
        s_bits = f64_to_bf16_bits(absmax / 6.0)
        s = bf16_bits_to_f64(s_bits)
        zero = s == 0.0
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = g / np.where(zero, 1.0, s)[..., None]
        c = e2m1_rne_codes(ratio)
        c[np.broadcast_to(zero[..., None], c.shape)] = 0
        codes[r0:r0 + _BLOCK_ROWS] = pack_nibbles(c.reshape(-1, k))
        scales[r0:r0 + _BLOCK_ROWS] = s_bits
    return codes, scales


def quantize_affine(w, bits, group_size):
    """fp32 [N, K] -> (codes uint32 [N, K*bits/32], scales, biases bf16 bits [N, K/gs])."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    w = _check_w(w, group_size)
    n, k = w.shape
    ng = k // group_size
    qmax = float((1 << bits) - 1)
    codes = np.empty((n, k * bits // 32), dtype=np.uint32)
    scales = np.empty((n, ng), dtype=np.uint16)
    biases = np.empty((n, ng), dtype=np.uint16)
    for r0 in range(0, n, _BLOCK_ROWS):
        g = w[r0:r0 + _BLOCK_ROWS].astype(np.float64).reshape(-1, ng, group_size)
        mn = g.min(axis=-1)
        mx = g.max(axis=-1)
        s_bits = f64_to_bf16_bits((mx - mn) / qmax)
        b_bits = f64_to_bf16_bits(mn)
        s = bf16_bits_to_f64(s_bits)[..., None]
        b = bf16_bits_to_f64(b_bits)[..., None]
        zero = s == 0.0
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.rint((g - b) / np.where(zero, 1.0, s))
        q = np.clip(q, 0.0, qmax)
        q = np.where(zero, 0.0, q).astype(np.uint8)
        codes[r0:r0 + _BLOCK_ROWS] = pack_u32(q.reshape(-1, k), bits)
        scales[r0:r0 + _BLOCK_ROWS] = s_bits
        biases[r0:r0 + _BLOCK_ROWS] = b_bits
    return codes, scales, biases


def quantize_fp8_e4m3_rowwise(w):
    """fp32 [N, K] -> (codes uint8 [N, K], row_scale float32 [N])."""
    w = _check_w(w)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    row_scale = np.empty(n, dtype=np.float32)
    for r0 in range(0, n, _BLOCK_ROWS):
        blk = w[r0:r0 + _BLOCK_ROWS]
        absmax = np.abs(blk).max(axis=-1)                     # float32, exact
        s = (absmax / np.float32(448.0)).astype(np.float32)   # one binary32 rounding
        zero = s == 0.0
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = blk.astype(np.float64) / np.where(zero, 1.0, s.astype(np.float64))[:, None]
        c = e4m3_rne_codes(ratio)
        c[np.broadcast_to(zero[:, None], c.shape)] = 0
        codes[r0:r0 + _BLOCK_ROWS] = c
        row_scale[r0:r0 + _BLOCK_ROWS] = s
    return codes, row_scale
