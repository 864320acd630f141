"""Dequantize-then-FP64-dot matvec for each weight format.  Test infrastructure.

The method computes, up to fp32 rounding, the plain product

    y[b, n] = sum_k  W^[n, k] * x^[b, k]

where x^ is the bf16 activation read exactly and W^ is the dequantized weight:

  FP4-E2M1   W^[n,k] = bf16(scale[n, k//gs]) * E2M1(code[n,k])
             (Part 2 post, "The assumption that failed the profiler": per-group
             scale folded out of the per-weight math; sign in code bit 3)
  affine     W^[n,k] = bf16(scale[n, k//gs]) * q[n,k] + bf16(bias[n, k//gs])
             (#683 "Step 2 result": group-64 min-max affine codes, u32
             low-first, bf16 scale and bias; the value is the exact real
             s*q + b, not re-rounded to bf16)
  FP8-E4M3   W^[n,k] = row_scale[n] * E4M3(code[n,k])
             (Part 2 post: the FP8 lm_head matvec applies a row scale once)

It is the double-precision, host-side check that the Part 2 post's section
"The test that catches what parity misses" calls for: the GPU's inputs, as
stored (bf16 activations, packed weights), summed without rounding error
worth the name.  Each function also
returns the conditioning mass A[b, n] = sum_k |W^[n,k] x^[b,k]|, which bounds
the rounding error of any summation order and is used by the parity criterion.

Rows are processed in blocks of at most 4096 so that the float64 dequantized
block stays small; within a block the dot is one float64 matrix product (a
library primitive standing for the plain sum).
"""

import numpy as np

from .formats import bf16_bits_to_f64, E2M1_TABLE, E4M3_TABLE
from .layout import unpack_nibbles, unpack_u32

ROW_BLOCK = 4096


def _x_f64(x_bits, k):
    x = np.atleast_2d(np.asarray(x_bits, dtype=np.uint16))
    if x.shape[1] != k:
        raise ValueError("x has %d columns, K=%d" % (x.shape[1], k))
    return bf16_bits_to_f64(x)                       # [B, K]


def _dot(w_hat, x_hat):
    """float64 y and A for one dequantized row block [n, K] and x^ [B, K].

    One matrix-vector product per activation row, so batch rows never
    influence each other's summation order.
    """
    abs_w = np.abs(w_hat)
    y = np.stack([w_hat @ xb for xb in x_hat])       # [B, n]
    a = np.stack([abs_w @ np.abs(xb) for xb in x_hat])
    return y, a


def dequant_fp4_e2m1(codes, scales, k, group_size):
    """FP4 codes [n, K/2] + bf16 scales [n, K/gs] -> W^ float64 [n, K]."""
    c = unpack_nibbles(codes, k)
    s = bf16_bits_to_f64(scales)
    if s.shape[1] * group_size != k:
        raise ValueError("scales have %d groups, K/gs=%d" % (s.shape[1], k // group_size))
    return np.repeat(s, group_size, axis=1) * E2M1_TABLE[c]


def dequant_affine(codes, scales, biases, k, bits, group_size):
    """u32 low-first codes + bf16 scales/biases [n, K/gs] -> W^ float64 [n, K]."""
    q = unpack_u32(codes, k, bits).astype(np.float64)
    s = bf16_bits_to_f64(scales)
    b = bf16_bits_to_f64(biases)
    if s.shape != b.shape or s.shape[1] * group_size != k:
        raise ValueError("scale/bias shape does not match K/gs")
    return np.repeat(s, group_size, axis=1) * q + np.repeat(b, group_size, axis=1)


def dequant_fp8_e4m3(codes, row_scale):
    """E4M3 codes [n, K] + fp32 row scales [n] -> W^ float64 [n, K]."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(row_scale, dtype=np.float32).astype(np.float64)
    return s[:, None] * E4M3_TABLE[c]


def _blocked(n, fn, x_hat):
    b = x_hat.shape[0]
    y = np.empty((b, n), dtype=np.float64)
    a = np.empty((b, n), dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        y[:, r0:r1], a[:, r0:r1] = _dot(fn(r0, r1), x_hat)
    return y, a


def gemv_fp4_e2m1(codes, scales, x_bits, group_size):
    """-> (y float64 [B, N], A float64 [B, N])."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint16)
    n, k = codes.shape[0], codes.shape[1] * 2
    x_hat = _x_f64(x_bits, k)
    return _blocked(n, lambda r0, r1: dequant_fp4_e2m1(codes[r0:r1], scales[r0:r1], k, group_size), x_hat)


def gemv_affine(codes, scales, biases, x_bits, bits, group_size):
    """-> (y float64 [B, N], A float64 [B, N])."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, k = codes.shape[0], codes.shape[1] * (32 // bits)
    x_hat = _x_f64(x_bits, k)
    return _blocked(n, lambda r0, r1: dequant_affine(codes[r0:r1], scales[r0:r1], biases[r0:r1],
                                                     k, bits, group_size), x_hat)


def gemv_fp8_e4m3(codes, row_scale, x_bits):
    """-> (y float64 [B, N], A float64 [B, N])."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    x_hat = _x_f64(x_bits, k)
    return _blocked(n, lambda r0, r1: dequant_fp8_e4m3(codes[r0:r1], row_scale[r0:r1]), x_hat)
