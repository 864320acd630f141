"""Int8 activation route for affine 4-bit and 8-bit weights.  Test infrastructure.

Source: "perf(cuda): generalize Gemma 4 batched prefill + flash attn + decode
graphs to dense Q4_K models", section "Item C2": the activation is quantized
to int8 blocks (q8_1) whose 32-bit word ds carries an fp16 pair, d in the low
half and the block's activation sum s = d * sum(q) in the high half; the
weight nibbles become int8, and the affine minimum is applied once per block
through s.  The decode notes of the same issue say the Q4_K matvec runs on
4-wide int8 dots.  The pages do not print the activation quantizer itself.
Reading taken here (the plainest one the rest supports):

  block   32 consecutive activations of one batch row (one Q4_K sub-block,
          which is also one 16-byte chunk of u4 codes)
  amax    max_k |x[k]| over the block (exact: x is bf16)
  d       fp16_rne(amax / 127), the value the block stores
  q[k]    clamp(rne(x[k] / d), -127, 127), with the stored d, so that d * q
          is the nearest point of the grid the block actually carries (the
          same rule as the affine weight quantizer, whose scale is rounded
          before its codes are chosen); q = 0 when d = 0 (an all-zero block,
          or a block whose amax / 127 rounds to zero in fp16)
  s       fp16_rne(d * sum_k q[k])

Every step here is exact real arithmetic followed by one rounding: amax / 127
and x / d are float64 quotients of short dyadic numbers, which never land on
an fp16 or integer rounding midpoint unless the exact quotient does, and
d * sum(q) is exact in float64.  The fp16 roundings are numpy's float64 ->
float16 cast (round to nearest even; results past the fp16 range become
infinite, so the route is defined for block maxima below 65520 * 127).

The matvec on those blocks then computes, in float64,

  y[b, r] = sum_blocks  scale[r, g] * d_blk * sum_{k in blk} u[r, k] * q[b, k]
                      + bias[r, g] * s_blk

with u the 4-bit or 8-bit codes and g the block's scale group.  Mathematically
this is sum_k (scale*u + bias)[r, k] * (d * q)[b, k] with the block's
activation sum rounded once to fp16 (s); tests pin it against the dequantized
weights of oracle.gemv applied to the dequantized activations d * q.
"""

import numpy as np

from .formats import bf16_bits_to_f64
from .layout import unpack_u32

BLOCK = 32
QMAX = 127


def quantize_q8_1(x_bits):
    """bf16 bits [B, K] -> (q int8 [B, K], d float16 [B, K/32], s float16 [B, K/32]).

    The device layout of a block's pair is one 32-bit word: d's fp16 bits in
    the low half, s's in the high half (see ``pack_ds``).
    """
    x_bits = np.atleast_2d(np.asarray(x_bits, dtype=np.uint16))
    bsz, k = x_bits.shape
    if k % BLOCK:
        raise ValueError("K=%d is not a multiple of %d" % (k, BLOCK))
    x = bf16_bits_to_f64(x_bits).reshape(bsz, k // BLOCK, BLOCK)      # exact
    amax = np.max(np.abs(x), axis=2)
    d16 = (amax / QMAX).astype(np.float16)                             # one RNE rounding
    d = d16.astype(np.float64)                                         # exact
    nz = d > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(nz[:, :, None], x / np.where(nz, d, 1.0)[:, :, None], 0.0)
    q = np.clip(np.rint(ratio), -QMAX, QMAX).astype(np.int8)          # rint: ties to even
    sq = q.astype(np.int64).sum(axis=2)                                # |sum| <= 4064
    s16 = (d * sq).astype(np.float16)                                  # d * sum exact, one rounding
    return q.reshape(bsz, k), d16, s16


def pack_ds(d16, s16):
    """The pairs as the library stores them: uint16 [B, K/32, 2], d then s
    (one little-endian 32-bit word per block, d in its low half)."""
    d16 = np.asarray(d16, dtype=np.float16)
    s16 = np.asarray(s16, dtype=np.float16)
    return np.stack([d16.view(np.uint16), s16.view(np.uint16)], axis=-1)


def gemv_affine_u4_q8(codes, scales, biases, q, d, s, group_size):
    """Affine u4 weights x int8 activation blocks -> (y float64 [B, N], A float64 [B, N]).

    codes uint32 [N, K/8] (low-first nibbles), scales/biases bf16 bits
    [N, K/gs], q int8 [B, K], d and s float16 [B, K/32].  A = sum_k |W^ x^|
    with W^ the dequantized weight and x^ = d * q, the conditioning mass of
    the parity criterion.
    """
    return gemv_affine_q8(codes, scales, biases, q, d, s, 4, group_size)


def gemv_affine_u8_q8(codes, scales, biases, q, d, s, group_size):
    """As gemv_affine_u4_q8 for 8-bit codes, uint32 [N, K/4] low-first bytes."""
    return gemv_affine_q8(codes, scales, biases, q, d, s, 8, group_size)


def gemv_affine_q8(codes, scales, biases, q, d, s, bits, group_size):
    """The block sum for affine codes of `bits` (4 or 8) bits."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, k = codes.shape[0], codes.shape[1] * (32 // bits)
    q = np.atleast_2d(np.asarray(q, dtype=np.int8))
    d = np.atleast_2d(np.asarray(d, dtype=np.float16)).astype(np.float64)
    s = np.atleast_2d(np.asarray(s, dtype=np.float16)).astype(np.float64)
    bsz = q.shape[0]
    nblk = k // BLOCK
    if q.shape[1] != k or d.shape != (bsz, nblk) or s.shape != (bsz, nblk):
        raise ValueError("activation blocks do not match K=%d" % k)
    if group_size % BLOCK or k % group_size:
        raise ValueError("group size %d does not hold whole 32-blocks of K=%d" % (group_size, k))
    sc = bf16_bits_to_f64(np.asarray(scales, dtype=np.uint16))
    bi = bf16_bits_to_f64(np.asarray(biases, dtype=np.uint16))
    grp = np.arange(nblk) * BLOCK // group_size                        # group of each block
    y = np.zeros((bsz, n), dtype=np.float64)
    a = np.zeros((bsz, n), dtype=np.float64)
    qb = q.astype(np.int64).reshape(bsz, nblk, BLOCK)
    xhat = (d[:, :, None] * qb).reshape(bsz, k)                        # d * q, exact in float64
    for r0 in range(0, n, 1024):
        r1 = min(n, r0 + 1024)
        u = unpack_u32(codes[r0:r1], k, bits).astype(np.int64).reshape(r1 - r0, nblk, BLOCK)
        s_blk = sc[r0:r1][:, grp]                                      # [rows, nblk]
        b_blk = bi[r0:r1][:, grp]
        for b in range(bsz):
            idot = np.einsum("rjk,jk->rj", u, qb[b])                   # exact integer dots
            y[b, r0:r1] = np.sum(s_blk * d[b][None, :] * idot + b_blk * s[b][None, :], axis=1)
            w_hat = (np.repeat(s_blk, BLOCK, axis=1) * u.reshape(r1 - r0, k)
                     + np.repeat(b_blk, BLOCK, axis=1))
            a[b, r0:r1] = np.abs(w_hat) @ np.abs(xhat[b])
    return y, a
