"""Int8 activation route for affine 4-bit and 8-bit weights.  Test infrastructure.

Source: "perf(cuda): generalize Gemma 4 batched prefill + flash attn + decode
graphs to dense Q4_K models", sections "Item C2" (the activation is
quantized to int8 blocks carrying a pair {d, s} with s = d * sum(q); the
weight nibbles become int8; the affine minimum is applied once per block
through the activation sum) and the decode notes that the Q4_K matvec runs on
4-wide int8 dots.  The pages do not print the activation quantizer itself.
Reading taken here (the plainest one the rest supports):

  block        32 consecutive activations of one batch row (one Q4_K
               sub-block, which is also one 16-byte chunk of u4 codes)
  amax         max_k |x[k]| over the block (exact: x is bf16)
  d            fp32( amax / 127 )                  (0 for an all-zero block)
  q[k]         rne( fp32( x[k] * fp32(127 / amax) ) ), in [-127, 127]
               (0 for an all-zero block)
  s            fp32( d * sum_k q[k] )

d and s are kept in fp32 (the pages pack them as an fp16 pair).  The
quantization decision (d, the reciprocal, the product and its rounding) is
taken in fp32, the precision the kernel takes it in, so the int8 codes are
compared bit for bit.

The matvec on those blocks then computes, in float64,

  y[b, r] = sum_blocks  scale[r, g] * d_blk * sum_{k in blk} u[r, k] * q[b, k]
                      + bias[r, g] * s_blk

with u the 4-bit or 8-bit codes and g the block's scale group.  Mathematically this is
sum_k (scale*u + bias)[r, k] * (d * q)[b, k] with the block's activation sum
rounded once to fp32 (s); tests pin it against the dequantized weights of
oracle.gemv applied to the dequantized activations d * q.
"""

import numpy as np

from .formats import bf16_bits_to_f64
from .layout import unpack_u32

BLOCK = 32
QMAX = 127


def quantize_q8_1(x_bits):
    """bf16 bits [B, K] -> (q int8 [B, K], d float32 [B, K/32], s float32 [B, K/32])."""
    x_bits = np.atleast_2d(np.asarray(x_bits, dtype=np.uint16))
    bsz, k = x_bits.shape
    if k % BLOCK:
        raise ValueError("K=%d is not a multiple of %d" % (k, BLOCK))
    # bf16 -> fp32 is exact
    x = bf16_bits_to_f64(x_bits).astype(np.float32).reshape(bsz, k // BLOCK, BLOCK)
    amax = np.max(np.abs(x), axis=2)                                   # fp32, exact
    nz = amax > 0
    one = np.float32(1.0)
    safe = np.where(nz, amax, one).astype(np.float32)
    d = np.where(nz, (safe / np.float32(QMAX)).astype(np.float32), np.float32(0)).astype(np.float32)
    inv = np.where(nz, (np.float32(QMAX) / safe).astype(np.float32), np.float32(0)).astype(np.float32)
    prod = (x * inv[:, :, None]).astype(np.float32)                    # one fp32 rounding
    q = np.clip(np.rint(prod), -QMAX, QMAX).astype(np.int8)            # rint: ties to even
    sq = q.astype(np.int64).sum(axis=2).astype(np.float32)             # exact (|sum| <= 4064)
    s = (d * sq).astype(np.float32)
    return q.reshape(bsz, k), d, s


def gemv_affine_u4_q8(codes, scales, biases, q, d, s, group_size):
    """Affine u4 weights x int8 activation blocks -> (y float64 [B, N], A float64 [B, N]).

    codes uint32 [N, K/8] (low-first nibbles), scales/biases bf16 bits
    [N, K/gs], q int8 [B, K], d and s float32 [B, K/32].  A = sum_k |W^ x^|
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
    d = np.atleast_2d(np.asarray(d, dtype=np.float32)).astype(np.float64)
    s = np.atleast_2d(np.asarray(s, dtype=np.float32)).astype(np.float64)
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
