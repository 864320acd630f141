"""RMSNorm of the activations, as the fused matvec variants consume it.  Test
infrastructure.

The Part 2 post ("Where it landed") ranks RMSNorm fusion into the decode step's
matvecs among the next levers; it does not print the norm itself.  This module
takes the standard RMSNorm, row by row, and hands the matvec what a separate
norm kernel would: the normalized activation rounded to bf16,

    r[b]     = 1 / sqrt( (1/K) * sum_k x[b,k]^2  +  eps )
    x~[b,k]  = bf16_rne( x[b,k] * r[b] * gamma[k] )

with x and gamma bf16 values read exactly and the arithmetic in float64.
(Models that scale by (1 + gamma) pass that vector as gamma.)  The fused
product is then the plain matvec of x~ (oracle.gemv).
"""

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_bits


def rms_factor(x_bits, eps):
    """r[b] = 1 / sqrt(mean_k x[b,k]^2 + eps), float64, one per batch row."""
    x = bf16_bits_to_f64(np.atleast_2d(np.asarray(x_bits, dtype=np.uint16)))
    return 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(eps))


def rmsnorm_f64(x_bits, gamma_bits, eps):
    """x * r * gamma in float64 [B, K], before the rounding to bf16."""
    x_bits = np.atleast_2d(np.asarray(x_bits, dtype=np.uint16))
    x = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(np.asarray(gamma_bits, dtype=np.uint16))
    if g.shape != (x.shape[1],):
        raise ValueError("gamma has shape %s, K=%d" % (g.shape, x.shape[1]))
    r = rms_factor(x_bits, eps)
    return x * r[:, None] * g[None, :]


def rmsnorm_bf16(x_bits, gamma_bits, eps):
    """bf16 bits [B, K] of x~ = bf16_rne(x * r * gamma)."""
    return f64_to_bf16_bits(rmsnorm_f64(x_bits, gamma_bits, eps))
