"""Number formats used by the quantized matvec, written from their definitions.

Test infrastructure (see ``oracle/__init__``): no product code may import this.

* bf16: the upper 16 bits of an IEEE binary32 (8 significant bits, exponent
  bias 127).  Activations x, FP4 group scales and affine scales/biases are bf16
  ("The test that catches what parity misses": the reference runs over the
  same bf16-rounded inputs; #683 "Step 2 result": bf16 scales and biases).
* E2M1 (FP4): sign in bit 3 of the 4-bit code, two exponent bits (bias 1) and
  one mantissa bit; exponent field 0 is subnormal.  Part 2 post, "The
  assumption that failed the profiler": the sign bit is bit 3 and all eight
  magnitudes are exact in BF16.
* E4M3 (FP8, OCP "FN" variant): sign bit 7, four exponent bits (bias 7), three
  mantissa bits, exponent field 0 subnormal, S.1111.111 is NaN, no infinities,
  largest finite 448.  The page names only "FP8" for the lm_head matvec;
  this module reads it as OCP E4M3 (FN), the usual weight format of that
  name.

All decoders return float64 and are exact (every value of these formats is a
float64).  Encoders round to nearest, ties to even, using exact float64
arithmetic (frexp/ldexp/rint), never a cast chain.
"""

import numpy as np

# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------

BF16_QNAN = np.uint16(0x7FC0)


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):       # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v):
    """Round float64 values to the nearest bf16 (ties to even); return bits.

    Normal bf16 numbers have 8 significant bits, so a value in
    [2**(e-1), 2**e) is rounded to a multiple of 2**(e-8); below the smallest
    normal 2**-126 the spacing is the subnormal step 2**-133.  Results of
    magnitude >= 2**128 become infinity; NaN becomes the quiet NaN 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    _, e = np.frexp(a_f)                      # a = m * 2**e, m in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)           # spacing of bf16 around a
    r = np.rint(np.ldexp(a_f, -q_exp))        # numpy rint: half to even
    val = np.ldexp(r, q_exp)                  # exactly representable in bf16
    overflow = val >= 2.0 ** 128
    val32 = np.where(overflow, 0.0, val).astype(np.float32)
    bits = (val32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(overflow | np.isinf(v), np.uint16(0x7F80), bits)
    bits = np.where(np.signbit(v), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(v), BF16_QNAN, bits)
    return bits.astype(np.uint16)


# ---------------------------------------------------------------------------
# E2M1 (FP4)
# ---------------------------------------------------------------------------

def e2m1_value(code):
    """Value of one 4-bit E2M1 code, from the bit fields."""
    code = int(code)
    if not 0 <= code < 16:
        raise ValueError("E2M1 code out of range: %r" % code)
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:                               # subnormal: 0 or 0.5
        mag = 0.5 * man
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return -mag if sign else mag


#: value of every code 0..15 (codes 8..15 are the negatives of 0..7)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_rne_codes(r):
    """Nearest E2M1 code to each real r, ties to the even mantissa bit.

    |r| above 6 saturates to 6.  The sign bit is set iff r < 0 (so a small
    negative value that rounds to magnitude 0 gives code 8, "-0").
    """
    r = np.asarray(r, dtype=np.float64)
    mags = E2M1_TABLE[:8]                      # ascending: codes 0..7
    a = np.minimum(np.abs(r), mags[-1])
    d = np.abs(a[..., None] - mags)            # distance to every magnitude
    tied = d == d.min(axis=-1, keepdims=True)
    # among the nearest magnitudes take the even code (mantissa bit 0)
    score = np.where(tied, np.arange(8) % 2, 2)
    idx = score.argmin(axis=-1)
    return (idx + np.where(r < 0, 8, 0)).astype(np.uint8)


# ---------------------------------------------------------------------------
# E4M3 (FP8, OCP FN)
# ---------------------------------------------------------------------------

def e4m3_value(code):
    """Value of one 8-bit E4M3 code (OCP FN: no inf, S.1111.111 = NaN)."""
    code = int(code)
    if not 0 <= code < 256:
        raise ValueError("E4M3 code out of range: %r" % code)
    sign = (code >> 7) & 1
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return -mag if sign else mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_rne_codes(r):
    """Nearest finite E4M3 code to each real r, ties to even; saturating.

    |r| is clamped to 448 before rounding, so the NaN code is never produced.
    The sign bit is set iff r < 0.
    """
    r = np.asarray(r, dtype=np.float64)
    mags = E4M3_TABLE[:127]                    # codes 0..126, ascending
    a = np.minimum(np.abs(r), E4M3_MAX)
    hi = np.searchsorted(mags, a, side="left")      # first mags[hi] >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a == mags[hi], hi, idx)
    return (idx + np.where(r < 0, 128, 0)).astype(np.uint8)
