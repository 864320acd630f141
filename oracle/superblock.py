"""Two-level super-block 4-bit format ("Q4_K-style").  Test infrastructure.

Source: "perf(cuda): generalize Gemma 4 batched prefill + flash attn + decode
graphs to dense Q4_K models", sections "Work Item C (C1) done" (a Q4_K
super-block decodes as d * sc * nibble - dmin * mn), "Item C2 - int8 MMQ Q4_K
prefill" (a 256-element super-block of 32-element sub-blocks, each with its
own scale and min, unpacked from the super-block's packed scale bytes) and
"All work items complete" (a decode repack that pre-unpacks the scales into a
separate array raised the matvec from 74% to 89% of HBM bandwidth).

The pages give the decode formula and the two levels but print neither the
bit layout of the packed scales nor the quantizer.  This module fixes both
with the plainest reading; it does not follow any other library's layout.

Storage layout (what the quantizer writes), one 144-byte record per
super-block of 256 consecutive weights of a row:

  bytes 0-1    d     fp16, little-endian (scale of the sub-block scales)
  bytes 2-3    dmin  fp16 (scale of the sub-block mins)
  bytes 4-9    sc[0..7]  six-bit unsigned, packed low-first: sc[j] in bits
               6j .. 6j+5 of the 48-bit little-endian field
  bytes 10-15  m[0..7]   six-bit unsigned, packed the same way
  bytes 16-143 the 256 four-bit codes, two per byte, the even weight in the
               low nibble

  weight i of sub-block j:  W^ = d * sc[j] * q - dmin * m[j]   (exact real)

Quantizer (float64, one rounding per operation):

  per sub-block j:  lo = min(min_i w, 0),  s_j = (max_i w - lo) / 15,
                    off_j = 0 - lo   (the min term is subtracted, so >= 0;
                    +0, not -0, when lo = 0)
  per super-block:  d = fp16_rne(max_j s_j / 63),
                    dmin = fp16_rne(max_j off_j / 63)
                    sc[j] = clamp(rne(s_j / d), 0, 63)     (0 when d = 0)
                    m[j] = clamp(rne(off_j / dmin), 0, 63)  (0 when dmin = 0)
  per weight:       q = clamp(rne((w + dmin*m[j]) / (d*sc[j])), 0, 15)
                    (0 when d*sc[j] = 0)

Both scales are rounded to fp16 before the six-bit factors are chosen, and
the codes are chosen against the stored products d*sc[j] and dmin*m[j] (the
self-consistency reading the affine quantizer also takes).

Device layout (the "pre-unpacked" repack the library's kernel reads):

  codes  uint32 [n, k/8], code i of a word in bits 4i .. 4i+3 (low-first):
         the storage layout's code bytes, contiguous per row
  sub    uint16 [n, k/32]: sc[j] | m[j] << 8 for sub-block j of the row
  super  uint32 [n, k/256]: d bits | dmin bits << 16
"""

import numpy as np

from .formats import bf16_bits_to_f64

SUPER = 256
SUB = 32
NSUB = SUPER // SUB
QMAX = 15
SMAX = 63
RECORD = 144


def _f16_bits(v):
    """float64 -> fp16 bits, round to nearest even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _f16_value(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def quantize_q4k(w):
    """float32 [n, k] -> storage records uint8 [n, k/256, 144] (k % 256 == 0)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % SUPER:
        raise ValueError("K=%d is not a multiple of %d" % (k, SUPER))
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    nsb = k // SUPER
    wb = w.astype(np.float64).reshape(n, nsb, NSUB, SUB)
    lo = np.minimum(wb.min(axis=3), 0.0)
    s = (wb.max(axis=3) - lo) / QMAX                                 # [n, nsb, 8]
    off = 0.0 - lo                                                     # +0 (not -0) for lo = 0
    d_bits = _f16_bits(s.max(axis=2) / SMAX)                          # [n, nsb]
    dmin_bits = _f16_bits(off.max(axis=2) / SMAX)
    d = _f16_value(d_bits)[:, :, None]
    dmin = _f16_value(dmin_bits)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > 0, np.clip(np.rint(s / np.where(d > 0, d, 1.0)), 0, SMAX), 0).astype(np.int64)
        m = np.where(dmin > 0, np.clip(np.rint(off / np.where(dmin > 0, dmin, 1.0)), 0, SMAX), 0).astype(np.int64)
    S = (d * sc)[:, :, :, None]                                        # exact in float64
    M = (dmin * m)[:, :, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(S > 0, np.clip(np.rint((wb + M) / np.where(S > 0, S, 1.0)), 0, QMAX), 0).astype(np.int64)
    return pack_records(d_bits, dmin_bits, sc, m, q.reshape(n, nsb, SUPER))


def pack_records(d_bits, dmin_bits, sc, m, q):
    """Fields -> storage records: d, dmin fp16 bits [n, nsb]; sc, m [n, nsb, 8]
    in 0..63; q [n, nsb, 256] in 0..15."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    n, nsb = d_bits.shape
    rec = np.zeros((n, nsb, RECORD), dtype=np.uint8)
    rec[:, :, 0] = d_bits & 0xFF
    rec[:, :, 1] = d_bits >> 8
    dmin_bits = np.asarray(dmin_bits, dtype=np.uint16)
    rec[:, :, 2] = dmin_bits & 0xFF
    rec[:, :, 3] = dmin_bits >> 8
    for base, f in ((4, np.asarray(sc, dtype=np.uint64)), (10, np.asarray(m, dtype=np.uint64))):
        field = np.zeros((n, nsb), dtype=np.uint64)
        for j in range(NSUB):
            field |= f[:, :, j] << np.uint64(6 * j)
        for b in range(6):
            rec[:, :, base + b] = ((field >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
    q = np.asarray(q, dtype=np.uint8)
    rec[:, :, 16:] = q[:, :, 0::2] | (q[:, :, 1::2] << 4)
    return rec


def unpack_records(rec):
    """Storage records -> (d fp16 bits [n, nsb], dmin bits, sc [n, nsb, 8],
    m [n, nsb, 8], q [n, nsb, 256])."""
    rec = np.asarray(rec, dtype=np.uint8)
    d_bits = rec[:, :, 0].astype(np.uint16) | (rec[:, :, 1].astype(np.uint16) << 8)
    dmin_bits = rec[:, :, 2].astype(np.uint16) | (rec[:, :, 3].astype(np.uint16) << 8)
    fields = []
    for base in (4, 10):
        field = np.zeros(rec.shape[:2], dtype=np.uint64)
        for b in range(6):
            field |= rec[:, :, base + b].astype(np.uint64) << np.uint64(8 * b)
        fields.append(np.stack([(field >> np.uint64(6 * j)) & np.uint64(SMAX) for j in range(NSUB)],
                               axis=2).astype(np.int64))
    codes = rec[:, :, 16:]
    q = np.empty(rec.shape[:2] + (SUPER,), dtype=np.int64)
    q[:, :, 0::2] = codes & 0x0F
    q[:, :, 1::2] = codes >> 4
    return d_bits, dmin_bits, fields[0], fields[1], q


def dequant_q4k(rec):
    """Storage records [n, k/256, 144] -> the exact weights float64 [n, k]."""
    d_bits, dmin_bits, sc, m, q = unpack_records(rec)
    n, nsb = d_bits.shape
    d = _f16_value(d_bits)[:, :, None, None]
    dmin = _f16_value(dmin_bits)[:, :, None, None]
    w = d * sc[:, :, :, None] * q.reshape(n, nsb, NSUB, SUB) - dmin * m[:, :, :, None]
    return w.reshape(n, nsb * SUPER)


def gemv_q4k(rec, x_bits, block_rows=4096):
    """y[b, r] = sum_k W^[r, k] x[b, k] and A = sum_k |W^ x| in float64."""
    rec = np.asarray(rec, dtype=np.uint8)
    x = np.atleast_2d(bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)))
    n = rec.shape[0]
    k = rec.shape[1] * SUPER
    if x.shape[1] != k:
        raise ValueError("x has K=%d, the records K=%d" % (x.shape[1], k))
    y = np.zeros((x.shape[0], n))
    a = np.zeros((x.shape[0], n))
    for r0 in range(0, n, block_rows):
        w = dequant_q4k(rec[r0:r0 + block_rows])
        y[:, r0:r0 + w.shape[0]] = x @ w.T
        a[:, r0:r0 + w.shape[0]] = np.abs(x) @ np.abs(w).T
    return y, a


def repack_q4k(rec):
    """Storage records -> the device layout (codes uint32 [n, k/8], sub uint16
    [n, k/32], super uint32 [n, k/256])."""
    d_bits, dmin_bits, sc, m, q = unpack_records(rec)
    n, nsb = d_bits.shape
    k = nsb * SUPER
    qq = q.reshape(n, k // 8, 8).astype(np.uint32)
    codes = np.zeros((n, k // 8), dtype=np.uint32)
    for i in range(8):
        codes |= qq[:, :, i] << np.uint32(4 * i)
    sub = (sc.astype(np.uint16) | (m.astype(np.uint16) << 8)).reshape(n, nsb * NSUB)
    sup = d_bits.astype(np.uint32) | (dmin_bits.astype(np.uint32) << 16)
    return codes, sub, sup


def bytes_storage(n, k):
    """Bytes of the storage records (4.5 bits per weight)."""
    return n * (k // SUPER) * RECORD


def bytes_device(n, k):
    """Bytes of the device layout: codes, sub-block pairs, super-block pairs."""
    return n * k // 2 + n * (k // SUB) * 2 + n * (k // SUPER) * 4
