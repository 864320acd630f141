/*
 * qgemv.h — C ABI of the MI355X block-quantized weight matvec library (libqgemv.so).
 *
 * The operation is the decode-step weight matvec
 *
 *     y[b, n] = sum_k  W^[n, k] * x[b, k]        b < batch, n < N, k < K
 *
 * where W is stored as packed low-bit codes plus per-group (or per-row) scales
 * and x is a bf16 activation vector or a small batch of them.  This is the
 * weight stream the "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus
 * (Part 2)" post identifies as the dominant bucket of a decode token (section
 * "The starting point", decomposition table: FP4 weight matvecs and the FP8
 * lm_head), and the "qmm GEMV" of the mlxcel issue "decode is bound by 8-bit
 * MLP weight bytes" (#683, "Summary").
 *
 * Conventions shared by every device entry point
 *  - Pointers marked DEVICE are device (HBM) pointers; HOST pointers are
 *    ordinary host memory.  Every matrix is dense row-major with K contiguous.
 *  - The caller allocates and owns every buffer.  The library never allocates,
 *    frees or synchronizes; work is enqueued on `stream` and runs
 *    asynchronously.  `stream` may be 0 (the null stream).
 *  - Arguments are validated completely before any HIP call.  On an error
 *    nothing is launched and y is not touched.  A launch that fails
 *    (hipLaunchKernel's own status) maps to QG_ERR_LAUNCH; the thread's
 *    last-error state is neither read nor cleared, so an error left by an
 *    earlier, unrelated HIP call is never reported as this call's.  No C++
 *    exception crosses the ABI.
 *  - Preconditions (else the listed error):
 *      n >= 1, k >= 1                                  QG_ERR_BAD_SHAPE
 *      k % group_size == 0, group_size in {32,64,128}  QG_ERR_BAD_GROUP_SIZE
 *      a code row is a whole number of 16-byte chunks:
 *        FP4 and u4: k % 32 == 0; u8 and FP8: k % 16 == 0   QG_ERR_BAD_SHAPE
 *      codes and x 16-byte aligned; scales/biases 2-byte;
 *        row_scale 4-byte; y 4-byte (f32) or 2-byte (bf16) QG_ERR_MISALIGNED
 *      1 <= batch <= 4                                 QG_ERR_BAD_BATCH
 *      out_dtype is QG_OUT_F32 or QG_OUT_BF16          QG_ERR_BAD_DTYPE
 *      n <= 2^31, k <= 2^30                            QG_ERR_BAD_SHAPE
 *      non-null pointers                               QG_ERR_NULL_POINTER
 *    There is no limit on k * batch beyond that: activations that do not fit
 *    the kernels' LDS staging are read from memory (through the caches) by
 *    the steps that use them.
 *  - Results: fp32 accumulation.  Within 1e-3 relative error of the exact
 *    product per element (elements whose exact value nearly cancels are judged
 *    against 2^-12 * sum|w x|).  Run-to-run deterministic (no atomics), and a
 *    batch row gives the same bits as a batch-1 call with that row.
 *  - bf16 output is the fp32 result rounded to nearest even.
 *  - Concurrent calls on different streams are safe; calls that write the
 *    same y race like any two kernels would.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 6

typedef enum qg_status {
    QG_OK = 0,
    QG_ERR_NULL_POINTER = 1,
    QG_ERR_BAD_SHAPE = 2,
    QG_ERR_BAD_GROUP_SIZE = 3,
    QG_ERR_MISALIGNED = 4,
    QG_ERR_BAD_BATCH = 5,
    QG_ERR_BAD_DTYPE = 6,
    QG_ERR_BAD_BITS = 7,
    QG_ERR_BAD_VALUE = 8,     /* a quantizer was given a non-finite weight,
                                 or a fused norm a negative / non-finite eps */
    QG_ERR_TOO_LARGE = 9,     /* beyond an LDS staging limit: the int8 route's
                                 activation blocks, the standalone norm's k */
    QG_ERR_DEVICE = 10,       /* no usable HIP device / attribute query failed */
    QG_ERR_LAUNCH = 11        /* the kernel launch itself failed              */
} qg_status;

typedef enum qg_out_dtype { QG_OUT_F32 = 0, QG_OUT_BF16 = 1 } qg_out_dtype;

/* Weight formats, used by the query functions. */
typedef enum qg_format {
    QG_FMT_FP4_E2M1 = 0,
    QG_FMT_AFFINE_U4 = 1,
    QG_FMT_AFFINE_U8 = 2,
    QG_FMT_FP8_E4M3 = 3,
    QG_FMT_Q4K = 4
} qg_format;

/* ------------------------------------------------------------------------
 * Device entry points
 * ---------------------------------------------------------------------- */

/*
 * FP4-E2M1 weights with one bf16 scale per group of `group_size` columns.
 * "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus (Part 2)",
 * section "The assumption that failed the profiler": E2M1 codes (sign in
 * code bit 3, every magnitude exact in BF16), a per-group scale folded out of
 * the per-weight math as one multiply-add per group.
 *
 *   codes   DEVICE uint8 [n, k/2]: two codes per byte, the code of the even
 *           column in the low nibble.
 *   scales  DEVICE bf16 bits [n, k/group_size].
 *   x       DEVICE bf16 bits [batch, k].
 *   y       DEVICE [batch, n] float (QG_OUT_F32) or bf16 bits (QG_OUT_BF16).
 *   W^[n,k] = scale[n, k/group_size] * E2M1(code[n,k]).
 */
qg_status qgemv_fp4_e2m1(const uint8_t *codes, const uint16_t *scales,
                         const uint16_t *x, void *y,
                         int64_t n, int64_t k, int32_t group_size, int32_t batch,
                         qg_out_dtype out_dtype, hipStream_t stream);

/*
 * Min-max affine 4-bit codes, one bf16 scale and one bf16 bias per group.
 * mlxcel issue #683, "Step 2 result": group-64 affine codes packed into u32
 * low-first, scales and biases rounded to bf16.
 *
 *   codes   DEVICE uint32 [n, k/8]: code j of a word in bits [4j, 4j+4).
 *   scales, biases  DEVICE bf16 bits [n, k/group_size].
 *   x, y    as for qgemv_fp4_e2m1.
 *   W^[n,k] = scale[n,g] * q[n,k] + bias[n,g],  g = k/group_size, computed as
 *   sum_g scale*sum(q*x) + bias*sum(x) (the bias folded via activation sums).
 */
qg_status qgemv_affine_u4(const uint32_t *codes, const uint16_t *scales,
                          const uint16_t *biases, const uint16_t *x, void *y,
                          int64_t n, int64_t k, int32_t group_size, int32_t batch,
                          qg_out_dtype out_dtype, hipStream_t stream);

/*
 * Min-max affine 8-bit codes (mlxcel issue #683, "Step 2 result" and "Why
 * gemma-4-12b is slow": the 8-bit group-64 MLP matrices that dominate the
 * decode bytes; same layout rules and bias fold as qgemv_affine_u4).
 *   codes   DEVICE uint32 [n, k/4]: code j of a word in bits [8j, 8j+8).
 */
qg_status qgemv_affine_u8(const uint32_t *codes, const uint16_t *scales,
                          const uint16_t *biases, const uint16_t *x, void *y,
                          int64_t n, int64_t k, int32_t group_size, int32_t batch,
                          qg_out_dtype out_dtype, hipStream_t stream);

/*
 * FP8-E4M3 (OCP "FN": max 448, S.1111.111 = NaN) weights with one fp32 scale
 * per row.  "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus
 * (Part 2)", section "The assumption that failed the profiler": the FP8
 * lm_head matvec does one multiply-add per weight byte with no separate
 * dequantization pass; the row scale is applied once to the row's sum.
 *
 *   codes      DEVICE uint8 [n, k].
 *   row_scale  DEVICE float [n].
 *   W^[n,k] = row_scale[n] * E4M3(code[n,k]); a NaN code gives a NaN row.
 *
 * With one or two activation rows the products are summed by the vector unit
 * (two-wide bf16 dots); with three or four, by the matrix cores in 4x4x4
 * blocks (4 weight rows x 4 batch rows per block), whose cost does not grow
 * with the batch.  The two orders of addition differ, so a row's bits from a
 * batch of 1 or 2 can differ from its bits in a batch of 3 or 4 (both within
 * the same bound of the exact sum); inside each group of batch sizes they
 * are identical.  The matrix-core path takes 4-row tiles: rows_per_tile of a
 * qg_plan is ignored there.
 */
qg_status qgemv_fp8_e4m3(const uint8_t *codes, const float *row_scale,
                         const uint16_t *x, void *y,
                         int64_t n, int64_t k, int32_t batch,
                         qg_out_dtype out_dtype, hipStream_t stream);

/*
 * Two-level super-block 4-bit weights ("Q4_K-style"), in the pre-unpacked
 * device layout that qg_repack_q4k writes.  The SharpInference issue
 * "perf(cuda): generalize Gemma 4 batched prefill + flash attn + decode
 * graphs to dense Q4_K models", section "Work Item C (C1) done": a
 * super-block of 256 weights decodes as d * sc * nibble - dmin * m with
 * per-32-weight factors sc and m; section "All work items complete": a
 * decode repack that pre-unpacks the scales lifted the matvec from 74% to
 * 89% of HBM bandwidth.  The pages print no bit layout; the one defined here
 * is described at qg_quantize_q4k.
 *
 *   codes  DEVICE uint32 [n, k/8]: code j of a word in bits [4j, 4j+4)
 *          (as qgemv_affine_u4), 16-byte aligned
 *   sub    DEVICE uint16 [n, k/32]: sc | m << 8 of each 32-weight sub-block
 *          (six-bit factors, one byte each), 2-byte aligned
 *   super  DEVICE uint32 [n, k/256]: fp16 d | fp16 dmin << 16 of each
 *          256-weight super-block, 4-byte aligned
 *   x, y   as for qgemv_fp4_e2m1
 *   W^[n,k] = d * sc[j] * q[n,k] - dmin * m[j],  j = k/32 (exact in fp32:
 *   d * sc has at most 17 significant bits), folded per sub-block as
 *   (d*sc) * sum(q*x) - (dmin*m) * sum(x).
 *   k % 256 == 0                                  else QG_ERR_BAD_SHAPE
 * Everything else (batch, output, errors, accuracy, determinism, plans) as
 * for qgemv_affine_u4.
 */
qg_status qgemv_q4k(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                    void *y, int64_t n, int64_t k, int32_t batch, qg_out_dtype out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Explicit launch shape.  The plain entry points pick a launch shape from the
 * matrix shape and the device's compute-unit count.  The *_plan variants take
 * the same arguments plus a qg_plan whose non-zero fields override that
 * choice (for tuning a deployment's own shapes); plan == NULL is the plain
 * call.  Results are bitwise the same for every plan: a row's terms are
 * added in an order fixed by the format and k alone (for FP8, also by
 * whether the batch is below 3), whichever wavefront, tile shape or grid
 * computes it.
 * ---------------------------------------------------------------------- */

typedef struct qg_plan {
    int32_t rows_per_tile;    /* rows one wavefront streams together: 1, 2 or 4 */
    int32_t waves_per_block;  /* wavefronts per workgroup: 1..8                 */
    int32_t blocks;           /* workgroups in the grid (persistent)            */
} qg_plan;

/* A plan field outside its range returns QG_ERR_BAD_SHAPE. */
qg_status qgemv_fp4_e2m1_plan(const uint8_t *codes, const uint16_t *scales,
                              const uint16_t *x, void *y,
                              int64_t n, int64_t k, int32_t group_size, int32_t batch,
                              qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);
qg_status qgemv_affine_u4_plan(const uint32_t *codes, const uint16_t *scales,
                               const uint16_t *biases, const uint16_t *x, void *y,
                               int64_t n, int64_t k, int32_t group_size, int32_t batch,
                               qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);
qg_status qgemv_affine_u8_plan(const uint32_t *codes, const uint16_t *scales,
                               const uint16_t *biases, const uint16_t *x, void *y,
                               int64_t n, int64_t k, int32_t group_size, int32_t batch,
                               qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);
qg_status qgemv_fp8_e4m3_plan(const uint8_t *codes, const float *row_scale,
                              const uint16_t *x, void *y,
                              int64_t n, int64_t k, int32_t batch,
                              qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);
qg_status qgemv_q4k_plan(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                         void *y, int64_t n, int64_t k, int32_t batch, qg_out_dtype out_dtype,
                         const qg_plan *plan, hipStream_t stream);

/* The launch shape the plain entry point would use on the current device
 * (needs a HIP device for its compute-unit count, else QG_ERR_DEVICE). */
qg_status qg_plan_query(qg_format format, int64_t n, int64_t k, int32_t batch, qg_plan *out);

/* ------------------------------------------------------------------------
 * Queries (host only, no device needed)
 * ---------------------------------------------------------------------- */

/* Static English description of a status; never NULL. */
const char *qg_status_string(qg_status status);

/* ------------------------------------------------------------------------
 * Fused RMSNorm variants: y = W . RMSNorm(x), in one launch.
 *
 * "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus (Part 2)",
 * section "Where it landed", ranks RMSNorm fusion into the decode step's matvecs
 * among the next levers (the norm takes hundreds of launches per token).  The
 * page does not print the norm; these calls take the standard one, row by row:
 *
 *     r[b]    = 1 / sqrt( (1/k) * sum_k x[b,k]^2 + eps )          (fp32)
 *     x~[b,k] = bf16_rne( (x[b,k] * r[b]) * gamma[k] )             (fp32 products)
 *
 * and compute the matvec of x~, exactly what the plain entry point returns
 * for an x~ computed by a separate norm (up to that norm's own rounding of
 * r[b]).  Models that scale by (1 + gamma) pass that vector as gamma.
 *
 *   gamma  bf16 [k] (DEVICE), 16-byte aligned     else QG_ERR_NULL_POINTER /
 *                                                  QG_ERR_MISALIGNED
 *   eps    >= 0 and finite                        else QG_ERR_BAD_VALUE
 *   plan   as in the *_plan variants (NULL: the default launch)
 *
 * Everything else (arguments, layouts, errors, accuracy, determinism, batch
 * consistency) is as in the plain calls.  r[b] is summed in an order fixed by
 * k, so the result is also bitwise the same for every plan and batch size.
 * x itself is not modified.  One exception to "exactly what the plain entry
 * point returns": where x and gamma do not fit in 128 KiB of LDS together
 * ((batch + 1) * k * 2 bytes for the 8-bit codes, and for FP8 at batch 1-2;
 * (1.25 * batch + 1) * k * 2 for the 4-bit formats at batch 1-2, whose x is
 * kept padded; e.g. the 8-bit codes at batch 4 and k = 15360), the call runs a
 * kernel that stages x per step and adds the terms in another order; it
 * meets the same accuracy bound but is not bitwise the plain call's, nor
 * the fused call's at a batch size that fits.
 * ---------------------------------------------------------------------- */

qg_status qgemv_fp4_e2m1_rmsnorm(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                                 const uint16_t *gamma, float eps, void *y, int64_t n, int64_t k,
                                 int32_t group_size, int32_t batch, qg_out_dtype out_dtype,
                                 const qg_plan *plan, hipStream_t stream);
qg_status qgemv_affine_u4_rmsnorm(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                  const uint16_t *x, const uint16_t *gamma, float eps, void *y,
                                  int64_t n, int64_t k, int32_t group_size, int32_t batch,
                                  qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);
qg_status qgemv_affine_u8_rmsnorm(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                  const uint16_t *x, const uint16_t *gamma, float eps, void *y,
                                  int64_t n, int64_t k, int32_t group_size, int32_t batch,
                                  qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);
qg_status qgemv_fp8_e4m3_rmsnorm(const uint8_t *codes, const float *row_scale, const uint16_t *x,
                                 const uint16_t *gamma, float eps, void *y, int64_t n, int64_t k,
                                 int32_t batch, qg_out_dtype out_dtype, const qg_plan *plan,
                                 hipStream_t stream);
qg_status qgemv_q4k_rmsnorm(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                            const uint16_t *gamma, float eps, void *y, int64_t n, int64_t k, int32_t batch,
                            qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream);

/* The fused variants' RMSNorm on its own ("Hand-Writing Gemma 4
 * Flash-Decoding + an FP4 Matvec Bonus (Part 2)", section "The starting
 * point": RMSNorm as a decode-step bucket of its own; "Where it landed": its
 * fusion as the next lever): out[b, k] = x~[b, k] as defined
 * above, with r[b] summed exactly as the fused matvec sums it, so the plain
 * entry point fed `out` returns bitwise what the fused variant returns.  For
 * consumers that need the normalized activations themselves.
 *   x, out   bf16 [batch, k] (DEVICE), gamma bf16 [k] (DEVICE), all 16-byte
 *            aligned; 8 <= k, k % 8 == 0; 1 <= batch <= 4; eps as above.
 *   out may be x (normalized in place); otherwise the two must not overlap.
 *   k above 2^23 returns QG_ERR_TOO_LARGE (the group sums of a row must fit
 *   in 64 KiB of LDS).
 * One workgroup per batch row, asynchronous on `stream`. */
qg_status qg_rmsnorm_bf16(const uint16_t *x, const uint16_t *gamma, float eps, uint16_t *out, int64_t k,
                          int32_t batch, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Small-batch GEMM: more than four activation rows.
 *
 * Y[m, n] = X[m, k] . W[n, k]^T for a short prefill or a speculative-decoding
 * batch, W in the FP4-E2M1 layout of qgemv_fp4_e2m1 (codes [n, k/2], bf16
 * group scales [n, k/group_size]), read from HBM once per 64 activation rows.
 * The SharpInference issue ("generalize Gemma 4 batched prefill ..."), items
 * C1 and C2, weighs a dequantized fp16 weight copy fed to a GEMM against a
 * kernel that reads the 4-bit weights once; this is the second kind: the
 * codes are decoded in registers and meet the activations in bf16 MFMA, and
 * each group's sum is scaled once, y += s * sum_{k in group} e2m1 * x, in
 * fp32.  The summation order depends on k and the group size only, so the
 * results are bitwise the same from run to run and for every m (row i of Y
 * does not depend on the other rows of X); they are not bitwise those of the
 * matvec (another order), and meet the same 1e-3 bar against the exact sum.
 *   codes     uint8 [n, k/2] (DEVICE), 16-byte aligned
 *   scales    bf16 [n, k/group_size] (DEVICE), 2-byte aligned
 *   x         bf16 [m, k] (DEVICE), 16-byte aligned
 *   y         [m, n] f32 or bf16 (DEVICE), 4- or 2-byte aligned
 *   n >= 1, 32 <= k <= 2^30, k % 32 == 0          QG_ERR_BAD_SHAPE
 *   group_size in {32, 64, 128}, k % group_size == 0   QG_ERR_BAD_GROUP_SIZE
 *   1 <= m <= QG_GEMM_MAX_M                       QG_ERR_BAD_BATCH
 * Up to 16 activation rows whose x fits in LDS (m * k * 2 bytes, k rounded
 * up to 256, at most 128 KiB) stage x once per workgroup and stream the
 * weight tiles without barriers; more rows take a kernel that stages x chunk
 * by chunk.  Both add a row's terms in the same order.
 * No device memory is allocated; asynchronous on `stream`.  For m <= 4 the
 * matvec entry points are the faster path. */
#define QG_GEMM_MAX_M 65536
qg_status qgemm_fp4_e2m1(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, void *y, int64_t n,
                         int64_t k, int32_t group_size, int32_t m, qg_out_dtype out_dtype, hipStream_t stream);

/* The same GEMM for min-max affine 4-bit weights in the layout of
 * qgemv_affine_u4 (codes uint32 [n, k/8] low-first, bf16 scales and biases
 * [n, k/group_size]).  The SharpInference issue ("generalize Gemma 4 batched
 * prefill ..."), "Item C2", runs its short-prompt GEMM on a 4-bit format with
 * a per-sub-block minimum, folded through the activations' sums; here the
 * codes meet bf16 activations in bf16 MFMA and each group folds as
 * y += s * sum_{k in group} q * x + b * sum_{k in group} x, in fp32 (the
 * decode and the activation-sum fold of the affine matvec).  The summation
 * order depends on k and the group size only: bitwise the same for every m
 * (row i of Y does not depend on the other rows of X), not bitwise the
 * matvec's, and within the same 1e-3 bar against the exact sum.
 *   codes     uint32 [n, k/8] (DEVICE), 16-byte aligned
 *   scales, biases  bf16 [n, k/group_size] (DEVICE), 2-byte aligned
 *   x, y, n, k, group_size, m: as for qgemm_fp4_e2m1, with the same errors
 *   (a null biases pointer: QG_ERR_NULL_POINTER)
 * As for qgemm_fp4_e2m1, up to 16 rows whose x fits in LDS take the kernel
 * that stages x once and streams the weight tiles, more rows the one that
 * stages x chunk by chunk, with the same order of additions.  No device
 * memory is allocated; asynchronous on `stream`. */
qg_status qgemm_affine_u4(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                          void *y, int64_t n, int64_t k, int32_t group_size, int32_t m, qg_out_dtype out_dtype,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Int8 activation route for affine 4-bit and 8-bit weights.
 *
 * The SharpInference issue ("generalize Gemma 4 batched prefill ..."),
 * "Item C2", quantizes the activation to int8 q8_1 blocks whose 32-bit ds
 * word carries an fp16 pair: d in the low half and, in the high half, the
 * block's activation sum s = d * sum(q); it widens the 4-bit weights to int8
 * and applies the affine minimum once per block through s.  The pages do not
 * print the quantizer; this library reads it as the symmetric one below,
 * with the codes chosen against the d the block stores.  The route changes
 * the result by at most sum_k |W^[n,k]| * d_blk / 2 against the bf16
 * product (each activation moves by at most half a step), plus the fp16
 * rounding of s times the bias.
 *
 * qg_quantize_q8_1: per batch row, per block of 32 consecutive activations,
 *   amax = max |x|,  d = fp16_rne(amax / 127),
 *   q = clamp(rne(x / d), -127, 127)  (q = 0 when d is 0: an all-zero block,
 *   or amax / 127 below half the smallest fp16 subnormal),
 *   s = fp16_rne(d * sum q).
 *   The decisions are those of exact arithmetic (correctly rounded fp32
 *   quotients, which never reach an fp16 or integer midpoint they are not
 *   on), so the codes and pairs are exact functions of x.  x must be finite;
 *   block maxima of 65520 * 127 or more make d infinite (unspecified result).
 *   x    bf16 [batch, k] (DEVICE), 16-byte aligned
 *   xq   int8 [batch, k] (DEVICE, caller-owned output), 16-byte aligned,
 *        natural column order
 *   ds   fp16 bits [batch, k/32, 2] = {d, s} (DEVICE, caller-owned output),
 *        4-byte aligned: one little-endian 32-bit word per block, d low
 *   k >= 32, k % 32 == 0                          QG_ERR_BAD_SHAPE
 *   1 <= batch <= 4                               QG_ERR_BAD_BATCH
 *
 * qgemv_affine_u4_q8: y[b, r] = sum over blocks of
 *   scale[r,g] * d[b,blk] * sum_{k in blk} u[r,k] * q[b,k]  +  bias[r,g] * s[b,blk]
 *   with the integer block dots exact (4-wide int8 dots) and the rest in
 *   fp32; one block is one 16-byte chunk of codes.  Codes, scales and biases
 *   are those of qgemv_affine_u4 (u32 low-first nibbles, bf16 [n, k/gs]).
 *   xq, ds  as written by qg_quantize_q8_1 (DEVICE)
 *   y       [batch, n] f32 or bf16 (DEVICE), 4- or 2-byte aligned
 *   group_size in {32, 64, 128}, k % group_size == 0   QG_ERR_BAD_GROUP_SIZE
 *   the activation codes and pairs are staged in LDS: batch * k * 1.125
 *   bytes must be at most 128 KiB                 QG_ERR_TOO_LARGE
 *   other checks and errors as for qgemv_affine_u4.
 * qgemv_affine_u4_q8_fused: the same product with the quantization of x
 *   done inside the matvec (each workgroup quantizes x as it stages it, with
 *   the arithmetic of qg_quantize_q8_1), so one launch replaces two and no
 *   int8 copy of x goes to memory.  Returns bitwise what qg_quantize_q8_1
 *   followed by qgemv_affine_u4_q8 returns.
 *   x       bf16 [batch, k] (DEVICE), 16-byte aligned, finite
 *   other arguments, checks and errors as for qgemv_affine_u4_q8.
 * qgemv_affine_u8_q8, qgemv_affine_u8_q8_fused: the same for the 8-bit
 *   codes of qgemv_affine_u8 (codes uint32 [n, k/4], code j of a word in
 *   bits [8j, 8j+8)).  One block is two 16-byte chunks of codes; a code c
 *   enters the 4-wide dot as the signed byte c - 128 (its top bit flipped)
 *   and 128 times the chunk's activation-code sum is added back to the
 *   integer dot, so that y[b, r] = sum over blocks of scale*d*sum(c*q) +
 *   bias*s exactly as for u4.
 * None of these calls allocates device memory; all are asynchronous on
 * `stream`. */
qg_status qg_quantize_q8_1(const uint16_t *x, int64_t k, int32_t batch, int8_t *xq, uint16_t *ds,
                           hipStream_t stream);
qg_status qgemv_affine_u4_q8(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                             const int8_t *xq, const uint16_t *ds, void *y, int64_t n, int64_t k,
                             int32_t group_size, int32_t batch, qg_out_dtype out_dtype, hipStream_t stream);
qg_status qgemv_affine_u4_q8_fused(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                   const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                                   int32_t batch, qg_out_dtype out_dtype, hipStream_t stream);
qg_status qgemv_affine_u8_q8(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                             const int8_t *xq, const uint16_t *ds, void *y, int64_t n, int64_t k,
                             int32_t group_size, int32_t batch, qg_out_dtype out_dtype, hipStream_t stream);
qg_status qgemv_affine_u8_q8_fused(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                   const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                                   int32_t batch, qg_out_dtype out_dtype, hipStream_t stream);

/* QG_ABI_VERSION of the loaded library. */
int qg_abi_version(void);


/* ------------------------------------------------------------------------
 * Measurement
 * ---------------------------------------------------------------------- */

/*
 * Stream probe: reads `bytes` bytes of `buf` with 16-byte coalesced loads per
 * lane (`unroll` in {1,2,4,8,16} loads in flight per lane) and writes one xor
 * of what each thread read to out[blocks * threads_per_block] (DEVICE).  It is
 * the reference for the achievable HBM read bandwidth that the matvec is
 * compared with: "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus
 * (Part 2)", section "What we'd tell the next person", proves a streaming
 * kernel's ceiling with a same-run reference kernel.
 *   pattern 0: grid-stride rounds; 1: each wavefront streams its own
 *   contiguous range; 2: as 1 with each lane reading two adjacent 16-byte
 *   units (unroll >= 2); 3, 4, 5: patterns 0, 1, 2 with non-temporal loads.
 * bytes must be a positive multiple of 16; buf 16-byte aligned.
 */
qg_status qg_stream_probe(const void *buf, int64_t bytes, int32_t pattern, int32_t unroll,
                          int32_t blocks, int32_t threads_per_block, uint32_t *out,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Host pack/layout module.  HOST pointers; the caller allocates every output.
 * These produce the packed layouts the device entry points read.  The
 * arithmetic is float64 with one rounding per operation (see the quantizer
 * definitions below); the functions are deterministic and thread-safe.
 * Every function returns QG_ERR_NULL_POINTER / QG_ERR_BAD_SHAPE /
 * QG_ERR_BAD_GROUP_SIZE / QG_ERR_BAD_BITS / QG_ERR_BAD_VALUE as applicable and
 * writes nothing on error.
 * ---------------------------------------------------------------------- */

/*
 * FP4-E2M1 group-absmax quantizer ("Hand-Writing Gemma 4 Flash-Decoding + an
 * FP4 Matvec Bonus (Part 2)", section "The assumption that failed the
 * profiler": E2M1 codes with the sign in bit 3 and per-group scales; section
 * "Where it landed": per-group scaling).  Per group: s = bf16_rne(absmax / 6);
 * code = nearest E2M1 value to w / s, ties to the even mantissa bit,
 * saturating at 6; sign bit set iff w < 0; s == 0 gives code 0.
 *   w       HOST float [n, k] (finite)
 *   codes   HOST uint8 [n, k/2] (low nibble = even column)
 *   scales  HOST bf16 bits [n, k/group_size]
 */
qg_status qg_quantize_fp4_e2m1(const float *w, int64_t n, int64_t k, int32_t group_size,
                               uint8_t *codes, uint16_t *scales);

/*
 * Min-max affine quantizer (mlxcel issue #683, "Step 2 result": scale and
 * bias rounded to bf16 before q is computed, self-consistent triples).  Per group: s = bf16_rne((max - min) / (2^bits-1)),
 * b = bf16_rne(min), q = clamp(rint((w - b) / s), 0, 2^bits - 1) with rint
 * rounding half to even; s == 0 gives q = 0.
 *   codes   HOST uint32 [n, k*bits/32], u32 low-first
 *   scales, biases  HOST bf16 bits [n, k/group_size]
 */
qg_status qg_quantize_affine(const float *w, int64_t n, int64_t k, int32_t bits,
                             int32_t group_size, uint32_t *codes, uint16_t *scales,
                             uint16_t *biases);

/*
 * FP8-E4M3 row-absmax quantizer ("Hand-Writing Gemma 4 Flash-Decoding + an
 * FP4 Matvec Bonus (Part 2)", section "The starting point": the FP8 lm_head
 * matvec, one multiply-add per weight byte, its scale applied once per row).
 * s_n = absmax_n / 448 (one binary32
 * division); code = nearest finite E4M3 to w / s_n (float64 quotient), ties to
 * even, saturating at 448; sign bit set iff w < 0; s_n == 0 gives code 0.
 *   codes      HOST uint8 [n, k];  row_scale  HOST float [n]
 */
qg_status qg_quantize_fp8_e4m3_rowwise(const float *w, int64_t n, int64_t k,
                                       uint8_t *codes, float *row_scale);

/* One code per byte (values < 16) <-> two per byte, even index in the low nibble
 * (the low-first order the mlxcel issue #683, "Step 2 result", states for
 * u32 words, applied to the two codes of a byte).  count must be even. */
qg_status qg_pack_nibbles(const uint8_t *one_code_per_byte, int64_t count, uint8_t *packed);
qg_status qg_unpack_nibbles(const uint8_t *packed, int64_t count, uint8_t *one_code_per_byte);

/* One code per byte (values < 2^bits) <-> u32 low-first words (mlxcel issue
 * #683, "Step 2 result": affine codes packed into u32 words low-first); bits 4
 * or 8; count a multiple of 32/bits. */
qg_status qg_pack_u32(const uint8_t *one_code_per_byte, int64_t count, int32_t bits,
                      uint32_t *packed);
qg_status qg_unpack_u32(const uint32_t *packed, int64_t count, int32_t bits,
                        uint8_t *one_code_per_byte);

/* Bytes of one packed weight matrix (codes + scales [+ biases]), or -1 for
 * invalid arguments (mlxcel issue #683, "Step 2 result" and "Why gemma-4-12b
 * is slow": checkpoint bytes at 8.5 and 4.5 bits per weight, which these
 * reproduce for the 144 MLP matrices).  These are also the weight part of the
 * algorithmic bytes a matvec must move. */
int64_t qg_bytes_fp4(int64_t n, int64_t k, int32_t group_size);
int64_t qg_bytes_affine(int64_t n, int64_t k, int32_t bits, int32_t group_size);
int64_t qg_bytes_fp8(int64_t n, int64_t k);

/*
 * Two-level super-block 4-bit quantizer ("perf(cuda): generalize Gemma 4
 * batched prefill + flash attn + decode graphs to dense Q4_K models",
 * sections "Work Item C (C1) done": the d*sc*nibble - dmin*mn decode of a
 * 256-element super-block; "Item C2": 32-element sub-blocks with their own
 * scale and min).  The pages print neither the packed layout nor the
 * quantizer; this library defines them.  Storage record, 144 bytes per
 * super-block of 256 consecutive weights of a row:
 *   bytes 0-1 d, 2-3 dmin (fp16, little-endian); bytes 4-9 the eight six-bit
 *   sub-block scale factors sc[0..7], sc[j] in bits 6j..6j+5 of the 48-bit
 *   little-endian field; bytes 10-15 the eight min factors m[j], the same
 *   way; bytes 16-143 the 256 codes, two per byte, the even weight in the
 *   low nibble.  W^ = d*sc[j]*q - dmin*m[j].
 * Quantization (IEEE double, one rounding per operation): per sub-block
 * lo = min(min w, 0), s = (max w - lo)/15 + 0, off = 0 - lo; d =
 * fp16_rne(max s / 63), dmin = fp16_rne(max off / 63); sc = clamp(rne(s/d),
 * 0, 63), m = clamp(rne(off/dmin), 0, 63) (0 when the fp16 value is 0); q =
 * clamp(rne((w + dmin*m)/(d*sc)), 0, 15) (0 when d*sc is 0).
 *   w        HOST float [n, k] (finite), k % 256 == 0
 *   records  HOST uint8 [n, k/256, 144]
 */
qg_status qg_quantize_q4k(const float *w, int64_t n, int64_t k, uint8_t *records);

/*
 * The decode repack of the SharpInference issue "perf(cuda): generalize
 * Gemma 4 batched prefill + flash attn + decode graphs to dense Q4_K
 * models" ("All work items complete": scales pre-unpacked into their own
 * array): storage records -> the device layout
 * of qgemv_q4k (codes uint32 [n, k/8], sub uint16 [n, k/32] = sc | m << 8,
 * super uint32 [n, k/256] = d | dmin << 16).  All HOST pointers.
 */
qg_status qg_repack_q4k(const uint8_t *records, int64_t n, int64_t k, uint32_t *codes, uint16_t *sub,
                        uint32_t *super);

/* Bytes of the super-block format ("generalize Gemma 4 batched prefill ...
 * dense Q4_K models", "All work items complete"):
 * the storage records (4.5 bits per weight) and the device layout the matvec
 * reads (4.625 bits per weight); -1 for invalid arguments. */
int64_t qg_bytes_q4k_records(int64_t n, int64_t k);
int64_t qg_bytes_q4k(int64_t n, int64_t k);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
