// C ABI of the small-batch GEMM (more than four activation rows): argument
// validation and the launch.  As for the matvec, every argument is checked
// before any HIP call, so a bad argument launches nothing and leaves y alone.

#include "qgemv.h"
#include "qgemm_kernels.hpp"
#include "qgemv_device.hpp"

#include <mutex>

namespace {

using qgl::aligned_to;

// compute units of the current device (cached per device), 0 if unknown
int device_cus() { return qgl::device_cu_count(); }

// K slices per workgroup, from n and k only (a row's bits must not depend
// on m): more slices when there are few 64-row tiles to spread over the
// chip, never more than there are 256-wide chunks
int gemm_k_slices(int64_t n, int64_t k) {
    const int64_t tiles = (n + qg::kGemmRows - 1) / qg::kGemmRows;
    const int64_t chunks = (k + qg::kGemmKC - 1) / qg::kGemmKC;
    int ks = tiles <= 64 ? 4 : (tiles <= 160 ? 2 : 1);
    while (ks > 1 && ks > chunks) ks /= 2;
    return ks;
}

// The general kernel (x staged chunk by chunk): blocks of 16 activation rows
// per workgroup as many as m needs, up to 4 / ks (LDS holds ks chunks of
// them); one wave per K slice and 16 rows per workgroup where the grid of
// 64-row workgroups would leave half the compute units idle (one block of
// 16 activation rows: 4x the workgroups, each staging its own activations),
// four waves and 64 rows otherwise.  The order of additions is the same for
// every shape.  (fc_down 3840 x 15360: 60 and 120 four-wave workgroups run
// 1.3-2x faster this way, 240 slower.)
template <bool kAffine>
qg_status gemm_general(const qg::GemmParams &p, int spg, int ks, hipStream_t stream) {
    const int64_t n = p.n;
    const int m = p.m;
    const int64_t tiles = (n + qg::kGemmRows - 1) / qg::kGemmRows;
    const int tb_max = 4 / ks;
    const int tb = m <= 16 ? 1 : (m <= 32 || tb_max == 2 ? 2 : 4);
    const int tbu = tb > tb_max ? tb_max : tb;
    const int64_t yblocks = (m + 16 * tbu - 1) / (16 * tbu);
    const int cus_all = device_cus();
    if (cus_all < 1) return QG_ERR_DEVICE;
    const int wps = (tbu == 1 && 2 * tiles * yblocks <= cus_all) ? 1 : 4;
    const int64_t rows_per_block = 16 * wps;
    const dim3 grid(unsigned((n + rows_per_block - 1) / rows_per_block), unsigned(yblocks));
    const dim3 block(unsigned(64 * wps * ks));
#define QG_GEMM_CASE(S, T, K, W)                                                                \
    if (spg == S && tbu == T && ks == K && wps == W) {                                          \
        constexpr int64_t lds = qg::gemm_general_lds(T, K, W, kAffine);                         \
        auto kern = qg::qgemm_fp4_kernel<S, T, K, W, kAffine>;                                  \
        if (lds > 64 * 1024) {                                                                  \
            static std::once_flag once;                                                         \
            static hipError_t attr = hipSuccess;                                                \
            std::call_once(once, [kern] {                                                       \
                attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),                \
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)); \
            });                                                                                 \
            if (attr != hipSuccess) return QG_ERR_LAUNCH;                                       \
        }                                                                                       \
        return qgl::launch_kernel(kern, grid, block, size_t(lds), stream, p);                   \
    }
#define QG_GEMM_SPG(S) QG_GEMM_CASE(S, 1, 1, 4) QG_GEMM_CASE(S, 2, 1, 4) QG_GEMM_CASE(S, 4, 1, 4) \
    QG_GEMM_CASE(S, 1, 2, 4) QG_GEMM_CASE(S, 2, 2, 4) QG_GEMM_CASE(S, 1, 4, 4)                   \
    QG_GEMM_CASE(S, 1, 1, 1) QG_GEMM_CASE(S, 1, 2, 1) QG_GEMM_CASE(S, 1, 4, 1)
    QG_GEMM_SPG(1)
    QG_GEMM_SPG(2)
    QG_GEMM_SPG(4)
#undef QG_GEMM_SPG
#undef QG_GEMM_CASE
    return QG_ERR_LAUNCH;     // not reached: every (group size, tb, ks, wps) above has an instance
}

// Up to 16 activation rows whose x fits in LDS: x staged once per
// workgroup, weight tiles streamed without barriers (the same bits as the
// general kernel)
bool gemm_small_fits(int64_t k, int32_t m) { return m <= 16 && qg::gemm_small_lds(k, m) <= 128 * 1024; }

template <bool kAffine>
qg_status gemm_small(const qg::GemmParams &p, int spg, int ks, hipStream_t stream) {
    const int cus = device_cus();
    if (cus < 1) return QG_ERR_DEVICE;
    const int64_t small_lds = qg::gemm_small_lds(p.k, p.m);
    // one workgroup per CU (x fills most of its LDS), with as many waves as
    // the 16-row tiles need to cover the chip, 1..8
    const int64_t rtiles = (p.n + 15) / 16;
    int64_t wpb = (rtiles + cus - 1) / cus;
    wpb = wpb < 1 ? 1 : (wpb > qg::kGemmSmallWaves ? qg::kGemmSmallWaves : wpb);
    int64_t blocks = (rtiles + wpb - 1) / wpb;
    if (blocks > cus) blocks = cus;
    const dim3 sgrid{unsigned(blocks)}, sblock{unsigned(64 * wpb)};
    // a chunk's group parameters as one vector load when they are aligned
    const int gpc = 8 / spg;
    const uintptr_t va = uintptr_t(2 * gpc);
    const bool vs = p.groups % gpc == 0 && aligned_to(p.scales, va) && (!kAffine || aligned_to(p.biases, va));
#define QG_GEMM_SMALL(S, K, V)                                                                          \
    if (spg == S && ks == K && vs == V) {                                                               \
        auto kern = qg::qgemm_fp4_small_kernel<S, K, V, kAffine>;                                       \
        static std::once_flag once;                                                                     \
        static hipError_t attr = hipSuccess;                                                            \
        std::call_once(once, [kern] {                                                                   \
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),                            \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);         \
        });                                                                                             \
        if (attr != hipSuccess) return QG_ERR_LAUNCH;                                                   \
        return qgl::launch_kernel(kern, sgrid, sblock, size_t(small_lds), stream, p);                   \
    }
#define QG_GEMM_SMALL_V(S, K) QG_GEMM_SMALL(S, K, true) QG_GEMM_SMALL(S, K, false)
    QG_GEMM_SMALL_V(1, 1) QG_GEMM_SMALL_V(1, 2) QG_GEMM_SMALL_V(1, 4)
    QG_GEMM_SMALL_V(2, 1) QG_GEMM_SMALL_V(2, 2) QG_GEMM_SMALL_V(2, 4)
    QG_GEMM_SMALL_V(4, 1) QG_GEMM_SMALL_V(4, 2) QG_GEMM_SMALL_V(4, 4)
#undef QG_GEMM_SMALL_V
#undef QG_GEMM_SMALL
    return QG_ERR_LAUNCH;     // not reached: every (group size, ks, vector load) above has an instance
}

// the arguments both GEMMs share, checked before any HIP call
qg_status gemm_check(const void *codes, const uint16_t *scales, const uint16_t *x, void *y, int64_t n, int64_t k,
                     int32_t group_size, int32_t m, qg_out_dtype out_dtype) {
    if (!codes || !scales || !x || !y) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 32 || k % 32 || k > (int64_t(1) << 30) || n > (int64_t(1) << 36))
        return QG_ERR_BAD_SHAPE;
    if (group_size != 32 && group_size != 64 && group_size != 128) return QG_ERR_BAD_GROUP_SIZE;
    if (k % group_size) return QG_ERR_BAD_GROUP_SIZE;
    if (m < 1 || m > QG_GEMM_MAX_M) return QG_ERR_BAD_BATCH;
    if (out_dtype != QG_OUT_F32 && out_dtype != QG_OUT_BF16) return QG_ERR_BAD_DTYPE;
    if (!aligned_to(codes, 16) || !aligned_to(x, 16) || !aligned_to(scales, 2) ||
        !aligned_to(y, out_dtype == QG_OUT_BF16 ? 2 : 4))
        return QG_ERR_MISALIGNED;
    return QG_OK;
}

qg::GemmParams gemm_params(const void *codes, const uint16_t *scales, const uint16_t *x, void *y, int64_t n,
                           int64_t k, int32_t group_size, int32_t m, qg_out_dtype out_dtype) {
    qg::GemmParams p{};
    p.codes = static_cast<const unsigned char *>(codes);
    p.scales = scales;
    p.x = x;
    p.y = y;
    p.n = n;
    p.k = int32_t(k);
    p.m = m;
    p.groups = int32_t(k / group_size);
    p.out_bf16 = out_dtype == QG_OUT_BF16 ? 1 : 0;
    return p;
}

}  // namespace

extern "C" {

qg_status qgemm_fp4_e2m1(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, void *y, int64_t n,
                         int64_t k, int32_t group_size, int32_t m, qg_out_dtype out_dtype, hipStream_t stream) {
    const qg_status st = gemm_check(codes, scales, x, y, n, k, group_size, m, out_dtype);
    if (st != QG_OK) return st;
    const qg::GemmParams p = gemm_params(codes, scales, x, y, n, k, group_size, m, out_dtype);
    const int ks = gemm_k_slices(n, k);
    const int spg = group_size / 32;
    if (gemm_small_fits(k, m)) return gemm_small<false>(p, spg, ks, stream);
    return gemm_general<false>(p, spg, ks, stream);
}

qg_status qgemm_affine_u4(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                          void *y, int64_t n, int64_t k, int32_t group_size, int32_t m, qg_out_dtype out_dtype,
                          hipStream_t stream) {
    if (!biases) return QG_ERR_NULL_POINTER;
    const qg_status st = gemm_check(codes, scales, x, y, n, k, group_size, m, out_dtype);
    if (st != QG_OK) return st;
    if (!aligned_to(biases, 2)) return QG_ERR_MISALIGNED;
    qg::GemmParams p = gemm_params(codes, scales, x, y, n, k, group_size, m, out_dtype);
    p.biases = biases;
    const int ks = gemm_k_slices(n, k);
    const int spg = group_size / 32;
    if (gemm_small_fits(k, m)) return gemm_small<true>(p, spg, ks, stream);
    return gemm_general<true>(p, spg, ks, stream);
}

}  // extern "C"
