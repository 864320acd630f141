// C ABI of the small-batch GEMM (more than four activation rows): argument
// validation and the launch.  As for the matvec, every argument is checked
// before any HIP call, so a bad argument launches nothing and leaves y alone.

#include "qgemv.h"
#include "qgemm_kernels.hpp"

namespace {

bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

qg_status qgemm_fp4_e2m1(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, void *y, int64_t n,
                         int64_t k, int32_t group_size, int32_t m, qg_out_dtype out_dtype, hipStream_t stream) {
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

    qg::GemmParams p{};
    p.codes = codes;
    p.scales = scales;
    p.x = x;
    p.y = y;
    p.n = n;
    p.k = int32_t(k);
    p.m = m;
    p.groups = int32_t(k / group_size);
    p.out_bf16 = out_dtype == QG_OUT_BF16 ? 1 : 0;
    const dim3 grid(unsigned((n + qg::kGemmRows - 1) / qg::kGemmRows),
                    unsigned((m + qg::kGemmTokens - 1) / qg::kGemmTokens));
    switch (group_size) {
        case 32: hipLaunchKernelGGL(qg::qgemm_fp4_kernel<1>, grid, dim3(256), 0, stream, p); break;
        case 64: hipLaunchKernelGGL(qg::qgemm_fp4_kernel<2>, grid, dim3(256), 0, stream, p); break;
        default: hipLaunchKernelGGL(qg::qgemm_fp4_kernel<4>, grid, dim3(256), 0, stream, p); break;
    }
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // extern "C"
