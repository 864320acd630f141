// Kernel instances of the FP8-E4M3 format (compiled on their own, in parallel
// with the other formats): the row and LDS kernels for one or two activation
// rows, the matrix-core kernel (qgemv_fp8_mfma.hpp) for three or four.
#include "qgemv_launch.hpp"
#include "qgemv_fp8_mfma.hpp"

namespace qgl {

namespace {

template <int PS, bool kNorm, bool kOne>
qg_status launch_fp8_ps1(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    constexpr int D = qg::fp8_mfma_depth(PS);
    static_assert(qg::kFp8MfmaMinBatch == 3, "instances for batch 3 and 4");
    if (batch == 3) return launch<qg::qgemv_fp8_mfma_kernel<3, PS, D, kNorm, kOne>>(p, pl, lds, s);
    return launch<qg::qgemv_fp8_mfma_kernel<4, PS, D, kNorm, kOne>>(p, pl, lds, s);
}

// rows of at most PS passes are one step
template <int PS, bool kNorm>
qg_status launch_fp8_ps(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    if (p.passes <= PS) return launch_fp8_ps1<PS, kNorm, true>(p, pl, batch, lds, s);
    return launch_fp8_ps1<PS, kNorm, false>(p, pl, batch, lds, s);
}

template <bool kNorm>
qg_status launch_fp8_n(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    switch (qg::fp8_mfma_step_passes(p.chunks)) {
        case 4: return launch_fp8_ps<4, kNorm>(p, pl, batch, lds, s);
        case 8: return launch_fp8_ps<8, kNorm>(p, pl, batch, lds, s);
        default: return launch_fp8_ps<16, kNorm>(p, pl, batch, lds, s);
    }
}

}  // namespace

qg_status launch_fp8(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    if (batch < qg::kFp8MfmaMinBatch) return launch_fmt<qg::FmtFP8>(p, pl, batch, lds, s);
    return p.norm ? launch_fp8_n<true>(p, pl, batch, lds, s) : launch_fp8_n<false>(p, pl, batch, lds, s);
}

}  // namespace qgl
