// Kernel instances of the FP8-E4M3 format (compiled on their own, in parallel
// with the other formats): the row and LDS kernels for one or two activation
// rows, the matrix-core kernel (qgemv_fp8_mfma.hpp) for three or four where
// the planner chose it (rows whose batch-4 activations fit its LDS).
#include "qgemv_launch.hpp"
#include "qgemv_fp8_mfma.hpp"

namespace qgl {

namespace {

template <int PS, bool kNorm, int kH>
qg_status launch_fp8_b(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    constexpr int D = kH > 0 ? 2 : qg::fp8_mfma_depth(PS);
    static_assert(qg::kFp8MfmaMinBatch == 3, "instances for batch 3 and 4");
    if (batch == 3) return launch<qg::qgemv_fp8_mfma_kernel<3, PS, D, kNorm, kH>>(p, pl, lds, s);
    return launch<qg::qgemv_fp8_mfma_kernel<4, PS, D, kNorm, kH>>(p, pl, lds, s);
}

template <bool kNorm>
qg_status launch_fp8_n(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    switch (qg::fp8_mfma_halves(p.chunks)) {
        case 1: return launch_fp8_b<8, kNorm, 1>(p, pl, batch, lds, s);
        case 2: return launch_fp8_b<8, kNorm, 2>(p, pl, batch, lds, s);
        default: break;
    }
    switch (qg::fp8_mfma_step_passes(p.chunks)) {
        case 4: return launch_fp8_b<4, kNorm, 0>(p, pl, batch, lds, s);
        case 8: return launch_fp8_b<8, kNorm, 0>(p, pl, batch, lds, s);
        default: return launch_fp8_b<16, kNorm, 0>(p, pl, batch, lds, s);
    }
}

}  // namespace

qg_status launch_fp8(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    if (!pl.mfma || batch < qg::kFp8MfmaMinBatch) return launch_fmt<qg::FmtFP8>(p, pl, batch, lds, s);
    return p.norm ? launch_fp8_n<true>(p, pl, batch, lds, s) : launch_fp8_n<false>(p, pl, batch, lds, s);
}

}  // namespace qgl
