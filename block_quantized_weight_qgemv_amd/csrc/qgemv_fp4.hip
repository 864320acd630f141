// Kernel instances of the FP4-E2M1 format (compiled on their own, in parallel
// with the other formats).
#include "qgemv_launch.hpp"

namespace qgl {

qg_status launch_fp4(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    return launch_fmt<qg::FmtFP4>(p, pl, batch, lds, s);
}

}  // namespace qgl
