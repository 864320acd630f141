// Kernel instances of the FP8-E4M3 format (compiled on their own, in parallel
// with the other formats).
#include "qgemv_launch.hpp"

namespace qgl {

qg_status launch_fp8(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    return launch_fmt<qg::FmtFP8>(p, pl, batch, lds, s);
}

}  // namespace qgl
