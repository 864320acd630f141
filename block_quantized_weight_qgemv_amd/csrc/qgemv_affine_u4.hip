// Kernel instances of the affine 4-bit format (compiled on their own, in parallel
// with the other formats).
#include "qgemv_launch.hpp"

namespace qgl {

qg_status launch_affine_u4(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    return launch_fmt<qg::FmtAffineU4>(p, pl, batch, lds, s);
}

}  // namespace qgl
