// Kernel instances of the affine 8-bit format (compiled on their own, in parallel
// with the other formats).
#include "qgemv_launch.hpp"

namespace qgl {

qg_status launch_affine_u8(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    return launch_fmt<qg::FmtAffineU8>(p, pl, batch, lds, s);
}

}  // namespace qgl
