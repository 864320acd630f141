// Kernel instances of the two-level super-block 4-bit format (compiled on
// their own, in parallel with the other formats).
#include "qgemv_launch.hpp"

namespace qgl {

qg_status launch_q4k(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    return launch_fmt<qg::FmtQ4K>(p, pl, batch, lds, s);
}

}  // namespace qgl
