// Launch shapes and the dispatch from a format, a batch size and a plan to a
// kernel instance.  The kernel instances of each format are compiled in a
// file of their own (qgemv_fp4.hip, ...), which defines that format's
// launcher; qgemv_api.hip plans the launch and calls it.
#pragma once

#include "qgemv.h"
#include "qgemv_device.hpp"
#include "qgemv_kernels.hpp"
#include "qgemv_mfma4.hpp"

#include <mutex>

namespace qgl {

using qg::Params;

// Largest dynamic LDS a workgroup may use for the staged activations.  MI355X
// has 160 KiB of LDS per compute unit; 128 KiB leaves room for a second,
// smaller workgroup.
constexpr int64_t kMaxLds = 128 * 1024;
// The matrix-block kernel runs one workgroup per compute unit and may take
// all of it.
constexpr int64_t kM4MaxLds = 160 * 1024;

struct Plan {
    int rows_per_tile;
    int waves_per_block;
    int blocks;
    bool row_kernel;       // x in registers (row kernel) or staged in LDS
    int passes;            // row kernel: passes per K segment (1, 2 or 4)
    bool mfma = false;     // batch 3-4 on a matrix-core kernel (FP8, or the 4-bit formats)
};


// One function per kernel instance, so that each instance raises its own
// LDS limit (kLimit) once.
template <auto Kern, int64_t kLimit = kMaxLds>
inline qg_status launch(const Params &p, const Plan &pl, int64_t lds, hipStream_t stream) {
    if (lds > 64 * 1024) {
        static std::once_flag attr_once;
        static hipError_t attr_err = hipSuccess;
        std::call_once(attr_once, [&] {
            attr_err = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(kLimit));
        });
        if (attr_err != hipSuccess) return QG_ERR_LAUNCH;
    }
    return launch_kernel(Kern, dim3(pl.blocks), dim3(pl.waves_per_block * qg::kWave), size_t(lds), stream, p);
}

// prefetch depth: about 8 code loads in flight per lane
// (two when more than 16 activation pieces already fill the registers)
constexpr int row_depth(int r, int j, int pieces) { return pieces > 16 ? 2 : (8 / (r * j) > 2 ? 8 / (r * j) : 2); }
constexpr int lds_depth(int r) { return r == 1 ? 8 : 4; }

// passes per K segment the planner gives a format: two for 16-byte-wide
// activation pieces (4-bit formats, u8), four for FP8's (half as wide)
constexpr int row_max_passes(int pieces) { return pieces >= 4 ? 2 : 4; }

// register budget of the row kernel: at most 32 activation pieces per lane,
// and fewer rows per tile when they are many (one row for the affine formats,
// whose chunk sums and biases take further registers); no instance spills
template <class Fmt, int R, int B, int J>
constexpr bool row_instance() {
    return B * J * Fmt::kPieces <= 32 && (B * J * Fmt::kPieces <= 16 || R <= (Fmt::kSums ? 1 : 2)) &&
           !(R == 4 && J == 4) && J <= row_max_passes(Fmt::kPieces);
}

template <class Fmt, int R, int B, bool kNorm>
qg_status launch_row_j(const Params &p, const Plan &pl, int64_t lds, hipStream_t s) {
    switch (pl.passes) {
        case 1:
            if constexpr (row_instance<Fmt, R, B, 1>())
                return launch<qg::qgemv_row_kernel<Fmt, R, B, row_depth(R, 1, B * 1 * Fmt::kPieces), 1, kNorm>>(p, pl, lds, s);
            break;
        case 2:
            if constexpr (row_instance<Fmt, R, B, 2>())
                return launch<qg::qgemv_row_kernel<Fmt, R, B, row_depth(R, 2, B * 2 * Fmt::kPieces), 2, kNorm>>(p, pl, lds, s);
            break;
        case 4:
            if constexpr (row_instance<Fmt, R, B, 4>())
                return launch<qg::qgemv_row_kernel<Fmt, R, B, row_depth(R, 4, B * 4 * Fmt::kPieces), 4, kNorm>>(p, pl, lds, s);
            break;
    }
    return QG_ERR_LAUNCH;     // not reached: the planner only picks existing instances
}

// The fused-norm variants run their own instances (kNorm), so the plain
// instances carry none of that code.  The LDS kernel's form for activations
// too large for LDS (p.x_global) always takes one-row tiles, two steps in
// flight (each step carries the lane's activation units as well).
template <class Fmt, int R, int B>
qg_status launch_rb(const Params &p, const Plan &pl, int64_t lds, hipStream_t s) {
    if (p.norm) {
        if (pl.row_kernel) return launch_row_j<Fmt, R, B, true>(p, pl, lds, s);
        if (p.x_global) return launch<qg::qgemv_lds_kernel<Fmt, 1, B, 2, true, true>>(p, pl, lds, s);
        return launch<qg::qgemv_lds_kernel<Fmt, R, B, lds_depth(R), true>>(p, pl, lds, s);
    }
    if (pl.row_kernel) return launch_row_j<Fmt, R, B, false>(p, pl, lds, s);
    if (p.x_global) return launch<qg::qgemv_lds_kernel<Fmt, 1, B, 2, false, true>>(p, pl, lds, s);
    return launch<qg::qgemv_lds_kernel<Fmt, R, B, lds_depth(R), false>>(p, pl, lds, s);
}

template <class Fmt, int R>
qg_status launch_r(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    switch (batch) {
        case 1: return launch_rb<Fmt, R, 1>(p, pl, lds, s);
        case 2: return launch_rb<Fmt, R, 2>(p, pl, lds, s);
        case 3: return launch_rb<Fmt, R, 3>(p, pl, lds, s);
        default: return launch_rb<Fmt, R, 4>(p, pl, lds, s);
    }
}

// The 4-bit formats at batch 3-4 on the matrix blocks (qgemv_mfma4.hpp):
// steps of kM4StepPasses passes, kM4Depth of them in flight per wave.
template <class Fmt, bool kNorm>
qg_status launch_mfma4_n(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    if (batch == 3) return launch<qg::qgemv_mfma4_kernel<Fmt, 3, kNorm>, kM4MaxLds>(p, pl, lds, s);
    return launch<qg::qgemv_mfma4_kernel<Fmt, 4, kNorm>, kM4MaxLds>(p, pl, lds, s);
}

template <class Fmt>
qg_status launch_fmt(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s) {
    if constexpr (Fmt::kWpc == 32) {
        if (pl.mfma && batch >= qg::kM4MinBatch)
            return p.norm ? launch_mfma4_n<Fmt, true>(p, pl, batch, lds, s) : launch_mfma4_n<Fmt, false>(p, pl, batch, lds, s);
    }
    switch (pl.rows_per_tile) {
        case 1: return launch_r<Fmt, 1>(p, pl, batch, lds, s);
        case 2: return launch_r<Fmt, 2>(p, pl, batch, lds, s);
        default: return launch_r<Fmt, 4>(p, pl, batch, lds, s);
    }
}

// One launcher per format, each defined in that format's file.
qg_status launch_fp4(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s);
qg_status launch_affine_u4(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s);
qg_status launch_affine_u8(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s);
qg_status launch_fp8(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s);
qg_status launch_q4k(const Params &p, const Plan &pl, int32_t batch, int64_t lds, hipStream_t s);

}  // namespace qgl
