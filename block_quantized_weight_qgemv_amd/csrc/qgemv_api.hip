// C ABI of the block-quantized weight matvec: argument validation, launch
// planning and dispatch to the per-format launchers (qgemv_launch.hpp; the
// kernel instances of each format are compiled in a file of their own).
//
// Validation runs completely before any HIP call, so a bad argument never
// launches anything and never touches y.  The only state kept across calls is
// a per-device cache of the compute-unit count and of which kernel instances
// have had their LDS limit raised; both are filled once, thread-safely.

#include "qgemv.h"
#include "qgemv_launch.hpp"
#include "qgemv_kernels.hpp"
#include "qgemv_fp8_mfma.hpp"
#include "stream_probe.hpp"
#include "qgemv_device.hpp"

#include <atomic>
#include <mutex>

namespace {

using qg::Params;
using qgl::kMaxLds;
using qgl::Plan;

constexpr int64_t kCounterBytes = 32;     // row kernel: up to 8 per-segment tile counters
constexpr int kMaxDevices = 64;

struct FmtInfo {
    int wpc;        // weights per 16-byte chunk
    int pieces;     // 16-byte LDS pieces per chunk and batch row
    bool sums;      // per-chunk activation sums staged
};

FmtInfo fmt_info(qg_format f) {
    switch (f) {
        case QG_FMT_FP4_E2M1: return {qg::FmtFP4::kWpc, qg::FmtFP4::kPieces, qg::FmtFP4::kSums};
        case QG_FMT_AFFINE_U4: return {qg::FmtAffineU4::kWpc, qg::FmtAffineU4::kPieces, qg::FmtAffineU4::kSums};
        case QG_FMT_AFFINE_U8: return {qg::FmtAffineU8::kWpc, qg::FmtAffineU8::kPieces, qg::FmtAffineU8::kSums};
        case QG_FMT_Q4K: return {qg::FmtQ4K::kWpc, qg::FmtQ4K::kPieces, qg::FmtQ4K::kSums};
        default: return {qg::FmtFP8::kWpc, qg::FmtFP8::kPieces, qg::FmtFP8::kSums};
    }
}

// must equal qg::LdsKernel<...>::lds_bytes
int64_t lds_bytes(qg_format f, int64_t k, int32_t batch) {
    const FmtInfo fi = fmt_info(f);
    const int64_t chunks = k / fi.wpc;
    return int64_t(batch) * fi.pieces * chunks * 16 + (fi.sums ? int64_t(batch) * chunks * 4 : 0) +
           qg::kLdsSink;
}

bool aligned(const void *p, uintptr_t a) { return qgl::aligned_to(p, a); }

qg_status check_common(qg_format f, const void *codes, const void *x, const void *y, int64_t n,
                       int64_t k, int32_t batch, qg_out_dtype out) {
    if (!codes || !x || !y) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 1) return QG_ERR_BAD_SHAPE;
    const FmtInfo fi = fmt_info(f);
    if (k % fi.wpc) return QG_ERR_BAD_SHAPE;
    if (n > (int64_t(1) << 31) || k > (int64_t(1) << 30)) return QG_ERR_BAD_SHAPE;
    if (batch < 1 || batch > 4) return QG_ERR_BAD_BATCH;
    if (out != QG_OUT_F32 && out != QG_OUT_BF16) return QG_ERR_BAD_DTYPE;
    if (!aligned(codes, 16) || !aligned(x, 16)) return QG_ERR_MISALIGNED;
    if (!aligned(y, out == QG_OUT_F32 ? 4 : 2)) return QG_ERR_MISALIGNED;
    return QG_OK;
}

qg_status check_groups(const void *scales, const void *biases, bool need_bias, int64_t k,
                       int32_t group_size, int wpc) {
    if (!scales || (need_bias && !biases)) return QG_ERR_NULL_POINTER;
    if (group_size != 32 && group_size != 64 && group_size != 128) return QG_ERR_BAD_GROUP_SIZE;
    if (group_size < wpc || k % group_size) return QG_ERR_BAD_GROUP_SIZE;
    if (!aligned(scales, 2) || (need_bias && !aligned(biases, 2))) return QG_ERR_MISALIGNED;
    return QG_OK;
}

int log2i(int v) {
    int s = 0;
    while ((1 << s) < v) ++s;
    return s;
}

// ---------------------------------------------------------------- device info

qg_status device_cus(int *cus) {
    const int v = qgl::device_cu_count();
    if (v <= 0) return QG_ERR_DEVICE;
    *cus = v;
    return QG_OK;
}

// ---------------------------------------------------------------- planning

int passes_of(int64_t chunks) { return int((chunks + qg::kWave - 1) / qg::kWave); }

// The row kernel keeps each wave's slice of x in registers: rows are cut into
// S = 1, 2, 4 or 8 equal K segments of at most two passes (four for FP8,
// whose activation pieces are half as wide).  S depends only on the format
// and k, so every batch size and launch shape adds a row's terms in the same
// order.  A segment's group parameters must be one dword per lane: an even
// number of groups, at most 128, on a group boundary, on 4-byte aligned rows.
struct Split {
    int segs, seg_chunks, seg_groups, passes;
    bool ok;
};

Split split_of(qg_format f, const Params &p) {
    const FmtInfo fi = fmt_info(f);
    Split sp{1, p.chunks, p.groups, 0, false};
    const int jmax = qgl::row_max_passes(fi.pieces);
    int need = int((p.chunks + 64 * jmax - 1) / (64 * jmax));
    int segs = 1;
    while (segs < need) segs <<= 1;
    if (segs > 8 || p.chunks % segs) return sp;
    sp.segs = segs;
    sp.seg_chunks = p.chunks / segs;
    sp.passes = passes_of(sp.seg_chunks);
    if (sp.passes != 1 && sp.passes != 2 && sp.passes != 4) return sp;
    if (f != QG_FMT_FP8_E4M3) {
        if (p.groups % segs) return sp;
        sp.seg_groups = p.groups / segs;
        if ((int64_t(sp.seg_chunks) << 0) % (int64_t(1) << p.group_shift)) return sp;
        if (sp.seg_groups < 2 || sp.seg_groups % 2 || sp.seg_groups > 128) return sp;
        // the two-level format: whole super-blocks of 8 groups per segment
        if (f == QG_FMT_Q4K && sp.seg_groups % 8) return sp;
    } else {
        sp.seg_groups = 0;
    }
    sp.ok = true;
    return sp;
}

bool row_kernel_fits(qg_format f, const Params &p, int32_t batch) {
    if (!p.segs) return false;
    const FmtInfo fi = fmt_info(f);
    if (int64_t(batch) * p.passes * fi.pieces > 32) return false;
    if (f != QG_FMT_FP8_E4M3) {
        if (!aligned(p.scales, 4)) return false;
        if (f != QG_FMT_FP4_E2M1 && !aligned(p.biases, 4)) return false;
    }
    return true;
}

int64_t row_lds_bytes(const Params &p, int blocks, int32_t batch) {
    if (p.segs <= 1) return 0;
    const int64_t rows = (p.n + blocks - 1) / blocks;
    return rows * p.segs * batch * 4;
}

Plan default_plan(qg_format f, const Params &p, int32_t batch, int cus) {
    Plan pl;
    pl.row_kernel = row_kernel_fits(f, p, batch);
    pl.passes = p.passes;
    if (pl.row_kernel) {
        // one workgroup of 8 waves per CU: its first four waves stage x for
        // the four dispatched after them.  One row per tile for FP8: its rows
        // hold twice the bytes of 4-bit rows of the same k, so a one-row tile
        // carries as many loads as a two-row 4-bit tile.
        pl.rows_per_tile = f == QG_FMT_FP8_E4M3 ? 1 : 2;
        pl.waves_per_block = 8;
    } else {
        pl.rows_per_tile = 2;
        pl.waves_per_block = 4;
    }
    const int64_t waves_per_cu = 8;
    int64_t blocks = int64_t(cus) * waves_per_cu / pl.waves_per_block;
    // FP4 at batch 1 with one to two tiles per wave: two workgroups per CU
    // and one tile per wave, so that every tile's loads go out at the start
    // (the instance fits four waves per SIMD; 8192 x 3840: 5.68 -> 5.37 us,
    // while every other shape measured, the formats whose instances take
    // more registers, and the fused norm, whose every workgroup computes
    // the norm, are slower with more workgroups)
    if (pl.row_kernel && f == QG_FMT_FP4_E2M1 && batch == 1 && p.segs == 1 && !p.norm) {
        const int64_t tiles = (p.n + pl.rows_per_tile - 1) / pl.rows_per_tile;
        const int64_t waves = blocks * pl.waves_per_block;
        if (tiles > waves && tiles <= 2 * waves) blocks *= 2;
        // Too few rows for one 8-wave workgroup per CU: fewer waves per
        // workgroup (below four each wave loads its own slice of x, with no
        // staging barrier) over more CUs (256 x 512: 2.92 -> 2.51 us,
        // 1024 x 3840: 3.20 -> 3.08)
        if (p.n < waves_per_cu * cus) {
            int64_t w = p.n / (2 * int64_t(cus));
            pl.waves_per_block = w >= 4 ? 4 : (w >= 2 ? 2 : 1);
            blocks = cus;
        }
    }
    const int64_t max_blocks = (p.n + pl.waves_per_block - 1) / pl.waves_per_block;
    if (blocks > max_blocks) blocks = max_blocks;
    pl.blocks = int(blocks < 1 ? 1 : blocks);
    return pl;
}

// Whether a row-kernel instance exists for these (R, B, passes).
template <class Fmt>
bool row_instance_exists(int r, int b, int j) {
    const int pcs = Fmt::kPieces;
    return b * j * pcs <= 32 && (b * j * pcs <= 16 || r <= (Fmt::kSums ? 1 : 2)) && !(r == 4 && j == 4) &&
           j <= qgl::row_max_passes(pcs);
}

qg_status check_plan(const qg_plan *plan) {
    if (!plan) return QG_OK;
    const int r = plan->rows_per_tile, w = plan->waves_per_block;
    if (r != 0 && r != 1 && r != 2 && r != 4) return QG_ERR_BAD_SHAPE;
    if (w < 0 || w > 8) return QG_ERR_BAD_SHAPE;
    if (plan->blocks < 0) return QG_ERR_BAD_SHAPE;
    return QG_OK;
}

bool row_instance_for(qg_format f, int r, int b, int j) {
    switch (f) {
        case QG_FMT_FP4_E2M1: return row_instance_exists<qg::FmtFP4>(r, b, j);
        case QG_FMT_AFFINE_U4: return row_instance_exists<qg::FmtAffineU4>(r, b, j);
        case QG_FMT_AFFINE_U8: return row_instance_exists<qg::FmtAffineU8>(r, b, j);
        case QG_FMT_Q4K: return row_instance_exists<qg::FmtQ4K>(r, b, j);
        default: return row_instance_exists<qg::FmtFP8>(r, b, j);
    }
}

// FP8 with three or four activation rows runs on the matrix-core kernel
// (qgemv_fp8_mfma.hpp): 4-row tiles, x in LDS.  Its default launch is one
// workgroup of 8 waves per CU (fewer workgroups when tiles are few);
// rows_per_tile is fixed.  It takes every k whose batch-4 activations fit its
// LDS beside the fused norm's sums (k <= 16304), at batch 3 as at batch 4 and
// with or without the norm, so that every call of the group adds a row's
// terms in the same order; longer rows take the vector kernels, as batch 1
// and 2 do.
bool fp8_mfma_takes(const Params &p) {
    // the fused norm's sums counted for the plain call too: both calls of a
    // k take the same kernel, so the fused one stays bitwise the plain one's
    const int64_t norm_bytes = int64_t(4) * ((p.k / 8 + qg::kWave - 1) / qg::kWave) * 4;
    return int64_t(4) * p.k * 2 + qg::kLdsSink + norm_bytes <= kMaxLds;
}

Plan fp8_default_plan(const Params &p, int cus) {
    Plan pl;
    pl.row_kernel = false;
    pl.mfma = true;
    pl.passes = p.passes;
    pl.rows_per_tile = qg::kFp8TileRows;
    pl.waves_per_block = 8;
    const int64_t tiles = (p.n + qg::kFp8TileRows - 1) / qg::kFp8TileRows;
    int64_t blocks = cus;
    const int64_t max_blocks = (tiles + pl.waves_per_block - 1) / pl.waves_per_block;
    if (blocks > max_blocks) blocks = max_blocks;
    pl.blocks = int(blocks < 1 ? 1 : blocks);
    return pl;
}

qg_status run_fp8(Params p, int32_t batch, const qg_plan *override_plan, hipStream_t stream, int cus) {
    p.passes = (p.chunks + qg::kFp8Slots - 1) / qg::kFp8Slots;
    Plan pl = fp8_default_plan(p, cus);
    if (override_plan) {
        if (override_plan->waves_per_block) pl.waves_per_block = override_plan->waves_per_block;
        if (override_plan->blocks) {
            pl.blocks = override_plan->blocks;
        } else {
            const int64_t tiles = (p.n + qg::kFp8TileRows - 1) / qg::kFp8TileRows;
            const int64_t max_blocks = (tiles + pl.waves_per_block - 1) / pl.waves_per_block;
            int64_t b = int64_t(cus) * 8 / pl.waves_per_block;
            pl.blocks = int(b > max_blocks ? max_blocks : (b < 1 ? 1 : b));
        }
    }
    // LDS: x and two zero units (Fp8XLayout), the tile counter, the norm's group sums
    const int64_t norm_bytes = p.norm ? int64_t(batch) * ((p.k / 8 + qg::kWave - 1) / qg::kWave) * 4 : 0;
    int64_t lds = int64_t(batch) * p.k * 2 + qg::kLdsSink;
    // the shared-tile counter, where it fits (otherwise each wave takes a
    // fixed range of tiles; the result is the same bits either way)
    if (lds + 16 + norm_bytes <= kMaxLds) {
        p.counter_offset = int32_t(lds);
        lds += 16;
    }
    p.norm_offset = int32_t(lds);
    lds += norm_bytes;
    if (lds > kMaxLds) return QG_ERR_TOO_LARGE;
    // fused norm: gamma in LDS too where it fits (the same bits as reading it
    // from memory)
    p.gamma_offset = 0;
    if (p.norm) {
        const int64_t g_off = (lds + 15) / 16 * 16;
        if (g_off + int64_t(p.k) * 2 <= kMaxLds) {
            p.gamma_offset = int32_t(g_off);
            lds = g_off + int64_t(p.k) * 2;
        }
    }
    p.total_waves = pl.blocks * pl.waves_per_block;
    return qgl::launch_fp8(p, pl, batch, lds, stream);
}

// LDS bytes of x in the fused norm's row kernel: with a 16-byte pad after
// every 64-byte chunk for the formats whose chunks hold 32 activations
int64_t norm_x_bytes(qg_format f, int64_t k, int32_t batch) {
    const int64_t bytes = int64_t(batch) * k * 2;
    return fmt_info(f).wpc == 32 ? bytes / 4 * 5 : bytes;
}

// Whether the fused norm's row kernel fits its LDS (x, gamma, the tile
// counters, one row's split-K partials, the norm's group sums).
bool norm_row_fits(qg_format f, const Params &p, int32_t batch) {
    const int64_t b = batch;
    const int64_t norm_bytes = b * ((p.k / 8 + qg::kWave - 1) / qg::kWave) * 4;
    return norm_x_bytes(f, p.k, batch) + p.k * 2 + kCounterBytes + int64_t(p.segs) * b * 4 + norm_bytes <= kMaxLds;
}

// The 4-bit formats (FP4, affine u4, the two-level format) at three or four
// activation rows run on the matrix blocks (qgemv_mfma4.hpp) where x at batch
// 4 fits its LDS (decided by k and the norm alone, so batch 3 and 4 add a
// row's terms in one order): 4-row tiles, one workgroup of 8 waves per CU
// (fewer when there are fewer tiles than CUs); rows_per_tile of a plan is
// ignored.
bool mfma4_format(qg_format f) { return f == QG_FMT_FP4_E2M1 || f == QG_FMT_AFFINE_U4 || f == QG_FMT_Q4K; }

int64_t mfma4_lds(qg_format f, const Params &p, int32_t batch) {
    const int64_t norm_bytes = p.norm ? int64_t(batch) * ((p.k / 8 + qg::kWave - 1) / qg::kWave) * 4 : 0;
    return qg::mfma4_lds_bytes(p.chunks, batch, fmt_info(f).sums) + norm_bytes;
}

// (the fused norm's sums are counted for the plain call too, as for FP8, and
// 1 KiB is kept for the split-K partials of at least one tile).  This kernel
// runs one workgroup per CU, so it may take all of gfx950's 160 KiB of LDS
// (qgl::kM4MaxLds).
constexpr int64_t kM4PartReserve = 1024;
using qgl::kM4MaxLds;

bool mfma4_takes(qg_format f, const Params &p) {
    const int64_t norm_bytes = int64_t(4) * ((p.k / 8 + qg::kWave - 1) / qg::kWave) * 4;
    return mfma4_format(f) &&
           qg::mfma4_lds_bytes(p.chunks, 4, fmt_info(f).sums) + norm_bytes + kM4PartReserve <= kM4MaxLds;
}

Plan mfma4_plan(const Params &p, int cus, const qg_plan *override_plan) {
    Plan pl;
    pl.row_kernel = false;
    pl.mfma = true;
    pl.passes = p.passes;
    pl.rows_per_tile = qg::kM4Rows;
    pl.waves_per_block = 8;
    if (override_plan && override_plan->waves_per_block) pl.waves_per_block = override_plan->waves_per_block;
    // at least one tile per workgroup (the waves split a workgroup's steps)
    const int64_t max_blocks = (p.n + qg::kM4Rows - 1) / qg::kM4Rows;
    int64_t blocks = int64_t(cus) * 8 / pl.waves_per_block;
    if (override_plan && override_plan->blocks) blocks = override_plan->blocks;
    else if (blocks > max_blocks) blocks = max_blocks;
    pl.blocks = int(blocks < 1 ? 1 : blocks);
    return pl;
}

qg_status run_mfma4(qg_format f, Params p, int32_t batch, const qg_plan *override_plan, hipStream_t stream, int cus) {
    p.passes = (p.chunks + qg::kM4Slots - 1) / qg::kM4Slots;
    Plan pl = mfma4_plan(p, cus, override_plan);
    const int64_t base = qg::mfma4_lds_bytes(p.chunks, batch, fmt_info(f).sums);
    const int64_t norm_bytes = mfma4_lds(f, p, batch) - base;
    // split-K partials: [tile row][step][batch row] floats for the
    // workgroup's tiles, when a tile has several steps; more, smaller
    // workgroups where they would not fit
    const int ps = qg::kM4StepPasses;
    const int64_t steps = (p.passes + ps - 1) / ps;
    const int64_t tiles = (p.n + qg::kM4Rows - 1) / qg::kM4Rows;
    int64_t part_bytes = 0;
    if (steps > 1) {
        const int64_t per_tile = int64_t(qg::kM4Rows) * steps * batch * 4;
        const int64_t max_tiles = (kM4MaxLds - base - norm_bytes) / per_tile;     // >= 1 (kM4PartReserve)
        if ((tiles + pl.blocks - 1) / pl.blocks > max_tiles) pl.blocks = int((tiles + max_tiles - 1) / max_tiles);
        part_bytes = (tiles + pl.blocks - 1) / pl.blocks * per_tile;
    }
    p.part_offset = int32_t(base);
    p.norm_offset = int32_t(base + part_bytes);
    int64_t lds = base + part_bytes + norm_bytes;
    // fused norm: gamma in LDS too where it fits (the same bits as reading it
    // from memory)
    p.gamma_offset = 0;
    if (p.norm) {
        const int64_t g_off = (lds + 15) / 16 * 16;
        if (g_off + int64_t(p.k) * 2 <= kM4MaxLds) {
            p.gamma_offset = int32_t(g_off);
            lds = g_off + int64_t(p.k) * 2;
        }
    }
    p.total_waves = pl.blocks * pl.waves_per_block;
    switch (f) {
        case QG_FMT_FP4_E2M1: return qgl::launch_fp4(p, pl, batch, lds, stream);
        case QG_FMT_AFFINE_U4: return qgl::launch_affine_u4(p, pl, batch, lds, stream);
        default: return qgl::launch_q4k(p, pl, batch, lds, stream);
    }
}

// Launch plan for the LDS kernel: the plan's rows per tile and waves, x
// staged in LDS when it fits beside the norm's sums, read from memory with
// the weights (one-row tiles) otherwise.
void lds_kernel_setup(qg_format f, Params &p, Plan &pl, int32_t batch, int64_t norm_bytes, int64_t &lds) {
    pl.row_kernel = false;
    p.passes = passes_of(p.chunks);               // the LDS kernel walks whole rows
    lds = lds_bytes(f, p.k, batch);
    p.x_global = lds + norm_bytes > kMaxLds ? 1 : 0;
    if (p.x_global) {
        lds = 0;
        pl.rows_per_tile = 1;
    }
    p.norm_offset = int32_t(lds);
    lds += norm_bytes;
}

qg_status run(qg_format f, Params p, int32_t batch, const qg_plan *override_plan, hipStream_t stream) {
    int cus = 0;
    qg_status st = device_cus(&cus);
    if (st != QG_OK) return st;
    if (f == QG_FMT_FP8_E4M3 && batch >= qg::kFp8MfmaMinBatch && fp8_mfma_takes(p))
        return run_fp8(p, batch, override_plan, stream, cus);
    if (batch >= qg::kM4MinBatch && mfma4_takes(f, p)) return run_mfma4(f, p, batch, override_plan, stream, cus);
    const Split sp = split_of(f, p);
    if (sp.ok) {
        p.segs = sp.segs;
        p.seg_chunks = sp.seg_chunks;
        p.seg_groups = sp.seg_groups;
        p.passes = sp.passes;
    } else {
        p.segs = 0;                               // the row kernel does not apply
        p.passes = passes_of(p.chunks);
    }
    // The fused norm's row kernel holds x and gamma in LDS.  Where they do not
    // fit ((batch + 1) * k * 2 bytes beside the split-K partials and the
    // norm's sums) the LDS kernel takes the call: the same bound, but its own
    // order of additions, so such a call is not bitwise the plain call on
    // the separately normalized x.
    if (p.norm && p.segs && !norm_row_fits(f, p, batch)) p.segs = 0;
    Plan pl = default_plan(f, p, batch, cus);
    auto apply_override = [&](Plan &q) {
        if (!override_plan) return;
        if (override_plan->rows_per_tile) q.rows_per_tile = override_plan->rows_per_tile;
        if (override_plan->waves_per_block) q.waves_per_block = override_plan->waves_per_block;
        if (override_plan->blocks) q.blocks = override_plan->blocks;
        else {
            const int64_t max_blocks = (p.n + q.waves_per_block - 1) / q.waves_per_block;
            int64_t b = int64_t(cus) * 8 / q.waves_per_block;
            q.blocks = int(b > max_blocks ? max_blocks : (b < 1 ? 1 : b));
        }
    };
    apply_override(pl);
    // fused RMSNorm: one float per group of 64 activation units per batch row
    const int64_t norm_bytes = p.norm ? int64_t(batch) * ((p.k / 8 + qg::kWave - 1) / qg::kWave) * 4 : 0;
    int64_t lds = 0;
    if (pl.row_kernel) {
        // a workgroup holds whole row groups of `segs` waves
        if (pl.waves_per_block % p.segs) {
            pl.waves_per_block = (pl.waves_per_block / p.segs + 1) * p.segs;
            if (pl.waves_per_block > 8) pl.waves_per_block = p.segs;
        }
        // fewer rows per tile where the register budget asks for it
        while (pl.rows_per_tile > 1 && !row_instance_for(f, pl.rows_per_tile, batch, pl.passes))
            pl.rows_per_tile /= 2;
        // x is shared through LDS when the workgroup has the four staging
        // waves and x fits their staging registers (k is a multiple of 8, so
        // x takes a multiple of 16 bytes)
        // (the fused norm always takes x through LDS instead)
        p.x_staged = (!p.norm && int64_t(pl.waves_per_block) * qg::kWave >= qg::kStageThreads &&
                      int64_t(batch) * p.k / 8 <= int64_t(qg::kStageThreads) * qg::kStageUnits &&
                      qg::row_can_stage(batch, pl.passes, fmt_info(f).pieces)) ? 1 : 0;
        // LDS: x (staged or normalized), gamma (fused norm), the per-segment
        // tile counters (x in LDS), the split-K partials, the norm's sums
        const bool via_lds = p.x_staged || p.norm;
        const int64_t x_bytes = !via_lds ? 0 : (p.norm ? norm_x_bytes(f, p.k, batch) : int64_t(batch) * p.k * 2);
        const int64_t g_bytes = p.norm ? int64_t(p.k) * 2 : 0;
        p.gamma_offset = int32_t(x_bytes);
        p.counter_offset = int32_t(x_bytes + g_bytes);
        p.part_offset = int32_t(x_bytes + g_bytes + (via_lds ? kCounterBytes : 0));
        lds = p.part_offset + row_lds_bytes(p, pl.blocks, batch);
        if (lds + norm_bytes > kMaxLds) {
            // more, smaller workgroups until the split-K partials fit
            const int64_t room = kMaxLds - p.part_offset - norm_bytes;
            pl.blocks = int((p.n * p.segs * batch * 4 + room - 1) / room);
            while (p.part_offset + row_lds_bytes(p, pl.blocks, batch) + norm_bytes > kMaxLds) ++pl.blocks;
            lds = p.part_offset + row_lds_bytes(p, pl.blocks, batch);
        }
        p.norm_offset = int32_t(lds);
        lds += norm_bytes;
    } else {
        lds_kernel_setup(f, p, pl, batch, norm_bytes, lds);
    }
    p.total_waves = pl.blocks * pl.waves_per_block;
    switch (f) {
        case QG_FMT_FP4_E2M1: return qgl::launch_fp4(p, pl, batch, lds, stream);
        case QG_FMT_AFFINE_U4: return qgl::launch_affine_u4(p, pl, batch, lds, stream);
        case QG_FMT_AFFINE_U8: return qgl::launch_affine_u8(p, pl, batch, lds, stream);
        case QG_FMT_Q4K: return qgl::launch_q4k(p, pl, batch, lds, stream);
        default: return qgl::launch_fp8(p, pl, batch, lds, stream);
    }
}

Params base_params(qg_format f, const void *codes, const void *x, void *y, int64_t n, int64_t k,
                   qg_out_dtype out) {
    const FmtInfo fi = fmt_info(f);
    Params p{};
    p.codes = static_cast<const unsigned char *>(codes);
    p.x = static_cast<const uint16_t *>(x);
    p.y = y;
    p.n = n;
    p.k = int32_t(k);
    p.chunks = int32_t(k / fi.wpc);
    p.row_bytes = int64_t(p.chunks) * qg::kChunkBytes;
    p.passes = (p.chunks + qg::kWave - 1) / qg::kWave;
    p.out_bf16 = out == QG_OUT_BF16 ? 1 : 0;
    return p;
}

// Fused RMSNorm arguments (gamma == nullptr in the plain entry points).
struct Norm {
    const uint16_t *gamma;
    float eps;
};

qg_status set_norm(Params &p, const Norm *nm) {
    if (!nm) return QG_OK;
    if (!nm->gamma) return QG_ERR_NULL_POINTER;
    if (!aligned(nm->gamma, 16)) return QG_ERR_MISALIGNED;
    if (!(nm->eps >= 0.0f) || nm->eps > 3.0e38f) return QG_ERR_BAD_VALUE;   // NaN, negative or infinite
    p.gamma = nm->gamma;
    p.eps = nm->eps;
    p.norm = 1;
    return QG_OK;
}

qg_status fp4_entry(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, void *y, int64_t n,
                    int64_t k, int32_t group_size, int32_t batch, qg_out_dtype out, const qg_plan *plan,
                    const Norm *nm, hipStream_t stream) {
    qg_status st = check_common(QG_FMT_FP4_E2M1, codes, x, y, n, k, batch, out);
    if (st != QG_OK) return st;
    st = check_groups(scales, nullptr, false, k, group_size, qg::FmtFP4::kWpc);
    if (st != QG_OK) return st;
    if ((st = check_plan(plan)) != QG_OK) return st;
    Params p = base_params(QG_FMT_FP4_E2M1, codes, x, y, n, k, out);
    if ((st = set_norm(p, nm)) != QG_OK) return st;
    p.scales = scales;
    p.groups = int32_t(k / group_size);
    p.group_shift = log2i(group_size / qg::FmtFP4::kWpc);
    return run(QG_FMT_FP4_E2M1, p, batch, plan, stream);
}

qg_status affine_entry(qg_format f, const uint32_t *codes, const uint16_t *scales,
                       const uint16_t *biases, const uint16_t *x, void *y, int64_t n, int64_t k,
                       int32_t group_size, int32_t batch, qg_out_dtype out, const qg_plan *plan,
                       const Norm *nm, hipStream_t stream) {
    qg_status st = check_common(f, codes, x, y, n, k, batch, out);
    if (st != QG_OK) return st;
    st = check_groups(scales, biases, true, k, group_size, fmt_info(f).wpc);
    if (st != QG_OK) return st;
    if ((st = check_plan(plan)) != QG_OK) return st;
    Params p = base_params(f, codes, x, y, n, k, out);
    if ((st = set_norm(p, nm)) != QG_OK) return st;
    p.scales = scales;
    p.biases = biases;
    p.groups = int32_t(k / group_size);
    p.group_shift = log2i(group_size / fmt_info(f).wpc);
    return run(f, p, batch, plan, stream);
}

qg_status fp8_entry(const uint8_t *codes, const float *row_scale, const uint16_t *x, void *y, int64_t n,
                    int64_t k, int32_t batch, qg_out_dtype out, const qg_plan *plan, const Norm *nm,
                    hipStream_t stream) {
    qg_status st = check_common(QG_FMT_FP8_E4M3, codes, x, y, n, k, batch, out);
    if (st != QG_OK) return st;
    if (!row_scale) return QG_ERR_NULL_POINTER;
    if (!aligned(row_scale, 4)) return QG_ERR_MISALIGNED;
    if ((st = check_plan(plan)) != QG_OK) return st;
    Params p = base_params(QG_FMT_FP8_E4M3, codes, x, y, n, k, out);
    if ((st = set_norm(p, nm)) != QG_OK) return st;
    p.row_scale = row_scale;
    return run(QG_FMT_FP8_E4M3, p, batch, plan, stream);
}

qg_status q4k_entry(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                    void *y, int64_t n, int64_t k, int32_t batch, qg_out_dtype out, const qg_plan *plan,
                    const Norm *nm, hipStream_t stream) {
    qg_status st = check_common(QG_FMT_Q4K, codes, x, y, n, k, batch, out);
    if (st != QG_OK) return st;
    if (!sub || !super) return QG_ERR_NULL_POINTER;
    if (k % 256) return QG_ERR_BAD_SHAPE;
    if (!aligned(sub, 2) || !aligned(super, 4)) return QG_ERR_MISALIGNED;
    if ((st = check_plan(plan)) != QG_OK) return st;
    Params p = base_params(QG_FMT_Q4K, codes, x, y, n, k, out);
    if ((st = set_norm(p, nm)) != QG_OK) return st;
    p.scales = sub;
    p.biases = reinterpret_cast<const uint16_t *>(super);
    p.groups = int32_t(k / 32);                 // sub-blocks: one 16-byte chunk each
    p.group_shift = 0;
    return run(QG_FMT_Q4K, p, batch, plan, stream);
}

}  // namespace

namespace qgl {

namespace {
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];
}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(g_cu_once[dev], [dev] {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
        g_cu_count[dev] = v;
    });
    return g_cu_count[dev];
}

}  // namespace qgl

extern "C" {

qg_status qgemv_fp4_e2m1_plan(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                              void *y, int64_t n, int64_t k, int32_t group_size, int32_t batch,
                              qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream) {
    return fp4_entry(codes, scales, x, y, n, k, group_size, batch, out_dtype, plan, nullptr, stream);
}

qg_status qgemv_fp4_e2m1(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, void *y,
                         int64_t n, int64_t k, int32_t group_size, int32_t batch,
                         qg_out_dtype out_dtype, hipStream_t stream) {
    return fp4_entry(codes, scales, x, y, n, k, group_size, batch, out_dtype, nullptr, nullptr, stream);
}

qg_status qgemv_fp4_e2m1_rmsnorm(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                                 const uint16_t *gamma, float eps, void *y, int64_t n, int64_t k,
                                 int32_t group_size, int32_t batch, qg_out_dtype out_dtype,
                                 const qg_plan *plan, hipStream_t stream) {
    const Norm nm{gamma, eps};
    return fp4_entry(codes, scales, x, y, n, k, group_size, batch, out_dtype, plan, &nm, stream);
}

qg_status qgemv_affine_u4_plan(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                               const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                               int32_t batch, qg_out_dtype out_dtype, const qg_plan *plan,
                               hipStream_t stream) {
    return affine_entry(QG_FMT_AFFINE_U4, codes, scales, biases, x, y, n, k, group_size, batch,
                        out_dtype, plan, nullptr, stream);
}

qg_status qgemv_affine_u4(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                          const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                          int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    return affine_entry(QG_FMT_AFFINE_U4, codes, scales, biases, x, y, n, k, group_size, batch,
                        out_dtype, nullptr, nullptr, stream);
}

qg_status qgemv_affine_u4_rmsnorm(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                  const uint16_t *x, const uint16_t *gamma, float eps, void *y,
                                  int64_t n, int64_t k, int32_t group_size, int32_t batch,
                                  qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream) {
    const Norm nm{gamma, eps};
    return affine_entry(QG_FMT_AFFINE_U4, codes, scales, biases, x, y, n, k, group_size, batch,
                        out_dtype, plan, &nm, stream);
}

qg_status qgemv_affine_u8_plan(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                               const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                               int32_t batch, qg_out_dtype out_dtype, const qg_plan *plan,
                               hipStream_t stream) {
    return affine_entry(QG_FMT_AFFINE_U8, codes, scales, biases, x, y, n, k, group_size, batch,
                        out_dtype, plan, nullptr, stream);
}

qg_status qgemv_affine_u8(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                          const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                          int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    return affine_entry(QG_FMT_AFFINE_U8, codes, scales, biases, x, y, n, k, group_size, batch,
                        out_dtype, nullptr, nullptr, stream);
}

qg_status qgemv_affine_u8_rmsnorm(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                  const uint16_t *x, const uint16_t *gamma, float eps, void *y,
                                  int64_t n, int64_t k, int32_t group_size, int32_t batch,
                                  qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream) {
    const Norm nm{gamma, eps};
    return affine_entry(QG_FMT_AFFINE_U8, codes, scales, biases, x, y, n, k, group_size, batch,
                        out_dtype, plan, &nm, stream);
}

qg_status qgemv_fp8_e4m3_plan(const uint8_t *codes, const float *row_scale, const uint16_t *x,
                              void *y, int64_t n, int64_t k, int32_t batch, qg_out_dtype out_dtype,
                              const qg_plan *plan, hipStream_t stream) {
    return fp8_entry(codes, row_scale, x, y, n, k, batch, out_dtype, plan, nullptr, stream);
}

qg_status qgemv_fp8_e4m3(const uint8_t *codes, const float *row_scale, const uint16_t *x, void *y,
                         int64_t n, int64_t k, int32_t batch, qg_out_dtype out_dtype,
                         hipStream_t stream) {
    return fp8_entry(codes, row_scale, x, y, n, k, batch, out_dtype, nullptr, nullptr, stream);
}

qg_status qgemv_fp8_e4m3_rmsnorm(const uint8_t *codes, const float *row_scale, const uint16_t *x,
                                 const uint16_t *gamma, float eps, void *y, int64_t n, int64_t k,
                                 int32_t batch, qg_out_dtype out_dtype, const qg_plan *plan,
                                 hipStream_t stream) {
    const Norm nm{gamma, eps};
    return fp8_entry(codes, row_scale, x, y, n, k, batch, out_dtype, plan, &nm, stream);
}

qg_status qgemv_q4k(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                    void *y, int64_t n, int64_t k, int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    return q4k_entry(codes, sub, super, x, y, n, k, batch, out_dtype, nullptr, nullptr, stream);
}

qg_status qgemv_q4k_plan(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                         void *y, int64_t n, int64_t k, int32_t batch, qg_out_dtype out_dtype,
                         const qg_plan *plan, hipStream_t stream) {
    return q4k_entry(codes, sub, super, x, y, n, k, batch, out_dtype, plan, nullptr, stream);
}

qg_status qgemv_q4k_rmsnorm(const uint32_t *codes, const uint16_t *sub, const uint32_t *super, const uint16_t *x,
                            const uint16_t *gamma, float eps, void *y, int64_t n, int64_t k, int32_t batch,
                            qg_out_dtype out_dtype, const qg_plan *plan, hipStream_t stream) {
    const Norm nm{gamma, eps};
    return q4k_entry(codes, sub, super, x, y, n, k, batch, out_dtype, plan, &nm, stream);
}

qg_status qg_rmsnorm_bf16(const uint16_t *x, const uint16_t *gamma, float eps, uint16_t *out, int64_t k,
                          int32_t batch, hipStream_t stream) {
    if (!x || !gamma || !out) return QG_ERR_NULL_POINTER;
    if (k < 8 || k % 8 || k > (int64_t(1) << 30)) return QG_ERR_BAD_SHAPE;
    if (batch < 1 || batch > 4) return QG_ERR_BAD_BATCH;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(out, 16)) return QG_ERR_MISALIGNED;
    Params p{};
    p.x = x;
    p.k = int32_t(k);
    const Norm nm{gamma, eps};
    qg_status st = set_norm(p, &nm);
    if (st != QG_OK) return st;
    // one workgroup of 8 waves per batch row (eight loading waves take up to
    // k = 16384 in one round of loads: k = 15360 2.89 us against 3.72 with 4
    // waves); x and gamma stay in LDS when they fit in 64 KiB with the group
    // sums
    const int64_t sums = qg::rmsnorm_sums_bytes(k);
    if (sums > 64 * 1024) return QG_ERR_TOO_LARGE;      // k > 2^23
    if (sums + 4 * k <= 64 * 1024)
        return qgl::launch_kernel(qg::qg_rmsnorm_kernel<true>, dim3(batch), dim3(512), size_t(sums + 4 * k), stream,
                                  p, out);
    return qgl::launch_kernel(qg::qg_rmsnorm_kernel<false>, dim3(batch), dim3(512), size_t(sums), stream, p, out);
}

qg_status qg_plan_query(qg_format format, int64_t n, int64_t k, int32_t batch, qg_plan *out) {
    if (!out) return QG_ERR_NULL_POINTER;
    if (format < QG_FMT_FP4_E2M1 || format > QG_FMT_Q4K) return QG_ERR_BAD_DTYPE;
    if (n < 1 || k < 1 || k % fmt_info(format).wpc) return QG_ERR_BAD_SHAPE;
    if (batch < 1 || batch > 4) return QG_ERR_BAD_BATCH;
    int cus = 0;
    qg_status st = device_cus(&cus);
    if (st != QG_OK) return st;
    // the format's usual group size, aligned parameter arrays
    Params p = base_params(format, nullptr, nullptr, nullptr, n, k, QG_OUT_F32);
    const int gs = format == QG_FMT_FP4_E2M1 || format == QG_FMT_Q4K ? 32 : (format == QG_FMT_FP8_E4M3 ? 0 : 64);
    p.groups = gs ? int32_t(k / gs) : 0;
    p.group_shift = gs ? log2i(gs / fmt_info(format).wpc) : 0;
    p.scales = p.biases = reinterpret_cast<const uint16_t *>(uintptr_t(256));
    if (batch >= qg::kM4MinBatch && mfma4_takes(format, p)) {
        p.passes = (p.chunks + qg::kM4Slots - 1) / qg::kM4Slots;
        const Plan pl = mfma4_plan(p, cus, nullptr);
        out->rows_per_tile = pl.rows_per_tile;
        out->waves_per_block = pl.waves_per_block;
        out->blocks = pl.blocks;
        return QG_OK;
    }
    if (format == QG_FMT_FP8_E4M3 && batch >= qg::kFp8MfmaMinBatch && fp8_mfma_takes(p)) {
        p.passes = (p.chunks + qg::kFp8Slots - 1) / qg::kFp8Slots;
        const Plan pl = fp8_default_plan(p, cus);
        out->rows_per_tile = pl.rows_per_tile;
        out->waves_per_block = pl.waves_per_block;
        out->blocks = pl.blocks;
        return QG_OK;
    }
    const Split sp = split_of(format, p);
    p.segs = sp.ok ? sp.segs : 0;
    p.passes = sp.ok ? sp.passes : passes_of(p.chunks);
    Plan pl = default_plan(format, p, batch, cus);
    if (pl.row_kernel)
        while (pl.rows_per_tile > 1 && !row_instance_for(format, pl.rows_per_tile, batch, pl.passes))
            pl.rows_per_tile /= 2;
    out->rows_per_tile = pl.rows_per_tile;
    out->waves_per_block = pl.waves_per_block;
    out->blocks = pl.blocks;
    return QG_OK;
}

const char *qg_status_string(qg_status status) {
    switch (status) {
        case QG_OK: return "ok";
        case QG_ERR_NULL_POINTER: return "a required pointer is null";
        case QG_ERR_BAD_SHAPE: return "bad shape (n, k, or k not a whole number of 16-byte code chunks)";
        case QG_ERR_BAD_GROUP_SIZE: return "group_size must be 32, 64 or 128 and divide k";
        case QG_ERR_MISALIGNED: return "a pointer is not aligned (codes and x: 16 bytes)";
        case QG_ERR_BAD_BATCH: return "batch must be 1..4";
        case QG_ERR_BAD_DTYPE: return "unknown output dtype or format";
        case QG_ERR_BAD_BITS: return "bits must be 4 or 8";
        case QG_ERR_BAD_VALUE: return "non-finite weight, out-of-range code, or eps negative or not finite";
        case QG_ERR_TOO_LARGE: return "the activations exceed the LDS staging limit of this call";
        case QG_ERR_DEVICE: return "no usable HIP device";
        case QG_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int qg_abi_version(void) { return QG_ABI_VERSION; }

qg_status qg_stream_probe(const void *buf, int64_t bytes, int32_t pattern, int32_t unroll,
                          int32_t blocks, int32_t threads_per_block, uint32_t *out, hipStream_t stream) {
    if (!buf || !out) return QG_ERR_NULL_POINTER;
    if (bytes < 16 || bytes % 16) return QG_ERR_BAD_SHAPE;
    if (pattern < 0 || pattern > 5) return QG_ERR_BAD_SHAPE;
    if (pattern % 3 == 2 && unroll < 2) return QG_ERR_BAD_SHAPE;
    if (blocks < 1 || threads_per_block < 64 || threads_per_block > 1024 || threads_per_block % 64)
        return QG_ERR_BAD_SHAPE;
    if (!aligned(buf, 16) || !aligned(out, 4)) return QG_ERR_MISALIGNED;
    const auto *b = static_cast<const uint4 *>(buf);
    const int64_t units = bytes / 16;
    const dim3 g(blocks), t(threads_per_block);
    switch (unroll) {
        case 1: return qgl::launch_kernel(qg::stream_probe_kernel<1>, g, t, 0, stream, b, units, pattern, out);
        case 2: return qgl::launch_kernel(qg::stream_probe_kernel<2>, g, t, 0, stream, b, units, pattern, out);
        case 4: return qgl::launch_kernel(qg::stream_probe_kernel<4>, g, t, 0, stream, b, units, pattern, out);
        case 8: return qgl::launch_kernel(qg::stream_probe_kernel<8>, g, t, 0, stream, b, units, pattern, out);
        case 16: return qgl::launch_kernel(qg::stream_probe_kernel<16>, g, t, 0, stream, b, units, pattern, out);
        default: return QG_ERR_BAD_SHAPE;
    }
}


}  // extern "C"
