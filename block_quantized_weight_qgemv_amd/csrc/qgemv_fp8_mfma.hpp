// FP8-E4M3 matvec on gfx950's 4x4x4 bf16 matrix blocks.
//
// "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus (Part 2)",
// section "The assumption that failed the profiler", describes the FP8
// lm_head matvec as one multiply-add per weight byte with the row scale
// applied once.  On the vector ALU that costs a conversion per two codes plus
// one two-wide dot per code pair and batch row: at four batch rows about 2.5
// instructions per weight, enough to fall behind the 8 TB/s weight stream.
// Here the multiply-adds run on the matrix cores instead.
//
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4x4 blocks D = A*B + C
// with 4 terms each.  Lane l supplies row (l & 3) of block (l >> 2)'s A and
// column (l & 3) of its B, and receives column (l & 3) of its D, row i in
// element i.  So a wave streams a tile of 4 weight rows: lane l loads 16-byte
// chunks of row (l & 3), chunk slot s = l >> 2 taking chunks s, s + 16, ...
// (each load instruction reads 256 consecutive bytes of each of the 4 rows),
// decodes them to bf16 with the scaled FP8 conversion (scale 1: exact), and
// feeds them as A, four columns per block; B is the same four columns of
// batch row (l & 3) of x, read from LDS.  Block s then accumulates, for every
// pair (tile row, batch row), the products of the columns in slot s.  Batch
// rows past the batch repeat the last one (their columns are never read).
//
// Each lane chains its blocks' products over the tile's passes in two
// accumulators (even and odd column quads); at the tile's end the 16 slots
// are added over the wave (DPP rotations inside each 16-lane row, then
// permlane swaps across rows) and lanes 0..3 write the 4 rows of y for batch
// rows 0..3, times the row scale.  The order of every addition is fixed by k
// alone: not by the tile, the wavefront, the launch shape or the batch size.
//
// Steps: a tile's passes (ceil(chunks / 16)) are cut into steps of PS passes,
// each one buffer of loads; loads run D steps ahead.  Rows of at most 16
// passes (k <= 4096) are one or two steps of 8 passes, a compile-time shape
// (kH): each lane's slice of x is then the same for every tile and is read
// from LDS into registers once.  Longer rows take steps of 4, 8 or 16 passes
// and read x from LDS pass by pass.  Chunks past the row end read zeros
// through the buffer resource and take x from zero units in LDS.
#pragma once

#include "qgemv_common.hpp"

namespace qg {

typedef short mfma_i16x4_t __attribute__((ext_vector_type(4)));
typedef float mfma_f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFp8TileRows = 4;        // weight rows per tile (the blocks' rows)
constexpr int kFp8Slots = 16;          // chunk slots per pass (the blocks)
constexpr int kFp8ChunksPerWave = 16;  // shared tiles are handed out in about 16 chunks per wave

// Smallest batch the FP8 matvec runs on the matrix cores.  The 4-row tiles
// read x from LDS and 4-row interleaved weight lines, which costs ~2% of the
// stream at one or two activation rows; the row kernel's vector dot then
// costs less.  From three rows on, its per-row dot instructions cost more
// (measured on the 262144 x 3840 lm_head, us per matvec, batch 1..4: row
// kernel 146.3, 148.6, 159.9, 166.0; this kernel 149.9, 152.2, 153.9, 156.7).
constexpr int kFp8MfmaMinBatch = 3;

// Rows of at most 16 passes: halves (steps of 8 passes) per tile, x in
// registers; 0 for longer rows.
__host__ __device__ constexpr int fp8_mfma_halves(int chunks) {
    const int passes = (chunks + kFp8Slots - 1) / kFp8Slots;
    return passes <= 8 ? 1 : (passes <= 16 ? 2 : 0);
}

// Passes per step of a longer row: 4, 8 or 16, whichever pads its passes the
// least (the larger on a tie).  Depends on the number of chunks alone.
__host__ __device__ constexpr int fp8_mfma_step_passes(int chunks) {
    const int passes = (chunks + kFp8Slots - 1) / kFp8Slots;
    int best = 16, best_pad = ((passes + 15) / 16) * 16 - passes;
    for (int ps = 8; ps >= 4; ps /= 2) {
        const int pad = ((passes + ps - 1) / ps) * ps - passes;
        if (pad < best_pad) {
            best = ps;
            best_pad = pad;
        }
    }
    return best;
}

__host__ __device__ constexpr int fp8_mfma_depth(int ps) { return ps == 16 ? 2 : (ps == 8 ? 3 : 4); }

// x in LDS, in 16-byte units: the first halves of every chunk's activations
// ([chunk][batch row]), a zero unit, the second halves, a zero unit.  Lane
// 4s + j reads unit c * B + j of each half: lanes of one slot read neighbouring
// units and the slots follow each other, so the reads are free of bank
// conflicts (with one batch row, lanes of one slot read the same unit).
// Chunks past the row end read the zero units.  Bytes: 2 * B * k + 32.
struct Fp8XLayout {
    int B, R;     // R = chunks * B units per half
    __device__ int operator()(int b, int u, int) const { return (u & 1) * (R + 1) + (u >> 1) * B + b; }
};

__device__ __forceinline__ float mfma_row_sum(float v) {
    // slots inside each 16-lane row: lanes l, l+4, l+8, l+12 (mod 16)
    v = v + dpp_f<0x124>(v);    // row_ror:4
    v = v + dpp_f<0x128>(v);    // row_ror:8
    // across the four rows
    float a = v, b = v;
    swap16(a, b);
    v = a + b;
    a = v;
    b = v;
    swap32(a, b);
    return a + b;
}

// kH > 0: rows of kH steps of PS = 8 passes, x in registers, D = 2 buffers
// (with kH = 2, buffer h always holds half h of a tile).  kH = 0: rows of
// any length, x read from LDS pass by pass.
template <int B, int PS, int D, bool kNorm, int kH>
__global__ void __launch_bounds__(512) qgemv_fp8_mfma_kernel(const Params p) {
    constexpr bool kXReg = kH > 0;
    static_assert(!kXReg || (PS == 8 && D == 2), "register-x shapes: steps of 8 passes, two buffers");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int ri = lane & 3;                  // A: tile row; B, D: batch column
    const int slot = lane >> 2;               // the lane's block: chunk slot
    const int jb = ri < B ? ri : B - 1;       // batch row this lane's B column carries

    // Tiles are whole groups of 4 rows from row 0, split evenly over the
    // workgroups.  A wave's work is a sequence of items in increasing order
    // (an item at or past n_items stands for "nothing": its loads read no
    // memory):
    //  * kH > 0, with room in LDS for a counter (p.counter_offset): items are
    //    the workgroup's tiles, cut into chunks of C consecutive tiles; wave w
    //    starts with chunk w and later chunks come from the counter, first
    //    come first served (the waves of a workgroup are served unevenly by
    //    the memory system; this way they finish together);
    //  * kH > 0 otherwise: the tiles of a contiguous range per wave;
    //  * kH = 0: the steps of a contiguous range of tiles per wave.
    const int64_t tiles_all = (p.n + kFp8TileRows - 1) / kFp8TileRows;
    const int nb = gridDim.x;
    const int64_t blk = logical_block();
    const int64_t t_begin = blk * tiles_all / nb, t_end = (blk + 1) * tiles_all / nb;
    const int T = int(t_end - t_begin);
    const int W = blockDim.x >> 6;
    const int w = wave_in_block();
    const int64_t tb = t_begin + int64_t(w) * T / W;
    const int64_t te = t_begin + int64_t(w + 1) * T / W;
    const int passes = p.passes;                              // ceil(chunks / 16)
    const int G = kXReg ? kH : (passes + PS - 1) / PS;        // steps per tile
    const bool shared = kXReg && p.counter_offset != 0;       // uniform
    const int n_items = shared ? T : int(te - tb) * (kXReg ? 1 : G);
    const int C = max(1, T / (kFp8ChunksPerWave * W));        // tiles per shared chunk
    unsigned *counter = reinterpret_cast<unsigned *>(smem + p.counter_offset);
    int chunk = w, cur = w * C;
    // the next shared tile (uniform; the counter is first used after the
    // barrier that follows its initialization: a chunk holds at least one tile)
    auto next_tile = [&]() __attribute__((always_inline)) -> int {
        const bool at_end = cur < T && cur == (chunk + 1) * C;
        unsigned v = 0;
        if (at_end && lane == 0) v = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        chunk = __builtin_amdgcn_readfirstlane(at_end ? int(v) : chunk);
        cur = at_end ? chunk * C : cur;
        const int t = min(cur, T);
        cur = __builtin_amdgcn_readfirstlane(cur < T ? cur + 1 : cur);
        return __builtin_amdgcn_readfirstlane(t);
    };
    // first row of an item's tile, and its step within the tile (kH > 0:
    // the step is the buffer's half, given)
    auto locate = [&](int item, int half, int64_t &row0, int &g) __attribute__((always_inline)) {
        if (kXReg) {
            row0 = ((shared ? t_begin : tb) + item) * kFp8TileRows;
            g = half;
        } else {
            const int tq = item / G;
            g = item - tq * G;
            row0 = (tb + tq) * kFp8TileRows;
        }
    };
    // the buffer a ring slot's half is (kH = 2: slot d holds half d)
    auto half_of = [](int d) { return kH == 2 ? d : 0; };

    struct Buf {
        uint4 c[PS];
        uint32_t rs;       // row scale of tile row (lane >> 2) & 3
    };
    const uint32_t row_bytes = uint32_t(p.row_bytes);
    auto issue = [&](Buf &bf, int item_in, int half) __attribute__((always_inline)) {
        const int item = __builtin_amdgcn_readfirstlane(item_in);
        int64_t row0;
        int g;
        locate(item, half, row0, g);
        const int64_t valid = item < n_items ? min(int64_t(kFp8TileRows), p.n - row0) : 0;
        const int64_t rb = valid ? row0 : 0;
        const rsrc_t rc = make_rsrc(p.codes + rb * p.row_bytes, uint32_t(valid) * row_bytes);
#pragma unroll
        for (int q = 0; q < PS; ++q) {
            const int c = slot + kFp8Slots * (g * PS + q);
            bf.c[q] = buffer_code_chunk(rc, c < p.chunks ? uint32_t(ri) * row_bytes + uint32_t(c) * kChunkBytes
                                                         : kOutOfRange);
        }
        const rsrc_t rr = make_rsrc(p.row_scale + rb, uint32_t(valid) * 4u);
        bf.rs = __builtin_amdgcn_raw_buffer_load_b32(rr, int(((lane >> 2) & 3) * 4), 0, kCacheNonTemporal);
    };

    // ---- x into LDS (Fp8XLayout).
    // The activation loads go out first, then the first step of weights, and
    // the wave waits for the activations alone (loads retire in order), so
    // the weight stream starts before x has arrived.  When x is larger than
    // kXu units per thread it is staged before any weight load.
    uint4 *xlds = reinterpret_cast<uint4 *>(smem);
    const int upr = p.k / 8;                                  // 16-byte units per batch row
    const int x_units = B * upr;
    const Fp8XLayout xl{B, p.chunks * B};
    auto xpos = [&](int u) {                                  // unit u of x [B][k/8] in LDS
        const int b = row_of<B>(u, upr);
        return xl(b, u - b * upr, upr);
    };
    // LDS unit of the first half of the activations of pass gq (the second
    // half is R + 1 units further)
    auto x_at = [&](int gq) {
        const int c = slot + kFp8Slots * gq;
        return c < p.chunks ? c * B + jb : xl.R;
    };
    constexpr int kStepLoads = PS + 1;
    Buf buf[D];
    int sl[D];
    sl[0] = shared ? next_tile() : 0;
    if (shared && threadIdx.x == 0) *counter = unsigned(W);       // the next chunk to hand out
    if constexpr (kNorm) {
        float rn[B];
        // gamma is copied to LDS with the norm's loads where the host found
        // room for it; the normalization then reads each gamma unit once and
        // applies it to that unit of every batch row (with one load from
        // memory per unit of x, each queued behind the first weight step, the
        // batch-4 fused lm_head took 2.7 us more than the plain call; 2.2 now)
        uint4 *glds = p.gamma_offset ? reinterpret_cast<uint4 *>(smem + p.gamma_offset) : nullptr;
        block_rms<B>(p, reinterpret_cast<float *>(smem + p.norm_offset), rn, xlds, glds, [&] {
            issue(buf[0], sl[0], half_of(0));
            wait_vm_loads<kStepLoads>();
        }, xl);
        for (int base = 0; base < upr; base += blockDim.x) {
            const int gu_in = base + int(threadIdx.x);
            const int gu = min(gu_in, upr - 1);
            const uint4 gv = glds ? glds[gu] : load_x_unit(p.gamma + int64_t(gu) * 8);
            if (gu_in < upr) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int i = xl(b, gu, upr);
                    xlds[i] = norm_unit(xlds[i], gv, rn[b]);
                }
            }
        }
    } else {
        constexpr int kXu = 4;
        const bool few = x_units <= kXu * int(blockDim.x);    // uniform
        uint4 xr[kXu];
        if (few) {
#pragma unroll
            for (int i = 0; i < kXu; ++i)
                xr[i] = load_x_unit(p.x + int64_t(min(int(threadIdx.x) + i * int(blockDim.x), x_units - 1)) * 8);
        }
        issue(buf[0], sl[0], half_of(0));
        if (few) {
            wait_vm_loads<kStepLoads>();
#pragma unroll
            for (int i = 0; i < kXu; ++i) {
                const int u = int(threadIdx.x) + i * int(blockDim.x);
                if (u < x_units) xlds[xpos(u)] = xr[i];
            }
        } else {
            for (int u = threadIdx.x; u < x_units; u += blockDim.x) xlds[xpos(u)] = load_x_unit(p.x + int64_t(u) * 8);
        }
    }
    if (threadIdx.x < 2) xlds[threadIdx.x * (xl.R + 1) + xl.R] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
#pragma unroll
    for (int d = 1; d < D; ++d) {
        sl[d] = kH == 2 ? sl[0] : (shared ? next_tile() : d);
        issue(buf[d], sl[d], half_of(d));
    }
    issue_fence();
    // the lane's slice of x for every pass of a tile (kH > 0)
    constexpr int kXr = kXReg ? kH * PS : 1;
    uint4 xreg[kXr][2];
    if constexpr (kXReg) {
#pragma unroll
        for (int gq = 0; gq < kXr; ++gq) {
            const int a = x_at(gq);
            xreg[gq][0] = xlds[a];
            xreg[gq][1] = xlds[a + xl.R + 1];
        }
    }

    mfma_f32x4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto mul_pass = [&](const uint4 cq, const uint4 x0, const uint4 x1) __attribute__((always_inline)) {
        const uint32_t xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const uint32_t wv[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[m], 1.0f, false);
            const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[m], 1.0f, true);
            const u32x2_t a2 = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            const u32x2_t b2 = {xv[2 * m], xv[2 * m + 1]};
            const mfma_i16x4_t a = __builtin_bit_cast(mfma_i16x4_t, a2);
            const mfma_i16x4_t bx = __builtin_bit_cast(mfma_i16x4_t, b2);
            if (m & 1)
                acc1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, bx, acc1, 0, 0, 0);
            else
                acc0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, bx, acc0, 0, 0, 0);
        }
    };
    auto consume = [&](const Buf &bf, int item, int half) __attribute__((always_inline)) {
        int64_t row0;
        int g;
        locate(item, half, row0, g);
        if constexpr (kXReg) {
#pragma unroll
            for (int q = 0; q < PS; ++q) mul_pass(bf.c[q], xreg[half * PS + q][0], xreg[half * PS + q][1]);
        } else {
            // x of pass q + 1 is read from LDS before pass q is multiplied
            int a = x_at(g * PS);
            uint4 xn0 = xlds[a], xn1 = xlds[a + xl.R + 1];
#pragma unroll
            for (int q = 0; q < PS; ++q) {
                const uint4 x0 = xn0, x1 = xn1;
                if (q + 1 < PS) {
                    a = x_at(g * PS + q + 1);
                    xn0 = xlds[a];
                    xn1 = xlds[a + xl.R + 1];
                    // keep these reads ahead of this pass's work (the scheduler
                    // would otherwise sink them to their use and expose their latency)
                    __builtin_amdgcn_sched_barrier(0);
                }
                mul_pass(bf.c[q], x0, x1);
            }
        }
        if (g == G - 1) {
            float tot[kFp8TileRows];
#pragma unroll
            for (int i = 0; i < kFp8TileRows; ++i) tot[i] = mfma_row_sum(acc0[i] + acc1[i]);
            float rsv[kFp8TileRows];
#pragma unroll
            for (int i = 0; i < kFp8TileRows; ++i)
                rsv[i] = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(bf.rs), 4 * i)));
            if (lane < B) {
#pragma unroll
                for (int i = 0; i < kFp8TileRows; ++i)
                    if (row0 + i < p.n) store_y(p, lane, row0 + i, tot[i] * rsv[i]);
            }
            acc0 = mfma_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            acc1 = mfma_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    // Buffers hold items in increasing order (kH = 2: both buffers the same
    // tile); the loop runs while the last one holds an item (then all do),
    // each buffer is refilled right after it is consumed (refills past the
    // end read nothing from memory), and the loop's only exit is its test at
    // the top.
    auto advance = [&](int d) __attribute__((always_inline)) -> int {
        if constexpr (kH == 2) return d == 0 ? (shared ? next_tile() : sl[0] + 1) : sl[0];
        return shared ? next_tile() : sl[d] + D;
    };
    // (The scheduling barriers keep each buffer's work in its place: hoisted
    // into the previous buffer's passes, the next buffer's tile-end reads
    // made the wait there cover every load in flight.)
    while (sl[D - 1] < n_items) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int nx = advance(d);
            consume(buf[d], sl[d], half_of(d));
            sl[d] = nx;
            issue(buf[d], nx, half_of(d));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (sl[d] < n_items) consume(buf[d], sl[d], half_of(d));
    wait_vm_loads<0>();
}

}  // namespace qg
