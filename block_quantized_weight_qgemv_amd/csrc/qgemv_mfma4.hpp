// 4-bit group-scaled matvec at three or four activation rows on gfx950's
// 4x4x4 bf16 matrix blocks (FP4-E2M1, affine u4, the two-level super-block
// format).
//
// On the vector ALU every batch row costs one two-wide dot per code pair: at
// four rows about 2.6 instructions per weight, enough to fall far behind the
// weight stream (the 30720 x 3840 FP4 matvec takes 1.7x its batch-1 time).
// Here the products run on v_mfma_f32_4x4x4_16b_bf16, as the FP8 kernel does
// (qgemv_fp8_mfma.hpp), and only the decode and the per-group scale fold stay
// on the vector ALU.
//
// A wave streams tiles of 4 weight rows.  Lane l = 4s + i loads 16-byte
// chunks of tile row i, chunk slot s taking chunks s, s + 16, ... (each load
// instruction reads 256 consecutive bytes of each of the 4 rows).  A chunk is
// 32 weights: decoded to bf16 pairs in registers (the format's decode, exact),
// it feeds 8 blocks of 4 columns as B; A is the same 4 columns of the 4 batch
// rows of x, read from LDS.  Block s accumulates the chunk's products in one
// chain of 8 steps; its result column i is the chunk's raw dot of tile row i
// with every batch row, in the lane that loaded row i, which folds its own
// group's parameters once per chunk: acc[b] += scale * raw[b] (+ bias *
// sum_x[b] for affine).  At a step's end the 16 slots are added over the
// wave and lanes 0..3 write tile row (lane) of every batch row.  Batch rows
// past the batch repeat the last one and are never written.
//
// The order of every addition is fixed by the format and k alone (chunk
// order per slot within a step, a fixed tree over slots, then the steps in
// order): not by the tile, the wave, the launch shape or the batch size (3
// or 4).  It is not the vector
// kernels' order, so a row's bits at batch 3-4 differ from its bits at batch
// 1-2; both meet the same bound.
//
// A tile's passes (ceil(chunks / 16)) are cut into steps of PS passes, one
// buffer of loads each, D steps in flight.  The steps of the workgroup's
// tiles are its work items, a contiguous range per wave; a step ends with its
// own sum over the slots, and a tile of several steps has them added in LDS
// in step order (split-K over the waves; the split is fixed by k).  x is
// staged once per workgroup in LDS in four
// quarters (unit q of every chunk's activations, [chunk][batch row]) plus a
// zero unit each, so lanes of one pass read neighbouring 16-byte units; the
// affine formats also stage each chunk's activation sums.
//
// Prior art, not the blueprint: "Hand-Writing Gemma 4 Flash-Decoding + an FP4
// Matvec Bonus (Part 2)", section "The assumption that failed the profiler"
// (the group scale folded out of the per-weight math, one multiply-add per
// group).
#pragma once

#include "qgemv_common.hpp"
#include "qgemv_formats.hpp"
#include "qgemv_fp8_mfma.hpp"

namespace qg {

constexpr int kM4Rows = 4;        // weight rows per tile (the blocks' rows)
constexpr int kM4Slots = 16;      // chunk slots per pass (the blocks)
constexpr int kM4MinBatch = 3;    // smallest batch that takes this kernel

// Passes per step and steps in flight per wave.  Each wave then has about
// 8 KiB of weights in flight and, on the large matrices, several times that
// in work items: deeper or longer steps put most of a wave's weights in
// flight at the start, and their decode and products then queue behind the
// stream's end instead of overlapping it (measured: 4 passes and 2 steps
// beat 8 and 3, 8 and 2, 4 and 4, 4 and 3, 2 and 2 to 4, on the 30720 x
// 3840 and 3840 x 15360 matrices).
constexpr int kM4StepPasses = 4;
constexpr int kM4Depth = 2;

// x in LDS, pass by pass: the activations of pass gq (chunks 16 gq .. 16 gq
// + 15) as [quarter][slot][batch row] units, quarter q holding columns 8q ..
// 8q + 7 of each chunk, so one quarter of a pass is 16 B consecutive units
// (a lane's 4 reads are 16 B units apart, and the lanes of one read take
// neighbouring units).  The chunks past the row end and one whole pass after
// the last are zero (steps past a tile's passes read that pass).  The
// affine formats also keep each chunk's activation sums, [chunk][4 batch
// rows] floats, zero past the row end.  The split-K partials ([tile row]
// [step][batch row] floats) follow.
__host__ __device__ constexpr int64_t mfma4_x_chunks(int64_t chunks) {
    return ((chunks + kM4Slots - 1) / kM4Slots + 1) * kM4Slots;
}
__host__ __device__ constexpr int64_t mfma4_lds_bytes(int64_t chunks, int64_t batch, bool sums) {
    return mfma4_x_chunks(chunks) * 4 * batch * 16 + (sums ? mfma4_x_chunks(chunks) * 16 : 0);
}

// LDS unit of unit u (8 columns) of batch row b
struct M4XLayout {
    int nb;               // batch rows
    __device__ int operator()(int b, int u, int) const {
        const int c = u >> 2;
        return (((c >> 4) * 4 + (u & 3)) * kM4Slots + (c & 15)) * nb + b;
    }
};

// Value of lane 4 * (lane / 4) + I (DPP quad broadcast).
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
    return dpp_f<I | (I << 2) | (I << 4) | (I << 6)>(v);
}

template <class Fmt, int B, bool kNorm>
__global__ void __launch_bounds__(512) qgemv_mfma4_kernel(const Params p) {
    constexpr int PS = kM4StepPasses, D = kM4Depth;
    static_assert(Fmt::kWpc == 32 && Fmt::kRawUnits == 4 && Fmt::kPpu == 1, "16-byte chunks of 32 weights");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr bool kSums = Fmt::kSums;
    const int lane = threadIdx.x & (kWave - 1);
    const int ri = lane & 3;                  // A: tile row; B, D: batch column
    const int slot = lane >> 2;               // the lane's block: chunk slot
    const int jb = ri < B ? ri : B - 1;       // batch row this lane's B column carries

    // Tiles of 4 rows from row 0, split evenly over the workgroups.  A
    // workgroup's work is its tiles' steps, items (tile, step) in tile-major
    // order, cut into one contiguous range per wave (an item at or past the
    // wave's end stands for "nothing": its loads read no memory).  A step's
    // sums go to LDS when a tile has several steps (split-K over the
    // workgroup's waves) and are added in step order at the end.
    const int64_t tiles_all = (p.n + kM4Rows - 1) / kM4Rows;
    const int nb = gridDim.x;
    const int64_t blk = logical_block();
    const int64_t t_begin = blk * tiles_all / nb, t_end = (blk + 1) * tiles_all / nb;
    const int T = int(t_end - t_begin);
    const int W = blockDim.x >> 6;
    const int w = wave_in_block();
    const int passes = p.passes;                              // ceil(chunks / 16)
    const int G = (passes + PS - 1) / PS;                     // steps per tile
    const int I = T * G;                                      // the workgroup's items
    const int i_begin = int(int64_t(w) * I / W), i_end = int(int64_t(w + 1) * I / W);
    const int n_items = i_end;
    auto locate = [&](int item, int64_t &row0, int &g) __attribute__((always_inline)) {
        const int tq = item / G;
        g = item - tq * G;
        row0 = (t_begin + tq) * kM4Rows;
    };

    struct Buf {
        uint4 c[PS];
        uint32_t a0[PS];      // this lane's row: scale (FP4, affine) or sub-block factors
        uint32_t a1[PS];      // bias (affine) or super-block word
    };
    const uint32_t row_bytes = uint32_t(p.row_bytes);
    const int sgroups = p.groups >> 3;
    // The group parameters are read with the default cache policy: a step's
    // 2-byte loads of a row touch part of a 128-byte line whose rest the next
    // step reads, and non-temporal loads let it be fetched again.
    constexpr int kParamCache = 0;
    auto issue = [&](Buf &bf, int item_in) __attribute__((always_inline)) {
        const int item = __builtin_amdgcn_readfirstlane(item_in);
        int64_t row0;
        int g;
        locate(item, row0, g);
        const int64_t valid = item < n_items ? min(int64_t(kM4Rows), p.n - row0) : 0;
        const int64_t rb = valid ? row0 : 0;
        const rsrc_t rc = make_rsrc(p.codes + rb * p.row_bytes, uint32_t(valid) * row_bytes);
        const rsrc_t rs = make_rsrc(p.scales + rb * p.groups, uint32_t(valid * p.groups * 2));
        const rsrc_t rbias = Fmt::kSuper ? make_rsrc(p.biases + rb * sgroups * 2, uint32_t(valid * sgroups * 4))
                                         : make_rsrc(p.biases + rb * p.groups, uint32_t(valid * p.groups * 2));
#pragma unroll
        for (int q = 0; q < PS; ++q) {
            const int c = slot + kM4Slots * (g * PS + q);
            const bool in = c < p.chunks;
            bf.c[q] = buffer_code_chunk(rc, in ? uint32_t(ri) * row_bytes + uint32_t(c) * kChunkBytes : kOutOfRange);
            const int grp = c >> p.group_shift;
            bf.a0[q] = __builtin_amdgcn_raw_buffer_load_b16(
                rs, int(in ? uint32_t(ri * p.groups + grp) * 2 : kOutOfRange), 0, kParamCache);
            if constexpr (Fmt::kSuper)
                bf.a1[q] = __builtin_amdgcn_raw_buffer_load_b32(
                    rbias, int(in ? uint32_t(ri * sgroups + (grp >> 3)) * 4 : kOutOfRange), 0, kParamCache);
            else if constexpr (Fmt::kAuxArrays >= 2)
                bf.a1[q] = __builtin_amdgcn_raw_buffer_load_b16(
                    rbias, int(in ? uint32_t(ri * p.groups + grp) * 2 : kOutOfRange), 0, kParamCache);
            else
                bf.a1[q] = 0;
        }
    };
    constexpr int kStepLoads = PS * (2 + ((Fmt::kSuper || Fmt::kAuxArrays >= 2) ? 1 : 0));

    // ---- x into LDS in the quarter layout, as the format's pieces, with
    // each chunk's activation sums (chunk_sum's tree) for the affine formats.
    // Plain call: rounds of 8 units per thread go from memory through the
    // conversion straight to LDS (the first round's loads go out before the
    // first weight step, and the wave waits for them alone).  Fused norm: the
    // norm's sums copy the raw units to LDS, then one pass normalizes and
    // converts them in place.
    uint4 *xlds = reinterpret_cast<uint4 *>(smem);
    const int upr = p.k / 8;                                  // 16-byte units per batch row
    const int x_units = B * upr;
    const int x_chunks = int(mfma4_x_chunks(p.chunks));
    float *xsum = reinterpret_cast<float *>(smem + int64_t(x_chunks) * 4 * B * 16);
    float *part = reinterpret_cast<float *>(smem + p.part_offset);    // [tile row][step][batch row]
    const M4XLayout xl{B};
    auto xpos = [&](int u) {
        const int b = row_of<B>(u, upr);
        return xl(b, u - b * upr, upr);
    };
    // unit u_in (clamped past the end, then not stored) to pieces and sums;
    // every lane of the wave calls it (the sums' shuffles), and the units of
    // one chunk sit in 4 consecutive lanes (units per row, the block size and
    // the round size are multiples of 4)
    auto put_unit = [&](int u_in, uint4 v) __attribute__((always_inline)) {
        const bool st = u_in < x_units;
        const int u = st ? u_in : x_units - 1;
        const int b = row_of<B>(u, upr);
        float sm = 0.0f;
        if constexpr (kSums) {
            sm = unit_sum(v);
            sm += __shfl_xor(sm, 1, kWave);
            sm += __shfl_xor(sm, 2, kWave);
        }
        uint4 pc[1];
        Fmt::unit_pieces(v, pc);
        if (st) {
            xlds[xpos(u)] = pc[0];
            if constexpr (kSums)
                if (((u - b * upr) & 3) == 0) xsum[((u - b * upr) >> 2) * 4 + b] = sm;
        }
    };
    Buf buf[D];
    if constexpr (kNorm) {
        float rn[B];
        // gamma is copied to LDS with the norm's loads where the host found
        // room for it beside x, the partials and the sums
        uint4 *glds = p.gamma_offset ? reinterpret_cast<uint4 *>(smem + p.gamma_offset) : nullptr;
        block_rms<B>(p, reinterpret_cast<float *>(smem + p.norm_offset), rn, xlds, glds, [&] {
            issue(buf[0], i_begin);
            wait_vm_loads<kStepLoads>();
        }, xl);
        // One gamma unit per thread and pass, applied to that unit of every
        // batch row (each thread rewrites only the units it read; lanes past
        // the row's end compute on its last unit and store nothing): one
        // gamma read per unit of a row, from LDS where it fits, instead of
        // one load from memory per unit of x.
        for (int base = 0; base < upr; base += blockDim.x) {
            const int gu_in = base + int(threadIdx.x);
            const int gu = min(gu_in, upr - 1);
            const uint4 gv = glds ? glds[gu] : load_x_unit(p.gamma + int64_t(gu) * 8);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const int u = b * upr + gu;
                put_unit(gu_in < upr ? u : x_units, norm_unit(xlds[xpos(u)], gv, rn[b]));
            }
        }
    } else {
        // The first step's loads go out right behind the activations', and
        // the wave waits for the activations alone; the rest of the prefetch
        // follows the barrier.  (Activations loaded first and waited for
        // before any weight load, or the whole prefetch issued before the
        // wait, both measured slower: a cold x takes 1 to 3 us to arrive
        // either way, and the stream needs one step per wave in flight
        // meanwhile, not more.)
        constexpr int kXu = 8;
        const int round = kXu * int(blockDim.x);
        uint4 xr[kXu];
        auto load_round = [&](int base) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kXu; ++i)
                xr[i] = load_x_unit(p.x + int64_t(min(base + int(threadIdx.x) + i * int(blockDim.x), x_units - 1)) * 8);
        };
        auto put_round = [&](int base) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kXu; ++i)
                if (base + i * int(blockDim.x) < x_units)     // uniform
                    put_unit(base + int(threadIdx.x) + i * int(blockDim.x), xr[i]);
        };
        load_round(0);
        issue(buf[0], i_begin);
        wait_vm_loads<kStepLoads>();
        put_round(0);
        for (int base = round; base < x_units; base += round) {
            load_round(base);
            put_round(base);
        }
    }
    // zeros: the chunks from the row end to the end of the zero pass
    for (int i = threadIdx.x; i < (x_chunks - p.chunks) * 4 * B; i += blockDim.x) {
        const int b = i % B, uq = i / B;
        xlds[xl(b, p.chunks * 4 + uq, upr)] = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (kSums)
            if ((uq & 3) == 0) xsum[(p.chunks + (uq >> 2)) * 4 + b] = 0.0f;
    }
    if constexpr (kSums)
        if (B < 4 && int(threadIdx.x) < x_chunks) xsum[threadIdx.x * 4 + 3] = 0.0f;
    __syncthreads();
#pragma unroll
    for (int d = 1; d < D; ++d) issue(buf[d], i_begin + d);
    issue_fence();

    // the lane's first LDS unit of a pass, less the pass's offset; a step's
    // passes past the tile's passes read the zero pass
    const int x_lane = slot * B + jb;
    auto x_pass = [&](int gq) { return min(gq, p.passes) * (4 * kM4Slots * B); };

    // acc[b]: batch row b of the lane's tile row (ri), this lane's slots
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // one chunk's 8 blocks of 4 columns in one chain: A = 4 batch rows of x,
    // B = the 4 tile rows' weights, so D column ri is the lane's own row
    auto mma_chunk = [&](const uint4 cq, const uint4 (&xq)[4], mfma_f32x4_t &c)
        __attribute__((always_inline)) {
        const uint32_t wv[4] = {cq.x, cq.y, cq.z, cq.w};
        c = mfma_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bf16x2_t d0, d1, d2, d3;
            if constexpr (Fmt::kSums) {
                // affine nibbles: (q0,q2), (q4,q6), (q1,q3), (q5,q7) scaled by
                // 2^-9, matching the pieces' column order
                const uint32_t lo = wv[m] & 0x0F0F0F0Fu, hi = (wv[m] >> 4) & 0x0F0F0F0Fu;
                d0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
                d1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
                d2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
                d3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
            } else {
                d0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv[m], 1.0f, 0);
                d1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv[m], 1.0f, 1);
                d2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv[m], 1.0f, 2);
                d3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv[m], 1.0f, 3);
            }
            const u32x2_t w_lo = {__builtin_bit_cast(uint32_t, d0), __builtin_bit_cast(uint32_t, d1)};
            const u32x2_t w_hi = {__builtin_bit_cast(uint32_t, d2), __builtin_bit_cast(uint32_t, d3)};
            const u32x2_t x_lo = {xq[m].x, xq[m].y};
            const u32x2_t x_hi = {xq[m].z, xq[m].w};
            c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(mfma_i16x4_t, x_lo),
                                                      __builtin_bit_cast(mfma_i16x4_t, w_lo), c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(mfma_i16x4_t, x_hi),
                                                      __builtin_bit_cast(mfma_i16x4_t, w_hi), c, 0, 0, 0);
        }
    };
    // the chunk's group fold with the lane's own row's parameters:
    // acc[b] += scale * raw[b] (+ bias * sum x[b])
    auto fold_chunk = [&](const mfma_f32x4_t &c, uint32_t a0, uint32_t a1, const float4 &xs)
        __attribute__((always_inline)) {
        float sv, bv = 0.0f;
        if constexpr (Fmt::kSuper) {
            Fmt::params(a0, a1, sv, bv);
        } else {
            sv = bf16_to_f32(a0);
            if constexpr (Fmt::kAuxArrays >= 2) bv = bf16_to_f32(a1);
        }
        if constexpr (Fmt::kSums) sv *= 512.0f;
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = fmaf(sv, c[b], acc[b]);
        if constexpr (Fmt::kSums) {
            acc[0] = fmaf(bv, xs.x, acc[0]);
            acc[1] = fmaf(bv, xs.y, acc[1]);
            acc[2] = fmaf(bv, xs.z, acc[2]);
            acc[3] = fmaf(bv, xs.w, acc[3]);
        }
    };
    const float4 *xsum4 = reinterpret_cast<const float4 *>(xsum);

    auto consume = [&](const Buf &bf, int item) __attribute__((always_inline)) {
        int64_t row0;
        int g;
        locate(item, row0, g);
        // Pass q + 1's products are issued before pass q's fold (which waits
        // for pass q's results), and x of pass q + 2 is read from LDS before
        // both, so the matrix blocks, the LDS reads and the folds overlap.
        uint4 xa[4], xb[4];
        float4 sa = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sb = sa;
        auto read_x = [&](int q, uint4 (&xq)[4], float4 &xs) __attribute__((always_inline)) {
            const int gq = __builtin_amdgcn_readfirstlane(g * PS + q);
            const uint4 *xp = xlds + x_pass(gq) + x_lane;
#pragma unroll
            for (int m = 0; m < 4; ++m) xq[m] = xp[m * kM4Slots * B];
            if constexpr (kSums) xs = xsum4[min(gq, p.passes) * kM4Slots + slot];
        };
        mfma_f32x4_t ca, cb;
        read_x(0, xa, sa);
        if (PS > 1) read_x(1, xb, sb);
        mma_chunk(bf.c[0], xa, ca);
#pragma unroll
        for (int q = 0; q < PS; ++q) {
            // even passes live in (xa, ca), odd passes in (xb, cb)
            const bool odd = q & 1;
            if (q + 1 < PS) {
                if (odd) mma_chunk(bf.c[q + 1], xa, ca);
                else mma_chunk(bf.c[q + 1], xb, cb);
            }
            const float4 xs_q = odd ? sb : sa;
            if (q + 2 < PS) {
                if (odd) read_x(q + 2, xb, sb);
                else read_x(q + 2, xa, sa);
            }
            if (odd) fold_chunk(cb, bf.a0[q], bf.a1[q], xs_q);
            else fold_chunk(ca, bf.a0[q], bf.a1[q], xs_q);
        }
        // the step's sums over the 16 slots: lanes 0..3 hold tile row
        // (lane) for every batch row
        float tot[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            tot[b] = mfma_row_sum(acc[b]);
            acc[b] = 0.0f;
        }
        if (lane < kM4Rows && row0 + lane < p.n) {
            const int64_t tl = row0 - t_begin * kM4Rows + lane;     // row in the workgroup
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (G == 1) store_y(p, b, row0 + lane, tot[b]);
                else part[(tl * G + g) * B + b] = tot[b];
            }
        }
    };

    // items in increasing order; the loop runs while the last buffer holds
    // one (then all do), each buffer is refilled right after it is consumed
    // (refills past the end read nothing), and the only exit is at the top
    int sl[D];
#pragma unroll
    for (int d = 0; d < D; ++d) sl[d] = i_begin + d;
    while (sl[D - 1] < n_items) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int nx = sl[d] + D;
            consume(buf[d], sl[d]);
            sl[d] = nx;
            issue(buf[d], nx);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (sl[d] < n_items) consume(buf[d], sl[d]);
    wait_vm_loads<0>();

    if (G > 1) {
        // add every row's step sums in step order and write y
        __syncthreads();
        const int rows = int(min(int64_t(T) * kM4Rows, p.n - t_begin * kM4Rows));
        for (int idx = threadIdx.x; idx < rows * B; idx += blockDim.x) {
            const int r = idx / B, b = idx - r * B;
            const float sum = sum_in_order(part + (r * G) * B + b, G, B);
            store_y(p, b, t_begin * kM4Rows + r, sum);
        }
    }
}

}  // namespace qg
