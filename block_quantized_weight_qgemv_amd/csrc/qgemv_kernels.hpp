// The block-quantized weight matvec kernels for gfx950 (MI355X).
//
// Both kernels stream packed weight rows with the same structure:
//
//  * Row ranges per wavefront.  Rows [0, n) are split into one contiguous
//    range per wavefront (sizes differ by at most one row); workgroups are
//    renumbered so that one XCD's workgroups own neighbouring ranges.  A wave
//    walks its range R rows (a tile) at a time.
//  * 16-byte chunks.  Lane l owns chunks l, l+64, l+128, ... of every row
//    ("pass" j covers chunks 64j .. 64j+63), so every load instruction of a
//    wave reads 1 KiB of consecutive bytes.
//  * Prefetch.  The loads of step s+D are issued as soon as step s has been
//    consumed, so D steps of codes and scales are always in flight.  The loads
//    are issued unconditionally (clamped to valid addresses) so the compiler's
//    wait before a step waits for that step's loads only.
//  * Decode in registers with the gfx950 conversion instructions, a raw dot
//    per chunk, one multiply-add per chunk for the group scale (plus the bias
//    times the chunk's activation sum for affine), see qgemv_formats.hpp.
//  * One wave reduction per tile (permlane swaps and DPP), then y is written.
//
// qgemv_row_kernel: one step is a whole tile, the wave's slice of x lives in
//    registers (shared once through LDS when x is small enough), and a row's
//    group parameters
//    arrive as one coalesced dword per lane, handed to the lane that needs
//    them with ds_bpermute.  Rows longer than a few passes are cut into K
//    segments streamed by the waves of one workgroup (split-K); the segment
//    sums meet in LDS once, at the end.
// qgemv_lds_kernel (any shape the row kernel does not take): one step is one
//    pass of a tile, x (and its per-chunk sums) is staged once per workgroup
//    in LDS, and each lane loads its own group parameter.  Where x does not
//    fit in LDS (kXGlobal), each step instead brings the lane's activation
//    units for its chunk from memory with the weights (they stay in the
//    caches: every wave reads the same x) and forms the pieces and sums from
//    them with the same arithmetic, so the bits are those of the staged form.
#pragma once

#include "qgemv_common.hpp"
#include "qgemv_formats.hpp"

#include <type_traits>

namespace qg {

// Consume steps [0, steps) in order from D rotating buffers that the caller
// has filled with steps 0..D-1.  In the main loop the loads of step s + D go
// out right after step s is consumed, unconditionally; the last (at most
// 2D - 1) steps drain without issuing past the end.
template <int D, class Buf, class Issue, class Consume>
__device__ __forceinline__ void run_pipeline(Buf (&buf)[D], int steps, Issue &&issue, Consume &&consume) {
    int s0 = 0;
    for (; s0 + 2 * D <= steps; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            consume(buf[d], s0 + d);
            issue(buf[d], s0 + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (s0 + d < steps) consume(buf[d], s0 + d);
        if (s0 + d + D < steps) issue(buf[d], s0 + d + D);
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (s0 + D + d < steps) consume(buf[d], s0 + D + d);
}

// ------------------------------------------------------------------ short rows

template <class Fmt, int R, int B, int D, int J>
struct RowKernel {
    static constexpr int NA = Fmt::kAuxArrays > 0 ? Fmt::kAuxArrays : 1;
    struct Buf {
        uint4 c[R][J];
        uint32_t a[R][NA];     // this lane's dword of each row's parameter arrays
        float rs[R];
    };
};

template <class Fmt, int R, int B, int D, int J, bool kNorm>
__global__ void __launch_bounds__(512) qgemv_row_kernel(const Params p) {
    using K = RowKernel<Fmt, R, B, D, J>;
    using Buf = typename K::Buf;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & (kWave - 1);

    // Rows are split into one contiguous range per workgroup, cut into tiles
    // of R rows, and the tiles into chunks of C consecutive tiles.  The
    // workgroup's waves form G = waves / segs waves per K segment (split-K
    // when segs > 1): the G waves of segment `seg` share the workgroup's
    // chunks, each streaming that segment of every tile it takes, and a row's
    // segment sums meet in LDS at the end.  Wave gw of a segment starts with
    // chunk gw.  With x in LDS, later chunks come from a per-segment LDS
    // counter, first come first served (waves dispatched first, or served
    // faster by the memory system, stream more chunks, so the waves of a
    // workgroup finish together), and chunks are small: about 16 per wave,
    // one tile when there are few.  Otherwise (x not in LDS, or one wave per
    // segment) each wave has one chunk.
    const int S = p.segs;
    const int nb = gridDim.x;
    const int64_t blk = logical_block();
    const int64_t b_begin = blk * p.n / nb, b_end = (blk + 1) * p.n / nb;
    const int w = wave_in_block();
    const int G = (blockDim.x >> 6) / S;
    const int gw = w / S, seg = w - gw * S;     // wave gw of segment seg
    const int64_t b_rows = b_end - b_begin;
    const int brows = int(b_rows);                        // rows of the workgroup (< 2^31)
    const int T = (brows + R - 1) / R;
    const int c_lo = seg * p.seg_chunks;
    const int c_hi = min(p.chunks, c_lo + p.seg_chunks);

    // ---- activations.  Three ways in, each ending with the wave's slice of x
    // in registers:
    //  * staged (p.x_staged): waves 0..3 of the workgroup load all of x with
    //    coalesced 16-byte loads and the workgroup shares it through LDS.  The
    //    later waves of a workgroup are dispatched after the weight stream of
    //    the whole chip has started, and their own activation loads would wait
    //    behind it (about 1.5 us at the start of a 30720 x 3840 FP4 matvec);
    //    through LDS they get x as soon as the first four waves have it.
    //  * fused RMSNorm (p.norm): the workgroup computes every batch row's
    //    norm factor, copying raw x and gamma to LDS on the way (its loads go
    //    out ahead of the wave's first weight step, as x's do in the other
    //    cases); after a barrier the workgroup normalizes x in LDS in place
    //    and, after another, every wave reads its slice as in the staged case.
    //  * otherwise every wave loads its own slice.
    float rn[B];
#pragma unroll
    for (int b = 0; b < B; ++b) rn[b] = 1.0f;
    constexpr bool norm = kNorm;                          // a separate instance: no cost to the plain call
    uint4 *xlds = reinterpret_cast<uint4 *>(smem);
    uint4 *glds = reinterpret_cast<uint4 *>(smem + p.gamma_offset);
    const int upr = p.k / 8;                              // 16-byte units per row of x

    constexpr bool kCanStage = row_can_stage(B, J, Fmt::kPieces);
    // vector-memory loads one tile issues (codes, parameter pairs, row scales)
    constexpr int kTileLoads = R * J + R * Fmt::kAuxArrays + (Fmt::kRowScale ? R : 0);
    const bool staged = !norm && kCanStage && p.x_staged != 0;    // uniform
    const bool via_lds = staged || norm;                  // uniform: x reaches the waves through LDS
    const bool shared = via_lds && G > 1;                 // uniform: tiles handed out through LDS
    const int C = shared ? max(1, T / (kChunksPerWave * G)) : max(1, (T + G - 1) / G);    // tiles per chunk
    const int x_units = B * p.k / 8;                      // 16-byte units of x
    const bool few_units = x_units <= 2 * kStageThreads;  // uniform
    uint4 xr[kCanStage ? kStageUnits : 1];
    uint4 xraw[B][J][Fmt::kRawUnits];
    // the staging threads' units (clamped indices repeat the last unit)
    auto stage_unit_index = [&](int i) { return min(int(threadIdx.x) + i * kStageThreads, x_units - 1); };
    if (!via_lds) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int c = min(c_lo + kWave * j + lane, c_hi - 1);
                const uint16_t *xc = p.x + int64_t(b) * p.k + c * Fmt::kWpc;
#pragma unroll
                for (int u = 0; u < Fmt::kRawUnits; ++u) xraw[b][j][u] = load_x_unit(xc + 8 * u);
            }
    } else if (staged && kCanStage && w < kStageThreads / kWave) {
        // a fixed number of loads per thread (2 or 8), so that the waits stay
        // exact
        if (few_units) {
#pragma unroll
            for (int i = 0; i < 2; ++i) xr[i] = load_x_unit(p.x + int64_t(stage_unit_index(i)) * 8);
        } else if constexpr (kCanStage) {
#pragma unroll
            for (int i = 0; i < kStageUnits; ++i) xr[i] = load_x_unit(p.x + int64_t(stage_unit_index(i)) * 8);
        }
    }

    // The weights of tile t are read through buffer resources that cover the
    // tile's rows inside the workgroup's range only: rows past it, and whole
    // tiles past the end, read as zeros without touching memory, while every
    // issue sends the same loads (so the waits stay exact).  A lane reads its
    // chunk of every pass, and one dword of each row segment's parameters:
    // elements 2l, 2l+1 of the segment (the host guarantees an even number of
    // groups per segment, at most 128, starting on 4-byte boundaries).
    const int g_lo = seg * p.seg_groups;
    const int aux_off = g_lo + 2 * min(lane, p.seg_groups / 2 - 1);
    // two-level format: the segment's super-block words, one per lane (the
    // host guarantees whole super-blocks of 8 groups per segment)
    const int sgroups = p.groups >> 3;                    // super-blocks per row
    const int sup_off = (g_lo >> 3) + min(lane, (p.seg_groups >> 3) - 1);
    // (lanes past the segment's last chunk read past the resource: no access)
    auto code_off = [&](int j) {
        const int c = c_lo + kWave * j + lane;
        return c < c_hi ? uint32_t(c) * kChunkBytes : kOutOfRange;
    };
    auto issue = [&](Buf &bf, int t_in) __attribute__((always_inline)) {
        // t is the same in every lane; saying so keeps the resources in scalar
        // registers (a resource the compiler cannot prove uniform is used
        // through a loop over its distinct values)
        const int t = __builtin_amdgcn_readfirstlane(t_in);
        const int64_t row0 = b_begin + int64_t(t) * R;
        const int valid = t < T ? min(R, brows - t * R) : 0;
        const int64_t rb = valid ? row0 : 0;
        const rsrc_t rc = make_rsrc(p.codes + rb * p.row_bytes, uint32_t(valid * p.row_bytes));
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int j = 0; j < J; ++j) bf.c[i][j] = buffer_code_chunk(rc, uint32_t(i * p.row_bytes) + code_off(j));
        const uint32_t pbytes = uint32_t(valid * p.groups * 2);
        if constexpr (Fmt::kAuxArrays >= 1) {
            const rsrc_t rs = make_rsrc(p.scales + rb * p.groups, pbytes);
#pragma unroll
            for (int i = 0; i < R; ++i) bf.a[i][0] = buffer_param_pair(rs, uint32_t(i * p.groups + aux_off) * 2);
        }
        if constexpr (Fmt::kAuxArrays >= 2 && !Fmt::kSuper) {
            const rsrc_t rbias = make_rsrc(p.biases + rb * p.groups, pbytes);
#pragma unroll
            for (int i = 0; i < R; ++i) bf.a[i][1] = buffer_param_pair(rbias, uint32_t(i * p.groups + aux_off) * 2);
        }
        if constexpr (Fmt::kSuper) {
            const rsrc_t rsup = make_rsrc(p.biases + rb * sgroups * 2, uint32_t(valid * sgroups * 4));
#pragma unroll
            for (int i = 0; i < R; ++i) bf.a[i][1] = buffer_param_pair(rsup, uint32_t(i * sgroups + sup_off) * 4);
        }
        if constexpr (Fmt::kRowScale) {
#pragma unroll
            for (int i = 0; i < R; ++i) bf.rs[i] = p.row_scale[min(row0 + i, p.n - 1)];
        }
    };

    // The wave's tiles in order: `cur` walks the current chunk; when the
    // chunk is used up the next one is taken, only when its first tile is
    // needed (so the wave's first tile never touches the counter, which is
    // set up behind the staging barrier).  Chunks are taken in increasing
    // order, so a tile at or past T means the wave is done; T itself stands
    // for "no tile" (an empty issue).
    // All of it is uniform (scalar) work, and says so through readfirstlane:
    // a value the compiler takes for divergent here would make the loop exit
    // divergent, and every load and wait in the loop conservative.
    unsigned *counter = reinterpret_cast<unsigned *>(smem + p.counter_offset);
    int chunk = gw, cur = gw * C;
    auto next_issue = [&]() __attribute__((always_inline)) -> int {
        const bool at_end = cur < T && cur == (chunk + 1) * C;    // chunk used up
        int taken = chunk + G;
        if (shared && at_end) {
            unsigned v = 0;
            if (lane == 0) v = __hip_atomic_fetch_add(counter + seg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            taken = int(v);
        }
        chunk = __builtin_amdgcn_readfirstlane(at_end ? taken : chunk);
        cur = at_end ? chunk * C : cur;
        const int t = min(cur, T);
        cur = __builtin_amdgcn_readfirstlane(cur < T ? cur + 1 : cur);
        return __builtin_amdgcn_readfirstlane(t);
    };
    // The wave's first tile goes out right behind the activations, then the
    // wave waits for the activations alone (loads retire in order) before it
    // issues the rest of the prefetch: the first burst of weight requests over
    // the whole chip is one tile per wave, and the activations are not queued
    // behind it.
    Buf buf[D];
    int tl[D];                               // tile in each buffer (uniform)
    tl[0] = next_issue();
    if constexpr (norm) {
        if (shared && int(threadIdx.x) < S) counter[threadIdx.x] = unsigned(G);   // next shared chunk
        // Formats with 64-byte chunks of x keep it in LDS with a 16-byte pad
        // after every chunk (PaddedChunks): the reads of the wave's chunks
        // after the normalization are then free of bank conflicts (the fused
        // qkv 5.87 -> 5.78 us, gate_up 13.45 -> 13.38, the 48-layer step with
        // fused norms 1519 -> 1510).  The host sizes x's LDS to match.
        constexpr bool kPad = Fmt::kRawUnits == 4;
        auto xu = [](int u) { return kPad ? u + (u >> 2) : u; };
        using XIdx = typename std::conditional<kPad, PaddedChunks, PackedRows>::type;
        block_rms<B>(p, reinterpret_cast<float *>(smem + p.norm_offset), rn, xlds, glds, [&] {
            issue(buf[0], tl[0]);
            wait_vm_loads<kTileLoads>();
        }, XIdx{});
        // x is normalized in LDS in place, the work spread over the
        // workgroup, and read into registers; the rest of the prefetch goes
        // out behind that (the barrier in block_rms has made the tile
        // counters visible).  Issued ahead of the normalization instead, the
        // other waves' loads hold up the barrier below: about 0.4 us more per
        // launch, measured.
        for (int u = threadIdx.x; u < x_units; u += blockDim.x) {
            const int b = row_of<B>(u, upr);
            xlds[xu(u)] = norm_unit(xlds[xu(u)], glds[u - b * upr], pick_uniform(rn, b));
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int c = min(c_lo + kWave * j + lane, c_hi - 1);
                const int u0 = (b * p.k + c * Fmt::kWpc) / 8;
#pragma unroll
                for (int u = 0; u < Fmt::kRawUnits; ++u) xraw[b][j][u] = xlds[xu(u0) + u];
            }
#pragma unroll
        for (int d = 1; d < D; ++d) {
            tl[d] = next_issue();
            issue(buf[d], tl[d]);
        }
    } else {
        // one issue ahead of both ways (a copy in each costs the plain
        // instances code and speed)
        issue(buf[0], tl[0]);
        if (!via_lds) {
            wait_vm_loads<kTileLoads>();
        } else {
            if (w < kStageThreads / kWave) {
                if (few_units) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) xlds[stage_unit_index(i)] = xr[i];
                } else if constexpr (kCanStage) {
#pragma unroll
                    for (int i = 0; i < kStageUnits; ++i) xlds[stage_unit_index(i)] = xr[i];
                }
            }
            if (shared && int(threadIdx.x) < S) counter[threadIdx.x] = unsigned(G);   // next shared chunk
            __syncthreads();
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int c = min(c_lo + kWave * j + lane, c_hi - 1);
                    const int u0 = (b * p.k + c * Fmt::kWpc) / 8;
#pragma unroll
                    for (int u = 0; u < Fmt::kRawUnits; ++u) xraw[b][j][u] = xlds[u0 + u];
                }
        }
    }
    // The rest of the prefetch: the tiles of buffers 1..D-1 (issued below,
    // on the path that runs the main loop, or only the real ones when the
    // wave has fewer tiles than buffers).
    if constexpr (!norm) {
#pragma unroll
        for (int d = 1; d < D; ++d) tl[d] = next_issue();
    }

    // activation pieces (and chunk sums) in registers
    uint4 xp[B][J][Fmt::kPieces];
    float xs[B][J];
    auto make_pieces = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < J; ++j) {
#pragma unroll
                for (int u = 0; u < Fmt::kRawUnits; ++u) {
                    uint4 pc[Fmt::kPpu];
                    Fmt::unit_pieces(xraw[b][j][u], pc);
#pragma unroll
                    for (int m = 0; m < Fmt::kPpu; ++m) xp[b][j][u * Fmt::kPpu + m] = pc[m];
                }
                xs[b][j] = Fmt::kSums ? chunk_sum(xraw[b][j]) : 0.0f;
            }
    };

    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;

    // split-K partials of the workgroup's rows: [row - b_begin][seg][b],
    // behind the staged activations
    float *part = reinterpret_cast<float *>(smem + p.part_offset);

    // Where the group parameters of this lane's chunk in each pass sit: the
    // lane whose dword holds them, and a byte selector that moves the right
    // 16-bit half of that dword to the top of a word (a bf16 parameter as
    // fp32) or, for the two-level format's factors, to the bottom: one v_perm
    // per parameter in place of a shift, a mask and a select.  The selectors
    // take a register per pass; instances whose activations already fill the
    // register file (more than one batch row with chunk sums) select in the
    // loop instead.
    constexpr bool kSelPerm = B == 1 || !Fmt::kSums;
    constexpr int JS = kSelPerm ? J : 1;
    int psrc[JS], psup[JS];
    uint32_t psel[JS];
    if constexpr (kSelPerm) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = ((c_lo + kWave * j + lane) >> p.group_shift) - g_lo;   // group in the segment
            psrc[j] = (e >> 1) & (kWave - 1);
            psup[j] = (e >> 3) & (kWave - 1);
            if constexpr (Fmt::kSuper)
                psel[j] = (e & 1) ? 0x0c0c0302u : 0x0c0c0100u;
            else
                psel[j] = (e & 1) ? 0x03020c0cu : 0x01000c0cu;
        }
    }

    auto consume = [&](const Buf &bf, int t) __attribute__((always_inline)) {
        const int64_t row0 = b_begin + int64_t(t) * R;
        const int rows = min(R, brows - t * R);            // rows of the tile in the workgroup's range
#pragma unroll
        for (int i = 0; i < R; ++i) {
            // group parameters of this lane's chunk in every pass
            float sv[J], bv[J];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                sv[j] = bv[j] = 0.0f;
                if constexpr (kSelPerm) {
                    if constexpr (Fmt::kSuper) {
                        const uint32_t v = lane_read(bf.a[i][0], psrc[j]);
                        const uint32_t w = lane_read(bf.a[i][1], psup[j]);
                        Fmt::params(__builtin_amdgcn_perm(v, v, psel[j]), w, sv[j], bv[j]);
                    } else {
                        if constexpr (Fmt::kAuxArrays >= 1) {
                            const uint32_t v = lane_read(bf.a[i][0], psrc[j]);
                            sv[j] = __uint_as_float(__builtin_amdgcn_perm(v, v, psel[j]));
                        }
                        if constexpr (Fmt::kAuxArrays >= 2) {
                            const uint32_t v = lane_read(bf.a[i][1], psrc[j]);
                            bv[j] = __uint_as_float(__builtin_amdgcn_perm(v, v, psel[j]));
                        }
                    }
                } else {
                    const int e = ((c_lo + kWave * j + lane) >> p.group_shift) - g_lo;   // group in the segment
                    const int src = (e >> 1) & (kWave - 1);
                    const bool hi = e & 1;
                    if constexpr (Fmt::kSuper) {
                        const uint32_t v = lane_read(bf.a[i][0], src);
                        const uint32_t w = lane_read(bf.a[i][1], (e >> 3) & (kWave - 1));
                        Fmt::params(hi ? (v >> 16) : (v & 0xFFFFu), w, sv[j], bv[j]);
                    } else {
                        if constexpr (Fmt::kAuxArrays >= 1) {
                            const uint32_t v = lane_read(bf.a[i][0], src);
                            sv[j] = __uint_as_float(hi ? (v & 0xFFFF0000u) : (v << 16));
                        }
                        if constexpr (Fmt::kAuxArrays >= 2) {
                            const uint32_t v = lane_read(bf.a[i][1], src);
                            bv[j] = __uint_as_float(hi ? (v & 0xFFFF0000u) : (v << 16));
                        }
                    }
                }
            }
            if (i < rows) {
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    if (c_lo + kWave * j + lane < c_hi) {
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            const float raw = Fmt::dot(bf.c[i][j], xp[b][j], 0.0f);
                            acc[i][b] = Fmt::fold(acc[i][b], raw, sv[j], bv[j], xs[b][j]);
                        }
                    }
                }
            }
        }
        if (S == 1) {
            reduce_store<R, B>(p, acc, row0, rows, lane, [&](int i) {
                if constexpr (Fmt::kRowScale) return pick_uniform(bf.rs, i);
                return 1.0f;
            });
        } else {
            reduce_tile<R, B>(acc, lane, [&](int i, int b, float total) {
                if (i < rows) part[((t * R + i) * S + seg) * B + b] = total;
            });
        }
    };

    // The buffers hold the wave's tiles in increasing order (T, "no tile",
    // once the wave's work is out), so when the last buffer holds a tile they
    // all do.  The loop runs while that is so: each step consumes a buffer
    // and refills it at once (a refill past the end is empty and costs no
    // memory traffic), and the loop's only exit is its test at the top.
    // Every way back to the head then passes all D refills, which is what
    // lets the compiler's wait before each step count exactly the loads of
    // the other buffers (with exits inside the body, some instances kept an
    // edge from a middle step to the head and waited for the whole prefetch
    // at every first step).  What the last refills brought is consumed after
    // the loop, in order.
    //
    // Workgroups with at least 3 tiles per wave run the D-deep pipeline from
    // the first step: the prefetch goes out before the first tile is
    // consumed (a fence keeps it there), which shortens the ramp (15360 x
    // 3840 u4: 9.25 -> 8.9 us).  Left to itself the compiler sinks those
    // loads to their first use, which measured faster with fewer tiles per
    // wave (8192 x 3840 FP4, 2 per wave: 5.68 against 5.85 us with the
    // fence, 6.07 one tile at a time), so the other workgroups keep that
    // form.  Each path has its own copy of the main loop, so the compiler's
    // waits in each count all D buffers.
    auto run_tiles = [&]() __attribute__((always_inline)) {
        make_pieces();
        while (tl[D - 1] < T) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int nt = next_issue();
                consume(buf[d], tl[d]);
                tl[d] = nt;
                issue(buf[d], nt);
            }
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (tl[d] < T) consume(buf[d], tl[d]);
    };
    if (T >= 3 * G) {
        if constexpr (!norm) {
#pragma unroll
            for (int d = 1; d < D; ++d) issue(buf[d], tl[d]);
        }
        issue_fence();
        run_tiles();
    } else {
        if constexpr (!norm) {
#pragma unroll
            for (int d = 1; d < D; ++d) issue(buf[d], tl[d]);
        }
        run_tiles();
    }
    wait_vm_loads<0>();

    if (S > 1) {
        // add the segments of every row in segment order and write y
        __syncthreads();
        for (int64_t idx = threadIdx.x; idx < b_rows * B; idx += blockDim.x) {
            const int64_t r = idx / B;
            const int b = int(idx - r * B);
            float sum = sum_in_order(part + (r * S) * B + b, S, B);
            const int64_t row = b_begin + r;
            if constexpr (Fmt::kRowScale) sum *= p.row_scale[row];
            store_y(p, b, row, sum);
        }
    }
}

// ------------------------------------------------------------------ long rows

template <class Fmt, int R, int B, int D, bool kXGlobal = false, bool kNorm = false>
struct LdsKernel {
    static constexpr int NA = Fmt::kAuxArrays > 0 ? Fmt::kAuxArrays : 1;
    static constexpr int XB = kXGlobal ? B : 1;                   // activation units carried by a step
    static constexpr int XU = kXGlobal ? Fmt::kRawUnits : 1;
    static constexpr int GU = kXGlobal && kNorm ? Fmt::kRawUnits : 1;
    struct Buf {
        uint4 c[R];
        uint32_t a[R][NA];     // this lane's group parameter of each row
        float rs[R];
        uint4 xr[XB][XU];      // kXGlobal: the lane's raw activation units for this step's chunk
        uint4 gr[GU];          // kXGlobal with the fused norm: gamma's units for the chunk
    };
    // bytes of dynamic LDS: activation pieces, per-chunk sums, and a 32-byte
    // sink for the stores of out-of-range staging lanes
    __host__ __device__ static constexpr int64_t lds_bytes(int chunks) {
        return int64_t(B) * Fmt::kPieces * chunks * 16 + (Fmt::kSums ? int64_t(B) * chunks * 4 : 0) + kLdsSink;
    }
};

template <class Fmt, int R, int B, int D, bool kNorm, bool kXGlobal = false>
__global__ void __launch_bounds__(512) qgemv_lds_kernel(const Params p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    using LK = LdsKernel<Fmt, R, B, D, kXGlobal, kNorm>;
    using Buf = typename LK::Buf;
    const int lane = threadIdx.x & (kWave - 1);
    // fused RMSNorm: every batch row's factor, before any weight load
    float rn[B];
#pragma unroll
    for (int b = 0; b < B; ++b) rn[b] = 1.0f;
    constexpr bool norm = kNorm;
    if constexpr (norm) block_rms<B>(p, reinterpret_cast<float *>(smem + p.norm_offset), rn, nullptr, nullptr, [] {});
    int64_t r_begin, r_end;
    wave_rows(p, r_begin, r_end);
    const int tiles = int((r_end - r_begin + R - 1) / R);
    const int passes = p.passes;
    const int steps = tiles * passes;
    const int64_t row_hi = r_end > r_begin ? r_end - 1 : min(r_begin, p.n - 1);
    const int chunks = p.chunks;
    const int last_chunk = chunks - 1;

    auto issue = [&](Buf &b, int s) {
        const int t = s / passes;
        const int j = s - t * passes;
        const int c = min(lane + kWave * j, last_chunk);
        const uint32_t lane_off = uint32_t(c) * kChunkBytes;
        const int64_t row0 = r_begin + int64_t(t) * R;
        const int g = c >> p.group_shift;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t row = min(row0 + i, row_hi);
            b.c[i] = load_code_chunk(p.codes + row * p.row_bytes + lane_off);
            if constexpr (Fmt::kAuxArrays >= 1) b.a[i][0] = load_param(p.scales + row * p.groups + g);
            if constexpr (Fmt::kSuper)
                b.a[i][1] = load_param_pair(p.biases + (row * (p.groups >> 3) + (g >> 3)) * 2);
            else if constexpr (Fmt::kAuxArrays >= 2)
                b.a[i][1] = load_param(p.biases + row * p.groups + g);
            if constexpr (Fmt::kRowScale) b.rs[i] = p.row_scale[row];
        }
        if constexpr (kXGlobal) {
#pragma unroll
            for (int bb = 0; bb < B; ++bb)
#pragma unroll
                for (int u = 0; u < Fmt::kRawUnits; ++u)
                    b.xr[bb][u] = load_x_unit(p.x + int64_t(bb) * p.k + int64_t(c) * Fmt::kWpc + 8 * u);
            if constexpr (norm) {
#pragma unroll
                for (int u = 0; u < Fmt::kRawUnits; ++u)
                    b.gr[u] = load_x_unit(p.gamma + int64_t(c) * Fmt::kWpc + 8 * u);
            }
        }
    };

    // ---- activations into LDS, overlapped with the weight prefetch.  Each
    // thread first loads up to kXU activation units, then the prefetch is
    // issued, and only then are the units used: the vector-load counter
    // retires in order, so waiting for them does not wait for the weights.
    uint4 *xs = reinterpret_cast<uint4 *>(smem);
    float *xsum = reinterpret_cast<float *>(smem + int64_t(B) * Fmt::kPieces * chunks * 16);
    unsigned char *sink_base = smem + int64_t(B) * Fmt::kPieces * chunks * 16 +
                               (Fmt::kSums ? int64_t(B) * chunks * 4 : 0);
    uint4 *sink = reinterpret_cast<uint4 *>(sink_base);
    float *sink_f = reinterpret_cast<float *>(sink_base + 16);
    const int units_per_row = p.k / 8;
    const int x_units = B * units_per_row;
    auto x_unit = [&](int u) -> uint4 {
        const int b = u / units_per_row;
        return load_x_unit(p.x + int64_t(b) * p.k + (u - b * units_per_row) * 8);
    };
    auto gamma_unit = [&](int u) -> uint4 {
        return load_x_unit(p.gamma + (u - (u / units_per_row) * units_per_row) * 8);
    };
    // Every lane runs the same staging code and stores unconditionally (an
    // out-of-range unit is clamped to the last one and stored to the sink),
    // so no activation load is sunk into a conditional block below the
    // prefetch.
    auto stage_unit = [&](int u_in, const uint4 v_raw, const uint4 g) {
        const bool st = u_in < x_units;
        const int u = st ? u_in : x_units - 1;
        const int b = u / units_per_row;
        const int e = (u - b * units_per_row) * 8;
        const int c = e / Fmt::kWpc, ru = (e % Fmt::kWpc) / 8;
        const uint4 v = norm ? norm_unit(v_raw, g, pick_uniform(rn, b)) : v_raw;
        uint4 pc[Fmt::kPpu];
        Fmt::unit_pieces(v, pc);
#pragma unroll
        for (int m = 0; m < Fmt::kPpu; ++m)
            *(st ? &xs[(b * Fmt::kPieces + ru * Fmt::kPpu + m) * chunks + c] : sink) = pc[m];
        if constexpr (Fmt::kSums) {
            float sm = unit_sum(v);
            // the units of one chunk sit in consecutive lanes (units per row
            // and the wave width are multiples of the units per chunk); the
            // tree matches chunk_sum()
#pragma unroll
            for (int m = 1; m < Fmt::kRawUnits; m <<= 1) sm += __shfl_xor(sm, m, kWave);
            *((st && ru == 0) ? &xsum[b * chunks + c] : sink_f) = sm;
        }
    };

    Buf buf[D];
    if constexpr (kXGlobal) {
        // nothing to stage: the steps carry their activations
#pragma unroll
        for (int d = 0; d < D; ++d) issue(buf[d], max(0, min(d, steps - 1)));
        issue_fence();
    } else {
        constexpr int kXU = 8;
        uint4 xr[kXU], gr[kXU];
#pragma unroll
        for (int i = 0; i < kXU; ++i) xr[i] = x_unit(min(int(threadIdx.x) + i * int(blockDim.x), x_units - 1));
        if (norm) {
#pragma unroll
            for (int i = 0; i < kXU; ++i) gr[i] = gamma_unit(min(int(threadIdx.x) + i * int(blockDim.x), x_units - 1));
        } else {
#pragma unroll
            for (int i = 0; i < kXU; ++i) gr[i] = make_uint4(0, 0, 0, 0);
        }

        // step 0 right behind the activations, the rest once they are in (as
        // in the row kernel)
        issue(buf[0], 0);
        wait_vm_loads<R + R * Fmt::kAuxArrays + (Fmt::kRowScale ? R : 0)>();
#pragma unroll
        for (int d = 1; d < D; ++d) issue(buf[d], max(0, min(d, steps - 1)));
        issue_fence();

#pragma unroll
        for (int i = 0; i < kXU; ++i) stage_unit(int(threadIdx.x) + i * int(blockDim.x), xr[i], gr[i]);
        // activations beyond kXU units per thread; the trip count is the same
        // for every lane of a wave
        for (int base = kXU * blockDim.x; base < x_units; base += blockDim.x) {
            const int u = min(base + int(threadIdx.x), x_units - 1);
            stage_unit(base + threadIdx.x, x_unit(u), norm ? gamma_unit(u) : make_uint4(0, 0, 0, 0));
        }
        __syncthreads();
    }

    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;

    auto consume = [&](const Buf &bf, int s) {
        const int t = s / passes;
        const int j = s - t * passes;
        const int c = lane + kWave * j;
        const int64_t row0 = r_begin + int64_t(t) * R;
        if (c < chunks) {
            float s_[R], b_[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                if constexpr (Fmt::kSuper) {
                    Fmt::params(bf.a[i][0], bf.a[i][1], s_[i], b_[i]);
                } else {
                    s_[i] = Fmt::kAuxArrays >= 1 ? bf16_to_f32(bf.a[i][0]) : 0.0f;
                    b_[i] = Fmt::kAuxArrays >= 2 ? bf16_to_f32(bf.a[i][LK::NA - 1]) : 0.0f;
                }
            }
            // one batch row at a time: its pieces are live only for its own
            // dots (each accumulator's order of additions is unchanged)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                uint4 xp[Fmt::kPieces];
                float xsv;
                if constexpr (kXGlobal) {
                    // the staged form's arithmetic: normalize, split into
                    // pieces, sum with chunk_sum's tree
                    uint4 v[Fmt::kRawUnits];
#pragma unroll
                    for (int u = 0; u < Fmt::kRawUnits; ++u) {
                        if constexpr (norm) v[u] = norm_unit(bf.xr[b][u], bf.gr[u], pick_uniform(rn, b));
                        else v[u] = bf.xr[b][u];
                        uint4 pc[Fmt::kPpu];
                        Fmt::unit_pieces(v[u], pc);
#pragma unroll
                        for (int m = 0; m < Fmt::kPpu; ++m) xp[u * Fmt::kPpu + m] = pc[m];
                    }
                    xsv = Fmt::kSums ? chunk_sum(v) : 0.0f;
                } else {
#pragma unroll
                    for (int q = 0; q < Fmt::kPieces; ++q) xp[q] = xs[(b * Fmt::kPieces + q) * chunks + c];
                    xsv = Fmt::kSums ? xsum[b * chunks + c] : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    if (row0 + i < r_end) {
                        const float raw = Fmt::dot(bf.c[i], xp, 0.0f);
                        acc[i][b] = Fmt::fold(acc[i][b], raw, s_[i], b_[i], xsv);
                    }
                }
            }
        }
        if (j == passes - 1) {
            reduce_store<R, B>(p, acc, row0, tile_rows<R>(row0, r_end), lane, [&](int i) {
                if constexpr (Fmt::kRowScale) return pick_uniform(bf.rs, i);
                return 1.0f;
            });
        }
    };

    run_pipeline<D>(buf, steps, issue, consume);
}

// ------------------------------------------------------------------ standalone norm

// The fused variants' RMSNorm on its own: out[b, k] = bf16_rne(x * r[b] *
// gamma), with r[b] summed exactly as the fused matvec sums it (block_rms).
// Workgroup b does batch row b.  LDS holds the row's group sums and, with
// kKeep (when they fit), the row's x and gamma as they were first read, so
// that each is read from memory once.
inline constexpr int64_t rmsnorm_sums_bytes(int64_t k) { return ((k / 8 + kWave - 1) / kWave * 4 + 15) / 16 * 16; }

template <bool kKeep>
__global__ void __launch_bounds__(512) qg_rmsnorm_kernel(Params p, uint16_t *out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int upr = p.k / 8;
    p.x += int64_t(blockIdx.x) * p.k;
    out += int64_t(blockIdx.x) * p.k;
    uint4 *xs = reinterpret_cast<uint4 *>(smem + rmsnorm_sums_bytes(p.k));
    uint4 *gs = xs + upr;
    float rn[1];
    block_rms<1>(p, reinterpret_cast<float *>(smem), rn, kKeep ? xs : nullptr, kKeep ? gs : nullptr, [] {});
    for (int u = threadIdx.x; u < upr; u += blockDim.x) {
        const uint4 xv = kKeep ? xs[u] : load_x_unit(p.x + int64_t(u) * 8);
        const uint4 gv = kKeep ? gs[u] : load_x_unit(p.gamma + int64_t(u) * 8);
        *reinterpret_cast<uint4 *>(out + int64_t(u) * 8) = norm_unit(xv, gv, rn[0]);
    }
}

}  // namespace qg
