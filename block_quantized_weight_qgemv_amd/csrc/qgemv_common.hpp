// Shared device helpers of the block-quantized weight matvec (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kWave = 64;
constexpr int kChunkBytes = 16;
constexpr int kLdsSink = 32;      // LDS bytes after the staged activations
constexpr int kStageThreads = 256;   // row kernel: threads (waves 0..3) that stage x
constexpr int kStageUnits = 8;       // row kernel: at most 8 x units per staging thread
constexpr int kChunksPerWave = 16;   // row kernel: shared tiles are handed out in about 16 chunks per wave

// Whether a row-kernel instance stages x through LDS: only where the staging
// registers fit beside the activation pieces (batch x passes x pieces of at
// most 16 registers of 16 bytes) without spilling.
__host__ __device__ constexpr bool row_can_stage(int batch, int passes, int pieces) {
    return batch * passes * pieces <= 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

struct Params {
    const unsigned char *codes;     // packed code rows, row_bytes each
    const uint16_t *scales;         // bf16 [n, groups]   (FP4, affine)
    const uint16_t *biases;         // bf16 [n, groups]   (affine)
    const float *row_scale;         // f32 [n]            (FP8)
    const uint16_t *x;              // bf16 [B, k]
    void *y;                        // f32 or bf16 [B, n]
    int64_t n;
    int64_t row_bytes;              // bytes of one code row (= 16 * chunks)
    int32_t k;
    int32_t chunks;                 // 16-byte chunks per code row
    int32_t passes;                 // ceil(chunks / 64)
    int32_t groups;                 // scale groups per row
    int32_t group_shift;            // chunk index >> group_shift = group index
    int32_t total_waves;            // waves in the grid
    int32_t out_bf16;               // 0: f32 output, 1: bf16 output
    int32_t segs;                   // row kernel: K segments per row (split-K)
    int32_t seg_chunks;             // row kernel: chunks per segment
    int32_t seg_groups;             // row kernel: scale groups per segment
    int32_t x_staged;               // row kernel: x shared through LDS (>= 4 waves per workgroup)
    int32_t part_offset;            // row kernel: LDS byte offset of the split-K partials
    int32_t counter_offset;         // row kernel: LDS byte offset of the per-segment tile counters
    const uint16_t *gamma;          // bf16 [k]: fused RMSNorm weights (norm != 0)
    float eps;                      // fused RMSNorm epsilon
    int32_t norm;                   // 1: x is RMS-normalized inside the kernel
    int32_t norm_offset;            // LDS byte offset of the norm's group sums
    int32_t gamma_offset;           // LDS byte offset of gamma (fused norm; matrix blocks: 0 = not in LDS)
    int32_t x_global;               // LDS kernel: x too large for LDS, read from memory with the weights
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;     // NaN stays NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Weight codes and scales are read exactly once: non-temporal loads keep them
// from displacing the activations and the other rows' lines in the caches
// (a plain read stream reaches 7.1 TB/s with them, 6.4 TB/s without).
__device__ __forceinline__ uint4 load_code_chunk(const unsigned char *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_param(const uint16_t *p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint32_t load_param_pair(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}

// Buffer resources for the row kernel's weight loads: a raw (untyped) buffer
// of `bytes` bytes at `base`; loads at offsets past its end return zeros
// without a memory access.  Word 3 is the gfx9 raw-buffer format (32-bit data
// format, no swizzle, no index stride).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCacheNonTemporal = 2;      // the nt bit of the buffer-load cache policy
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;   // an offset past every resource

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kRsrcWord3);
}

__device__ __forceinline__ uint4 buffer_code_chunk(rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kCacheNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t buffer_param_pair(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, kCacheNonTemporal);
}

// Keeps the loads issued before it above it.  The compiler may otherwise
// sink a prefetch's loads to their first use, past the steps consumed
// before it, so that a wave starts with one step in flight instead of D.
// Emits no instruction.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Activations are shared by every wave: ordinary cached loads.
__device__ __forceinline__ uint4 load_x_unit(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Wait until at most N vector-memory loads of this wave are outstanding.
// gfx9 encoding of s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt and
// lgkmcnt (bits [6:4], [11:8]) left at their maximum, i.e. not waited for.
// The compiler still places the waits correctness needs; this one only
// orders issue (what comes after it is issued once the older loads are in).
template <int N>
__device__ __forceinline__ void wait_vm_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Value of lane `src` of v (every lane must be active).
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(v)));
}

// v[i] for a lane-dependent i, where every v[ii] is the same in all lanes.
// Each value passes through readfirstlane first: a select between plain loads
// of a register array would otherwise be folded back into one load with a
// run-time index, which moves the whole array (and everything stored beside
// it) to scratch memory.
template <int N>
__device__ __forceinline__ float pick_uniform(const float (&v)[N], int i) {
    float r = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v[0])));
#pragma unroll
    for (int ii = 1; ii < N; ++ii) {
        const float t = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v[ii])));
        r = (i == ii) ? t : r;
    }
    return r;
}

constexpr int pow2_ceil(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// ------------------------------------------------------------------ fused RMSNorm

// Sum of the squares of the 8 bf16 values of a 16-byte unit, in a fixed order.
__device__ __forceinline__ float unit_sumsq(const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = bf16_to_f32(w[i] & 0xFFFFu), b = bf16_to_f32(w[i] >> 16);
        s = fmaf(a, a, s);
        s = fmaf(b, b, s);
    }
    return s;
}

// bf16_rne(x * r * g) for a pair of bf16 values (x, g in the low and high
// halves).  The rounding is gfx950's packed f32 -> bf16 conversion (one
// instruction for both halves, against ten for the bit-level rounding of
// f32_to_bf16_rne): checked on the GPU over every f32 bit pattern, it gives
// the same bits for every number, and a NaN stays a NaN.
__device__ __forceinline__ uint32_t norm_pair(uint32_t xw, uint32_t gw, float r) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const float lo = (bf16_to_f32(xw & 0xFFFFu) * r) * bf16_to_f32(gw & 0xFFFFu);
    const float hi = (__uint_as_float(xw & 0xFFFF0000u) * r) * __uint_as_float(gw & 0xFFFF0000u);
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The normalized activation unit: what a separate RMSNorm would hand over.
__device__ __forceinline__ uint4 norm_unit(const uint4 x, const uint4 g, float r) {
    return make_uint4(norm_pair(x.x, g.x, r), norm_pair(x.y, g.y, r), norm_pair(x.z, g.z, r), norm_pair(x.w, g.w, r));
}

// ------------------------------------------------------------------ launch geometry

// Workgroups are dispatched round-robin over the 8 XCDs; renumbering them so
// that the workgroups of one XCD own neighbouring rows keeps a row range's
// neighbours (shared scale lines, the activations) in one L2.
__device__ __forceinline__ int logical_block() {
    int lblock = blockIdx.x;
    if ((gridDim.x & 7) == 0) lblock = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    return lblock;
}

__device__ __forceinline__ int wave_in_block() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int64_t wave_index() {
    return int64_t(logical_block()) * (blockDim.x >> 6) + wave_in_block();
}

// Rows [begin, end) of this wave: the n rows split into total_waves ranges
// whose sizes differ by at most one.
__device__ __forceinline__ void wave_rows(const Params &p, int64_t &begin, int64_t &end) {
    const int64_t w = wave_index();
    begin = w * p.n / p.total_waves;
    end = (w + 1) * p.n / p.total_waves;
}

// ------------------------------------------------------------------ reduction

__device__ __forceinline__ void swap32(float &a, float &b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void swap16(float &a, float &b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

template <int Ctrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl, 0xF, 0xF, false));
}

// Sum every lane's V partials over the wave (V a power of two).  Step A adds
// lanes l and l^32 (when V >= 2 the two halves of the wave keep different
// halves of the values), step B adds l and l^16 the same way, then a 16-lane
// row is summed by DPP rotations.  Afterwards the first lane of each 16-lane
// row holds kCnt = max(V/4, 1) totals.  The tree of additions a value sees
// does not depend on V, so a value's bits are the same whatever tile shape or
// batch carried it.  Must run with all 64 lanes active.
template <int V>
struct WaveSum {
    static_assert((V & (V - 1)) == 0, "WaveSum needs a power-of-two count");
    static constexpr bool kSplitA = V >= 2;
    static constexpr int kAfterA = kSplitA ? V / 2 : 1;
    static constexpr bool kSplitB = kAfterA >= 2;
    static constexpr int kCnt = kSplitB ? kAfterA / 2 : 1;

    __device__ static __forceinline__ void run(float (&v)[V]) {
        if constexpr (kSplitA) {
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                swap32(v[i], v[i + V / 2]);
                v[i] = v[i] + v[i + V / 2];
            }
        } else {
            float a = v[0], b = v[0];
            swap32(a, b);
            v[0] = a + b;
        }
        if constexpr (kSplitB) {
#pragma unroll
            for (int i = 0; i < kAfterA / 2; ++i) {
                swap16(v[i], v[i + kAfterA / 2]);
                v[i] = v[i] + v[i + kAfterA / 2];
            }
        } else {
            float a = v[0], b = v[0];
            swap16(a, b);
            v[0] = a + b;
        }
#pragma unroll
        for (int i = 0; i < kCnt; ++i) {
            float t = v[i];
            t = t + dpp_f<0x128>(t);    // row_ror:8
            t = t + dpp_f<0x124>(t);    // row_ror:4
            t = t + dpp_f<0x122>(t);    // row_ror:2
            t = t + dpp_f<0x121>(t);    // row_ror:1
            v[i] = t;
        }
    }

    // Does this lane write totals, and which value index does slot q hold?
    __device__ static __forceinline__ bool writer(int lane) {
        if (lane & 15) return false;
        if (!kSplitA && (lane & 32)) return false;
        if (!kSplitB && (lane & 16)) return false;
        return true;
    }
    __device__ static __forceinline__ int value_index(int lane, int q) {
        int idx = q;
        if constexpr (kSplitB) idx += ((lane >> 4) & 1) * kCnt;
        if constexpr (kSplitA) idx += ((lane >> 5) & 1) * (kSplitB ? 2 * kCnt : kCnt);
        return idx;
    }
};

// i / per for i < B * per, by comparisons (B <= 4: no integer division)
template <int B>
__device__ __forceinline__ int row_of(int i, int per) {
    int b = 0;
#pragma unroll
    for (int r = 1; r < B; ++r) b += i >= r * per ? 1 : 0;
    return b;
}

// src[0] + src[stride] + ... + src[(n - 1) * stride] (n >= 1), added in that
// order.  Above four terms the LDS reads go out eight at a time, so the sum
// waits for the LDS latency once per eight terms instead of once per term
// (the split-K sums at the end of a launch: u8 3840 x 15360 13.5 -> 13.3 us,
// FP4 fc_down at batch 4 12.2 -> 12.0; with two terms the batch of eight
// reads cost FP4 gate_up at batch 4 0.1 us).  The norm's sum of group sums
// stays a plain loop: this form made the fused and standalone norms slower.
__device__ __forceinline__ float sum_in_order(const float *src, int n, int stride) {
    float t = src[0];
    if (n <= 4) {                                 // (uniform) a few terms: one read per add
        for (int i = 1; i < n; ++i) t += src[int64_t(i) * stride];
        return t;
    }
    for (int i = 1; i < n; i += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[int64_t(min(i + j, n - 1)) * stride];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (i + j < n) t += v[j];
    }
    return t;
}

// RMSNorm factors r[b] = 1 / sqrt(mean_k x[b,k]^2 + eps) for the fused
// variants, computed by the whole workgroup (every thread must call it).  Row
// b's 16-byte units are cut into groups of 64 consecutive units; a wave sums a
// group's squares over its lanes (WaveSum, whose tree does not depend on how
// many groups it carries) and keeps the sum in LDS (gsum); after a barrier
// every wave adds a row's group sums 64 at a time with the same tree (lane l
// holding group 64c + l) and those totals in order, taking lane 0's value, so
// all threads hold the same r.  (Added one by one in group order, the LDS
// reads of the chain cost the standalone norm at k = 15360 ~0.4 us and the
// batch-4 fused call ~1.3 us.)  So r[b] depends on
// x[b] and k alone: not on the launch shape, the kernel or the batch size.
// Only the workgroup's first four waves load (four groups per wave at a time):
// the waves dispatched after them would find their loads queued behind the
// weight stream of the whole chip.  Where four waves would need more than one
// round of loads (more than 16 groups: k above 8192 at batch 1, batch 3-4 at
// k = 3840), the first eight load, so that fewer rounds of memory latency
// come before the first barrier.  `between` is called once by every wave,
// by the loading waves right after their first loads are issued (the caller
// can send its own loads behind them and wait for these alone).  With xdst
// (and gdst) given, the raw units of x (and of gamma, [k/8]) are copied to LDS
// on the way: unit u of batch row b to xdst[xidx(b, u, k / 8)].
struct PackedRows {
    __device__ int operator()(int b, int u, int upr) const { return b * upr + u; }
};
// The same with one 16-byte unit of padding after every 4 (a 64-byte chunk
// of 32 activations): a wave's lanes reading their chunks (80 bytes apart)
// then hit distinct banks, where 64 bytes apart every fourth lane shared them.
struct PaddedChunks {
    __device__ int operator()(int b, int u, int upr) const { const int i = b * upr + u; return i + (i >> 2); }
};

template <int B, class Between, class XIndex = PackedRows>
__device__ __forceinline__ void block_rms(const Params &p, float *gsum, float (&r)[B], uint4 *xdst, uint4 *gdst,
                                          Between &&between, XIndex xidx = XIndex{}) {
    using Red = WaveSum<4>;
    const int lane = threadIdx.x & (kWave - 1);
    const int upr = p.k / 8;                       // 16-byte units per row
    const int gpr = (upr + kWave - 1) / kWave;     // groups per row
    const int ng = B * gpr;
    constexpr int W4 = kStageThreads / kWave;
    const int W = min(int(blockDim.x >> 6), ng > 4 * W4 ? 2 * W4 : W4);    // loading waves
    const int w = wave_in_block();
    const bool loader = w < W;                     // uniform
    uint4 v[4], gv[4];
    int uu[4], bb[4];
    auto load_round = [&](int g0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = g0 + i * W;
            const int gi = min(g, ng - 1);
            bb[i] = row_of<B>(gi, gpr);
            uu[i] = (gi - bb[i] * gpr) * kWave + lane;
            v[i] = load_x_unit(p.x + (int64_t(bb[i]) * upr + min(uu[i], upr - 1)) * 8);
            if (gdst && g < gpr) gv[i] = load_x_unit(p.gamma + int64_t(min(uu[i], upr - 1)) * 8);
        }
    };
    auto sum_round = [&](int g0) {
        float sq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool real = g0 + i * W < ng && uu[i] < upr;
            sq[i] = real ? unit_sumsq(v[i]) : 0.0f;
            if (xdst && real) xdst[xidx(bb[i], uu[i], upr)] = v[i];
            if (gdst && real && g0 + i * W < gpr) gdst[uu[i]] = gv[i];
        }
        Red::run(sq);
        if (Red::writer(lane)) {
            const int g = g0 + Red::value_index(lane, 0) * W;
            if (g < ng) gsum[g] = sq[0];
        }
    };
    if (loader) load_round(w);
    between();
    if (loader) {
        sum_round(w);
        for (int g0 = w + 4 * W; g0 < ng; g0 += 4 * W) {
            load_round(g0);
            sum_round(g0);
        }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float t = 0.0f;
        for (int g0 = 0; g0 < gpr; g0 += kWave) {
            const float gl = gsum[b * gpr + min(g0 + lane, gpr - 1)];
            float v[1] = {g0 + lane < gpr ? gl : 0.0f};
            WaveSum<1>::run(v);
            t += __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[0])));
        }
        r[b] = 1.0f / sqrtf(t / float(p.k) + p.eps);
    }
}

// Reduce a tile's R x B accumulators over the wave; the writer lanes get
// (row i, batch b, total) through emit(i, b, total).  Zeroes acc.
template <int R, int B, class Emit>
__device__ __forceinline__ void reduce_tile(float (&acc)[R][B], int lane, Emit emit) {
    constexpr int V = R * B;
    constexpr int VP = pow2_ceil(V);
    using Red = WaveSum<VP>;
    float v[VP];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            v[i * B + b] = acc[i][b];
            acc[i][b] = 0.0f;
        }
#pragma unroll
    for (int i = V; i < VP; ++i) v[i] = 0.0f;
    Red::run(v);
    if (Red::writer(lane)) {
#pragma unroll
        for (int q = 0; q < Red::kCnt; ++q) {
            const int idx = Red::value_index(lane, q);
            if (idx < V) emit(idx / B, idx % B, v[q]);
        }
    }
}

__device__ __forceinline__ void store_y(const Params &p, int b, int64_t row, float out) {
    if (p.out_bf16)
        reinterpret_cast<uint16_t *>(p.y)[int64_t(b) * p.n + row] = static_cast<uint16_t>(f32_to_bf16_rne(out));
    else
        reinterpret_cast<float *>(p.y)[int64_t(b) * p.n + row] = out;
}

// Reduce a tile's R x B accumulators over the wave and write the first
// `rows` rows of the tile (rows <= R, the same in every lane) to y from row0
// on.  rs(i) is the scale applied to row i (1 unless the format has per-row
// scales).  Zeroes acc.
template <int R, int B, class RowScale>
__device__ __forceinline__ void reduce_store(const Params &p, float (&acc)[R][B], int64_t row0, int rows, int lane,
                                             RowScale rs) {
    reduce_tile<R, B>(acc, lane, [&](int i, int b, float total) {
        if (i < rows) store_y(p, b, row0 + i, total * rs(i));
    });
}

// rows of a tile of R rows starting at row0 that lie before row_end (0..R);
// row0 and row_end are uniform
template <int R>
__device__ __forceinline__ int tile_rows(int64_t row0, int64_t row_end) {
    const int64_t d = row_end - row0;
    return d < R ? (d > 0 ? int(d) : 0) : R;
}

}  // namespace qg
