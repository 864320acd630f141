// Device side of the block-quantized weight matvec for gfx950 (MI355X).
//
// One kernel template streams the packed weight rows of every format:
//
//  * Row tiles per wavefront.  The rows [0, n) are split into one contiguous
//    range per wavefront (ranges differ by at most one row) and a wave walks
//    its range R rows at a time.  Workgroups are renumbered so that the
//    workgroups of one XCD own neighbouring row ranges.
//  * 16-byte chunks.  A code row is a sequence of 16-byte chunks
//    (32 four-bit or 16 eight-bit weights).  Lane l of a wave owns chunks
//    l, l+64, l+128, ... of every row it visits ("pass" j covers chunks
//    64j .. 64j+63), so each load instruction of a wave reads 1 KiB of
//    consecutive bytes per row.
//  * Prefetch.  A "step" is one pass over the R rows of a tile; the loads of
//    step s+D are issued as soon as step s has been consumed, so D steps of
//    weight codes and group scales are always in flight per wave.
//  * Decode in registers.  E2M1 and E4M3 codes become bf16 pairs with the
//    gfx950 scaled-conversion instructions (one instruction per two weights),
//    u4 codes go through the E4M3 converter (a byte holding q < 16 is the
//    E4M3 number q * 2^-9 exactly), u8 codes through the byte-to-float
//    converters.  No lookup table is read from memory.
//  * Raw dot, then one multiply-add per chunk for the group scale (two for
//    affine: scale * raw + bias * sum(x over the chunk)).
//  * The activation vector (and, for affine, its per-chunk sums) is staged
//    once per workgroup in LDS; LDS holds nothing else.
//  * A wave reduces its R * B per-lane partials once per tile with
//    permlane32/permlane16 swaps and DPP row rotations, then writes y.
//
// Prior art, not the blueprint: "Hand-Writing Gemma 4 Flash-Decoding + an FP4
// Matvec Bonus (Part 2)", section "The assumption that failed the profiler"
// (byte-permute decode instead of a constant-memory table, group scale folded
// into one multiply-add, loads pipelined one iteration ahead).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kWave = 64;
constexpr int kChunkBytes = 16;
constexpr int kLdsSink = 32;      // LDS bytes after the staged activations

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
};

// ------------------------------------------------------------------ helpers

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

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Weight codes and scales are read exactly once: non-temporal loads keep them
// from displacing the activations and the other rows' lines in the caches
// (a plain read stream reaches 7.1 TB/s with them, 6.4 TB/s without).
__device__ __forceinline__ uint4 load_code_chunk(const unsigned char *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_param(const uint16_t *p) { return __builtin_nontemporal_load(p); }

// ------------------------------------------------------------------ formats
//
// Each format describes:
//   kWpc      weights per 16-byte code chunk
//   kPieces   16-byte LDS pieces of staged activation per chunk and batch row
//   kSums     whether the per-chunk activation sums are staged too (affine)
//   Aux       per (row, chunk) parameters loaded with the codes
//   load_aux  reads Aux for (row, chunk)
//   stage     writes one 16-byte unit of x (8 bf16, element e..e+7) to LDS
//             (to the sink slot when the unit is out of range)
//   dot       raw dot of one code chunk with the staged activation pieces
//   fold      accumulates the raw dot into the row accumulator

struct FmtFP4 {
    static constexpr int kWpc = 32;
    static constexpr int kPieces = 4;          // 32 bf16
    static constexpr bool kSums = false;
    static constexpr bool kRowScale = false;
    struct Aux { uint32_t s; };

    __device__ static __forceinline__ Aux load_aux(const Params &p, int64_t row, int c) {
        const uint16_t *srow = p.scales + row * p.groups;       // uniform
        return Aux{load_param(srow + (c >> p.group_shift))};
    }
    __device__ static __forceinline__ Aux zero_aux() { return Aux{0u}; }

    // piece q holds columns 8q .. 8q+7 in natural order
    __device__ static __forceinline__ void stage(uint4 v, int e, uint4 *piece_base, int chunks, uint4 *sink, bool st) {
        const int c = e / kWpc, q = (e % kWpc) / 8;
        *(st ? &piece_base[q * chunks + c] : sink) = v;
    }

    // word i of the chunk holds columns 8i..8i+7; its byte b holds columns
    // 8i+2b (low nibble) and 8i+2b+1 (high nibble), matching dword b of piece i
    __device__ static __forceinline__ float dot(const uint4 q, const uint4 *xp, float raw) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 xv = xp[i];
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 0), xv.x, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 1), xv.y, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 2), xv.z, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 3), xv.w, raw);
        }
        return raw;
    }
    __device__ static __forceinline__ float fold(float acc, float raw, Aux a, float) {
        return fmaf(bf16_to_f32(a.s), raw, acc);
    }
};

struct FmtAffineU4 {
    static constexpr int kWpc = 32;
    static constexpr int kPieces = 4;
    static constexpr bool kSums = true;
    static constexpr bool kRowScale = false;
    struct Aux { uint32_t s, b; };

    __device__ static __forceinline__ Aux load_aux(const Params &p, int64_t row, int c) {
        const int64_t base = row * p.groups;                      // uniform
        const int g = c >> p.group_shift;
        return Aux{load_param(p.scales + base + g), load_param(p.biases + base + g)};
    }
    __device__ static __forceinline__ Aux zero_aux() { return Aux{0u, 0u}; }

    // piece q holds columns 8q..8q+7 reordered as (0,2),(4,6),(1,3),(5,7):
    // the pairs the decode below produces from one u32 word
    __device__ static __forceinline__ void stage(uint4 v, int e, uint4 *piece_base, int chunks, uint4 *sink, bool st) {
        const int c = e / kWpc, q = (e % kWpc) / 8;
        uint4 o;
        o.x = (v.x & 0xFFFFu) | (v.y << 16);            // x0, x2
        o.y = (v.z & 0xFFFFu) | (v.w << 16);            // x4, x6
        o.z = (v.x >> 16) | (v.y & 0xFFFF0000u);        // x1, x3
        o.w = (v.z >> 16) | (v.w & 0xFFFF0000u);        // x5, x7
        *(st ? &piece_base[q * chunks + c] : sink) = o;
    }

    // word i holds codes of columns 8i..8i+7 (code j at bits 4j).  Masking the
    // low and the high nibble of every byte leaves bytes < 16, and a byte
    // q < 16 read as E4M3 is exactly q * 2^-9, so the FP8 converter yields the
    // bf16 pairs (q0,q2),(q4,q6) and (q1,q3),(q5,q7) scaled by 2^-9.
    __device__ static __forceinline__ float dot(const uint4 q, const uint4 *xp, float raw) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 xv = xp[i];
            const uint32_t lo = w[i] & 0x0F0F0F0Fu;
            const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false), xv.x, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true), xv.y, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false), xv.z, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true), xv.w, raw);
        }
        return raw;
    }
    // sum_k (s q_k + b) x_k = (s * 2^9) * raw + b * X   (raw carries q * 2^-9)
    __device__ static __forceinline__ float fold(float acc, float raw, Aux a, float xsum) {
        acc = fmaf(bf16_to_f32(a.s) * 512.0f, raw, acc);
        return fmaf(bf16_to_f32(a.b), xsum, acc);
    }
};

struct FmtAffineU8 {
    static constexpr int kWpc = 16;
    static constexpr int kPieces = 4;          // 16 activations as f32
    static constexpr bool kSums = true;
    static constexpr bool kRowScale = false;
    struct Aux { uint32_t s, b; };

    __device__ static __forceinline__ Aux load_aux(const Params &p, int64_t row, int c) {
        const int64_t base = row * p.groups;                      // uniform
        const int g = c >> p.group_shift;
        return Aux{load_param(p.scales + base + g), load_param(p.biases + base + g)};
    }
    __device__ static __forceinline__ Aux zero_aux() { return Aux{0u, 0u}; }

    // 8 bf16 (columns e..e+7) become two f32 pieces: columns 4q..4q+3
    __device__ static __forceinline__ void stage(uint4 v, int e, uint4 *piece_base, int chunks, uint4 *sink, bool st) {
        const int c = e / kWpc, q = (e % kWpc) / 4;
        uint4 a, b;
        a.x = v.x << 16; a.y = v.x & 0xFFFF0000u; a.z = v.y << 16; a.w = v.y & 0xFFFF0000u;
        b.x = v.z << 16; b.y = v.z & 0xFFFF0000u; b.z = v.w << 16; b.w = v.w & 0xFFFF0000u;
        *(st ? &piece_base[q * chunks + c] : sink) = a;
        *(st ? &piece_base[(q + 1) * chunks + c] : sink) = b;
    }

    // word i holds codes of columns 4i..4i+3, one byte each
    __device__ static __forceinline__ float dot(const uint4 q, const uint4 *xp, float raw) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 xv = xp[i];
            raw = fmaf(static_cast<float>(w[i] & 0xFFu), __uint_as_float(xv.x), raw);
            raw = fmaf(static_cast<float>((w[i] >> 8) & 0xFFu), __uint_as_float(xv.y), raw);
            raw = fmaf(static_cast<float>((w[i] >> 16) & 0xFFu), __uint_as_float(xv.z), raw);
            raw = fmaf(static_cast<float>(w[i] >> 24), __uint_as_float(xv.w), raw);
        }
        return raw;
    }
    __device__ static __forceinline__ float fold(float acc, float raw, Aux a, float xsum) {
        acc = fmaf(bf16_to_f32(a.s), raw, acc);
        return fmaf(bf16_to_f32(a.b), xsum, acc);
    }
};

struct FmtFP8 {
    static constexpr int kWpc = 16;
    static constexpr int kPieces = 2;          // 16 bf16
    static constexpr bool kSums = false;
    static constexpr bool kRowScale = true;
    // the row scale rides along with every step of the row (a uniform
    // address: a scalar load, which does not hold up the vector-load queue)
    struct Aux { float rs; };

    __device__ static __forceinline__ Aux load_aux(const Params &p, int64_t row, int) {
        return Aux{p.row_scale[row]};
    }
    __device__ static __forceinline__ Aux zero_aux() { return Aux{0.0f}; }

    __device__ static __forceinline__ void stage(uint4 v, int e, uint4 *piece_base, int chunks, uint4 *sink, bool st) {
        const int c = e / kWpc, q = (e % kWpc) / 8;
        *(st ? &piece_base[q * chunks + c] : sink) = v;
    }

    // word i holds columns 4i..4i+3; piece i/2 holds columns 8(i/2)..8(i/2)+7
    __device__ static __forceinline__ float dot(const uint4 q, const uint4 *xp, float raw) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 xv = xp[i / 2];
            const uint32_t x01 = (i & 1) ? xv.z : xv.x;
            const uint32_t x23 = (i & 1) ? xv.w : xv.y;
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false), x01, raw);
            raw = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true), x23, raw);
        }
        return raw;
    }
    // the row scale is applied once, after the row's sum is complete
    __device__ static __forceinline__ float fold(float acc, float raw, Aux, float) { return acc + raw; }
};

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

// Sum every lane's V partials over the wave (V a power of two).  Step A adds lanes l and l^32
// (when V >= 2 the two halves of the wave keep different halves of the
// values), step B adds l and l^16 the same way, then a 16-lane row is summed
// by DPP rotations.  Afterwards the first lane of each 16-lane row holds
// CNT = max(V/4, 1) totals.  The tree of additions seen by a value does not
// depend on V, so a value's bits are the same whatever tile shape or batch
// carried it.  Must run with all 64 lanes active.
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

// ------------------------------------------------------------------ kernel

constexpr int pow2_ceil(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

template <class Fmt, int R, int B, int D>
struct Kernel {
    using Aux = typename Fmt::Aux;
    static constexpr int V = R * B;
    static constexpr int VP = pow2_ceil(V);     // WaveSum halves the count twice

    struct Buf {
        uint4 c[R];
        Aux a[R];
    };

    // bytes of dynamic LDS the kernel needs: activation pieces, per-chunk
    // sums, and a 32-byte sink for the stores of out-of-range staging lanes
    __host__ __device__ static constexpr int64_t lds_bytes(int chunks) {
        return int64_t(B) * Fmt::kPieces * chunks * 16 + (Fmt::kSums ? int64_t(B) * chunks * 4 : 0) + kLdsSink;
    }
};

template <class Fmt, int R, int B, int D>
__global__ void __launch_bounds__(512) qgemv_kernel(const Params p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    using K = Kernel<Fmt, R, B, D>;
    using Red = WaveSum<K::VP>;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves_per_block = blockDim.x >> 6;

    // workgroups are dispatched round-robin over the 8 XCDs; renumber them so
    // the workgroups of one XCD own neighbouring rows
    int lblock = blockIdx.x;
    if ((gridDim.x & 7) == 0) lblock = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int64_t wave = int64_t(lblock) * waves_per_block + wave_in_block;
    const int64_t r_begin = wave * p.n / p.total_waves;
    const int64_t r_end = (wave + 1) * p.n / p.total_waves;
    const int tiles = int((r_end - r_begin + R - 1) / R);
    const int passes = p.passes;
    const int steps = tiles * passes;

    typename K::Buf buf[D];

    // Every prefetch is issued unconditionally, so the number of loads that
    // follow a buffer is the same on every path and the compiler's wait
    // before consuming it only waits for that buffer.  Rows past the wave's
    // range are clamped to its own last row and chunks past the row end to
    // the row's last chunk: redundant re-reads of lines the same wave is
    // loading anyway, which consume() ignores.
    const int64_t row_hi = r_end > r_begin ? r_end - 1 : min(r_begin, p.n - 1);
    const int last_chunk = p.chunks - 1;
    auto issue = [&](typename K::Buf &b, int s) {
        const int t = s / passes;
        const int j = s - t * passes;
        const int c = min(lane + kWave * j, last_chunk);
        const uint32_t lane_off = uint32_t(c) * kChunkBytes;
        const int64_t row0 = r_begin + int64_t(t) * R;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t row = min(row0 + i, row_hi);
            const unsigned char *rp = p.codes + row * p.row_bytes;   // uniform
            b.c[i] = load_code_chunk(rp + lane_off);
            b.a[i] = Fmt::load_aux(p, row, c);
        }
    };

    // ---- stage x (and per-chunk sums) into LDS, overlapped with the prefetch.
    // Each thread first loads up to kXU activation units into registers, then
    // the weight prefetch is issued, and only then are the activation units
    // used: the vector-load counter retires in order, so waiting for the
    // activations does not wait for the weight loads issued after them.
    const int chunks = p.chunks;
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
        return *reinterpret_cast<const uint4 *>(p.x + int64_t(b) * p.k + (u - b * units_per_row) * 8);
    };
    // Every lane runs the same staging code and stores unconditionally (an
    // out-of-range unit is clamped to the last one and stored to the sink),
    // so no activation load is sunk into a conditional block below the
    // weight prefetch.
    auto stage_unit = [&](int u_in, const uint4 v) {
        constexpr int kUnitsPerChunk = Fmt::kWpc / 8;
        const bool st = u_in < x_units;
        const int u = st ? u_in : x_units - 1;
        const int b = u / units_per_row;
        const int e = (u - b * units_per_row) * 8;
        Fmt::stage(v, e, xs + b * Fmt::kPieces * chunks, chunks, sink, st);
        if constexpr (Fmt::kSums) {
            float sm = 0.0f;
            sm += bf16_to_f32(v.x & 0xFFFFu); sm += bf16_to_f32(v.x >> 16);
            sm += bf16_to_f32(v.y & 0xFFFFu); sm += bf16_to_f32(v.y >> 16);
            sm += bf16_to_f32(v.z & 0xFFFFu); sm += bf16_to_f32(v.z >> 16);
            sm += bf16_to_f32(v.w & 0xFFFFu); sm += bf16_to_f32(v.w >> 16);
            // the units of one chunk sit in consecutive lanes; units per row
            // and the wave width are multiples of the units per chunk
#pragma unroll
            for (int m = 1; m < kUnitsPerChunk; m <<= 1) sm += __shfl_xor(sm, m, kWave);
            *((st && (u % kUnitsPerChunk) == 0) ? &xsum[b * chunks + e / Fmt::kWpc] : sink_f) = sm;
        }
    };
    constexpr int kXU = 8;
    uint4 xr[kXU];
#pragma unroll
    for (int i = 0; i < kXU; ++i) xr[i] = x_unit(min(int(threadIdx.x) + i * int(blockDim.x), x_units - 1));

#pragma unroll
    for (int d = 0; d < D; ++d) issue(buf[d], d);

#pragma unroll
    for (int i = 0; i < kXU; ++i) stage_unit(int(threadIdx.x) + i * int(blockDim.x), xr[i]);
    // activations beyond kXU units per thread (k * batch above 8 * 8 * blockDim);
    // the trip count is the same for every lane of a wave
    for (int base = kXU * blockDim.x; base < x_units; base += blockDim.x) {
        const int u = base + threadIdx.x;
        stage_unit(u, x_unit(min(u, x_units - 1)));
    }
    __syncthreads();

    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;

    auto consume = [&](const typename K::Buf &bf, int s) {
        const int t = s / passes;
        const int j = s - t * passes;
        const int c = lane + kWave * j;
        const int64_t row0 = r_begin + int64_t(t) * R;
        if (c < chunks) {
            uint4 xp[B][Fmt::kPieces];
            float xsv[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
#pragma unroll
                for (int q = 0; q < Fmt::kPieces; ++q) xp[b][q] = xs[(b * Fmt::kPieces + q) * chunks + c];
                xsv[b] = Fmt::kSums ? xsum[b * chunks + c] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                if (row0 + i < r_end) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float raw = Fmt::dot(bf.c[i], xp[b], 0.0f);
                        acc[i][b] = Fmt::fold(acc[i][b], raw, bf.a[i], xsv[b]);
                    }
                }
            }
        }
        if (j == passes - 1) {
            // tile complete: wave-reduce the R x B partials and write y
            float v[K::VP];
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    v[i * B + b] = acc[i][b];
                    acc[i][b] = 0.0f;
                }
#pragma unroll
            for (int i = K::V; i < K::VP; ++i) v[i] = 0.0f;
            Red::run(v);
            if (Red::writer(lane)) {
#pragma unroll
                for (int q = 0; q < Red::kCnt; ++q) {
                    const int idx = Red::value_index(lane, q);
                    const int i = idx / B, b = idx % B;
                    const int64_t row = row0 + i;
                    if (idx < K::V && row < r_end) {
                        float out = v[q];
                        if constexpr (Fmt::kRowScale) {
                            // the buffer of the tile's last pass carries its rows' scales
                            float rs = bf.a[0].rs;
#pragma unroll
                            for (int ii = 1; ii < R; ++ii)
                                if (i == ii) rs = bf.a[ii].rs;
                            out *= rs;
                        }
                        if (p.out_bf16)
                            reinterpret_cast<uint16_t *>(p.y)[int64_t(b) * p.n + row] =
                                static_cast<uint16_t>(f32_to_bf16_rne(out));
                        else
                            reinterpret_cast<float *>(p.y)[int64_t(b) * p.n + row] = out;
                    }
                }
            }
        }
    };

    for (int s0 = 0; s0 < steps; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int s = s0 + d;
            if (s < steps) consume(buf[d], s);
            issue(buf[d], s + D);
        }
    }
}

}  // namespace qg
