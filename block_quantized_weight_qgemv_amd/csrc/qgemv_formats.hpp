// Weight formats of the block-quantized matvec: in-register decode, the raw
// dot of one 16-byte code chunk, and the fold of the group parameters.
//
// A format describes
//   kWpc        weights per 16-byte code chunk
//   kRawUnits   16-byte units of bf16 activations per chunk (kWpc / 8)
//   kPieces     16-byte activation pieces per chunk as the dot reads them
//   kPpu        pieces per raw unit (kPieces / kRawUnits)
//   kSums       whether the fold needs the chunk's activation sum (affine)
//   kAuxArrays  per-group parameter arrays (0 FP8, 1 FP4, 2 affine)
//   kRowScale   whether rows carry one fp32 scale (FP8)
//   kSuper      whether the second parameter array holds one 32-bit word per
//               super-block of 8 chunks (the two-level format) instead of a
//               16-bit value per group
//   unit_pieces turns one raw unit of x into its kPpu pieces (reorders or
//               widens the activations to match the decode's output order)
//   dot         raw dot of one code chunk with the chunk's pieces
//   fold        acc + scale * raw (+ bias * chunk_sum)
//
// Prior art, not the blueprint: "Hand-Writing Gemma 4 Flash-Decoding + an FP4
// Matvec Bonus (Part 2)", section "The assumption that failed the profiler":
// decode by register permutes instead of a constant-memory table, and the
// group scale folded out of the per-weight math into one multiply-add.
#pragma once

#include "qgemv_common.hpp"

namespace qg {

// FP4-E2M1 codes, two per byte (even column in the low nibble), one bf16
// scale per group.  gfx950's scaled conversion turns the two codes of a byte
// into a bf16 pair in one instruction (scale 1: the E2M1 values are exact).
struct FmtFP4 {
    static constexpr int kWpc = 32;
    static constexpr int kRawUnits = 4;
    static constexpr int kPieces = 4;
    static constexpr int kPpu = 1;
    static constexpr bool kSums = false;
    static constexpr int kAuxArrays = 1;
    static constexpr bool kRowScale = false;
    static constexpr bool kSuper = false;

    // piece q holds columns 8q .. 8q+7 in natural order
    __device__ static __forceinline__ void unit_pieces(uint4 v, uint4 (&out)[kPpu]) { out[0] = v; }

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
    __device__ static __forceinline__ float fold(float acc, float raw, float s, float, float) {
        return fmaf(s, raw, acc);
    }
};

// Min-max affine 4-bit codes, u32 low-first, bf16 scale and bias per group.
// Masking the low and the high nibble of every byte leaves bytes q < 16, and
// such a byte read as E4M3 is exactly q * 2^-9 (subnormals and the first
// binade share the spacing 2^-9), so the FP8 converter yields exact bf16
// pairs (q0,q2),(q4,q6) and (q1,q3),(q5,q7) scaled by 2^-9.
struct FmtAffineU4 {
    static constexpr int kWpc = 32;
    static constexpr int kRawUnits = 4;
    static constexpr int kPieces = 4;
    static constexpr int kPpu = 1;
    static constexpr bool kSums = true;
    static constexpr int kAuxArrays = 2;
    static constexpr bool kRowScale = false;
    static constexpr bool kSuper = false;

    // piece q holds columns 8q..8q+7 reordered as (0,2),(4,6),(1,3),(5,7)
    __device__ static __forceinline__ void unit_pieces(uint4 v, uint4 (&out)[kPpu]) {
        out[0].x = (v.x & 0xFFFFu) | (v.y << 16);            // x0, x2
        out[0].y = (v.z & 0xFFFFu) | (v.w << 16);            // x4, x6
        out[0].z = (v.x >> 16) | (v.y & 0xFFFF0000u);        // x1, x3
        out[0].w = (v.z >> 16) | (v.w & 0xFFFF0000u);        // x5, x7
    }

    // word i holds the codes of columns 8i..8i+7 (code j at bits 4j)
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
    __device__ static __forceinline__ float fold(float acc, float raw, float s, float b, float xsum) {
        acc = fmaf(s * 512.0f, raw, acc);
        return fmaf(b, xsum, acc);
    }
};

// Two-level super-block 4-bit codes: the codes and their decode are those of
// the affine 4-bit format (u32 low-first nibbles); a 32-weight sub-block is
// one 16-byte chunk, with six-bit factors sc and m (one 16-bit word,
// sc | m << 8), and every 8 sub-blocks share a 32-bit word of fp16 d and
// dmin (d | dmin << 16).  The sub-block's weights are d*sc*q - dmin*m, so
// its scale is d*sc (exact in fp32: 11 x 6 bits) and its bias -dmin*m, folded
// as the affine bias through the chunk's activation sum.
//
// "perf(cuda): generalize Gemma 4 batched prefill + flash attn + decode
// graphs to dense Q4_K models", sections "Work Item C (C1) done" (the
// d*sc*nibble - dmin*mn decode) and "All work items complete" (the
// pre-unpacked scale layout of the decode matvec).
struct FmtQ4K : FmtAffineU4 {
    static constexpr bool kSuper = true;

    __device__ static __forceinline__ float f16_lo(uint32_t w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
    }
    // scale and bias of a sub-block from its factors and its super-block word
    __device__ static __forceinline__ void params(uint32_t sub16, uint32_t sup, float &s, float &b) {
        s = f16_lo(sup) * static_cast<float>(sub16 & 0xFFu);
        b = -(f16_lo(sup >> 16) * static_cast<float>((sub16 >> 8) & 0xFFu));
    }
};

// Min-max affine 8-bit codes, u32 low-first: bytes become f32 with the byte
// converters and meet f32 activations.
struct FmtAffineU8 {
    static constexpr int kWpc = 16;
    static constexpr int kRawUnits = 2;
    static constexpr int kPieces = 4;          // 16 activations as f32
    static constexpr int kPpu = 2;
    static constexpr bool kSums = true;
    static constexpr int kAuxArrays = 2;
    static constexpr bool kRowScale = false;
    static constexpr bool kSuper = false;

    // 8 bf16 (columns 8u..8u+7 of the chunk) become two f32 pieces
    __device__ static __forceinline__ void unit_pieces(uint4 v, uint4 (&out)[kPpu]) {
        out[0] = make_uint4(v.x << 16, v.x & 0xFFFF0000u, v.y << 16, v.y & 0xFFFF0000u);
        out[1] = make_uint4(v.z << 16, v.z & 0xFFFF0000u, v.w << 16, v.w & 0xFFFF0000u);
    }

    // word i holds the codes of columns 4i..4i+3, one byte each
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
    __device__ static __forceinline__ float fold(float acc, float raw, float s, float b, float xsum) {
        acc = fmaf(s, raw, acc);
        return fmaf(b, xsum, acc);
    }
};

// FP8-E4M3 (OCP) codes, one fp32 scale per row applied once to the row's sum.
struct FmtFP8 {
    static constexpr int kWpc = 16;
    static constexpr int kRawUnits = 2;
    static constexpr int kPieces = 2;          // 16 bf16
    static constexpr int kPpu = 1;
    static constexpr bool kSums = false;
    static constexpr int kAuxArrays = 0;
    static constexpr bool kRowScale = true;
    static constexpr bool kSuper = false;

    __device__ static __forceinline__ void unit_pieces(uint4 v, uint4 (&out)[kPpu]) { out[0] = v; }

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
    __device__ static __forceinline__ float fold(float acc, float raw, float, float, float) { return acc + raw; }
};

// Sum of the 8 bf16 activations of one raw unit, in f32.
__device__ __forceinline__ float unit_sum(const uint4 v) {
    float s = 0.0f;
    s += bf16_to_f32(v.x & 0xFFFFu); s += bf16_to_f32(v.x >> 16);
    s += bf16_to_f32(v.y & 0xFFFFu); s += bf16_to_f32(v.y >> 16);
    s += bf16_to_f32(v.z & 0xFFFFu); s += bf16_to_f32(v.z >> 16);
    s += bf16_to_f32(v.w & 0xFFFFu); s += bf16_to_f32(v.w >> 16);
    return s;
}

}  // namespace qg

namespace qg {

// Activation sum of one chunk from its raw units, with the addition tree the
// LDS staging uses (pairs of neighbouring units, then pairs of pairs), so both
// kernels fold bit-identical sums.
template <int U>
__device__ __forceinline__ float chunk_sum(const uint4 (&raw)[U]) {
    static_assert(U == 2 || U == 4, "chunks hold 2 or 4 raw units");
    if constexpr (U == 2) {
        return unit_sum(raw[0]) + unit_sum(raw[1]);
    } else {
        return (unit_sum(raw[0]) + unit_sum(raw[1])) + (unit_sum(raw[2]) + unit_sum(raw[3]));
    }
}

}  // namespace qg
