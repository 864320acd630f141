// Block-quantized weight GEMM for more than four activation rows (a short
// prefill or a speculative-decoding batch): Y[m, n] = X[m, k] . W[n, k]^T with
// W as FP4-E2M1 codes and bf16 group scales, the layout the matvec reads.
//
// The weights are decoded in registers and fed to bf16 MFMA; nothing is
// written back to memory, so each weight byte is read from HBM once per 64
// activation rows.  ("Hand-Writing Gemma 4 ..." is about decode; the
// SharpInference issue, items C1 and C2, shows the trade-off for prefill: a
// dequantized fp16 copy of the weights fed to a library GEMM against an int8
// MMA kernel that reads the 4-bit weights once, and the second winning at
// short prompts.)
//
// A workgroup of four waves owns 64 weight rows (16 per wave) and up to 64
// activation rows (four blocks of 16).  K is walked in chunks of 256: the
// workgroup stages the chunk's activations and group scales in LDS while
// each wave's lanes load their own weight dwords, one chunk ahead.  One MFMA
// step (v_mfma_f32_16x16x32_bf16) covers 32 k, which lies inside one scale
// group (group sizes 32, 64, 128), so the group's raw sums come out of the
// MFMA accumulator and are scaled once: y += s . sum_{k in group} e2m1 . x.
//
// MFMA operand layout (checked on the device): lane l holds A[l%16][8(l/16)+i]
// and B[8(l/16)+i][l%16] for i < 8, and gets D[4(l/16)+v][l%16] for v < 4.
// A's rows are weight rows, B's columns are activation rows.
#pragma once

#include "qgemv_common.hpp"

namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct GemmParams {
    const unsigned char *codes;    // [n, k/2]: column 2j in the low nibble of byte j
    const uint16_t *scales;        // [n, k/gs] bf16
    const uint16_t *x;             // [m, k] bf16
    void *y;                       // [m, n] f32 or bf16
    int64_t n;
    int32_t k, m;
    int32_t groups;                // k / gs
    int32_t out_bf16;
};

constexpr int kGemmRows = 64;      // weight rows per workgroup, 16 per wave
constexpr int kGemmTokens = 64;    // activation rows per workgroup, 4 blocks of 16
constexpr int kGemmKC = 256;       // k per chunk: 8 MFMA steps of 32
constexpr int kGemmXPad = 8;       // LDS row padding (bf16) against bank conflicts

// SPG = MFMA steps per scale group (group size / 32): each group's steps form
// one straight-line chain of MFMAs from a zero accumulator, read once.
template <int SPG>
__global__ void __launch_bounds__(256) qgemm_fp4_kernel(const GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kGemmTokens][kGemmKC + kGemmXPad];
    __shared__ __attribute__((aligned(16))) uint16_t ss[kGemmKC / 32][kGemmRows];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid >> 6;
    const int g = lane >> 4;                       // k quarter of an MFMA step / D row quarter
    const int li = lane & 15;                      // A row / B column inside a block
    const int64_t rbase = int64_t(blockIdx.x) * kGemmRows;
    const int t0 = blockIdx.y * kGemmTokens;
    const int mt = min(kGemmTokens, p.m - t0);     // activation rows of this workgroup
    const int nblk = (mt + 15) >> 4;               // blocks of 16 in use (uniform)
    const int64_t row_bytes = p.k / 2;
    const int nch = (p.k + kGemmKC - 1) / kGemmKC;
    constexpr int gpc = kGemmKC / 32 / SPG;        // scale groups per chunk

    // this lane's weight row (rows past n read row n-1; their results are dropped)
    const int64_t arow = min(rbase + 16 * w + li, p.n - 1);
    const unsigned char *wrow = p.codes + arow * row_bytes;

    uint32_t wn[8];            // next chunk's weight dwords (one per MFMA step)
    uint4 xr[8];               // next chunk's activations, staged through registers
    uint16_t sr[2];            // next chunk's scales
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
        const int64_t kb = int64_t(c) * (kGemmKC / 2);        // byte offset of the chunk in a row
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            // a step past k reads the row's last 16 bytes instead (never used)
            const int64_t off = min(kb + 16 * s, row_bytes - 16) + 4 * g;
            wn[s] = *reinterpret_cast<const uint32_t *>(wrow + off);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int u = tid + 256 * j;                      // unit of 8 activations
            const int tt = u >> 5, ku = u & 31;
            const int kk = c * kGemmKC + ku * 8;
            const int tok = t0 + min(tt, mt - 1);
            xr[j] = kk < p.k ? load_x_unit(p.x + int64_t(tok) * p.k + kk) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + 256 * j;
            const int grp = e >> 6, r = e & 63;
            const int gg = c * gpc + grp;
            const int64_t row = min(rbase + r, p.n - 1);
            sr[j] = (grp < gpc && gg < p.groups) ? p.scales[row * p.groups + gg] : uint16_t(0);
        }
    };

    f32x4_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[b][v] = 0.0f;

    load_chunk(0);
    for (int c = 0; c < nch; ++c) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int u = tid + 256 * j;
            *reinterpret_cast<uint4 *>(&xs[u >> 5][(u & 31) * 8]) = xr[j];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + 256 * j;
            ss[e >> 6][e & 63] = sr[j];
        }
        __syncthreads();
        uint32_t wc[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) wc[s] = wn[s];
        if (c + 1 < nch) load_chunk(c + 1);

        // whole groups in this chunk (k is a multiple of the group size)
        const int ngr = min(8, (p.k - c * kGemmKC) / 32) / SPG;
#pragma unroll
        for (int gi = 0; gi < gpc; ++gi) {
            if (gi < ngr) {
                // 8 weights of row li per step, k = 32s + 8g + i: one dword, four pair conversions
                bf16x8_t a[SPG];
#pragma unroll
                for (int j = 0; j < SPG; ++j) {
                    const uint32_t q = wc[gi * SPG + j];
                    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0);
                    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1);
                    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2);
                    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3);
                    a[j] = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                                   __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
                }
                const uint2 sp = *reinterpret_cast<const uint2 *>(&ss[gi][16 * w + 4 * g]);
                const float sc[4] = {bf16_to_f32(sp.x & 0xFFFFu), bf16_to_f32(sp.x >> 16), bf16_to_f32(sp.y & 0xFFFFu),
                                     bf16_to_f32(sp.y >> 16)};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    if (b < nblk) {
                        f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int j = 0; j < SPG; ++j) {
                            const int s = gi * SPG + j;
                            const bf16x8_t xv = *reinterpret_cast<const bf16x8_t *>(&xs[16 * b + li][32 * s + 8 * g]);
                            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], xv, d, 0, 0, 0);
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[b][v] = fmaf(sc[v], d[v], acc[b][v]);
                    }
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int tok = t0 + 16 * b + li;
        if (b < nblk && tok < p.m) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = rbase + 16 * w + 4 * g + v;
                if (row < p.n) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t *>(p.y)[int64_t(tok) * p.n + row] =
                            static_cast<uint16_t>(f32_to_bf16_rne(acc[b][v]));
                    else
                        reinterpret_cast<float *>(p.y)[int64_t(tok) * p.n + row] = acc[b][v];
                }
            }
        }
    }
}

}  // namespace qg
