// Block-quantized weight GEMM for more than four activation rows (a short
// prefill or a speculative-decoding batch): Y[m, n] = X[m, k] . W[n, k]^T with
// W as FP4-E2M1 codes and bf16 group scales, or as min-max affine 4-bit codes
// with bf16 group scales and biases (kAffine), in the layouts the matvec
// reads.
//
// The weights are decoded in registers and fed to bf16 MFMA; nothing is
// written back to memory, so each weight byte is read from HBM once per 64
// activation rows.  ("Hand-Writing Gemma 4 ..." is about decode; the
// SharpInference issue, items C1 and C2, shows the trade-off for prefill: a
// dequantized fp16 copy of the weights fed to a library GEMM against an int8
// MMA kernel that reads the 4-bit weights once, and the second winning at
// short prompts.)
//
// A workgroup of four waves owns 64 weight rows (16 per wave) and 16, 32 or
// 64 activation rows (TB blocks of 16).  K is walked in chunks of 256: the
// workgroup stages each chunk's activations and group scales in LDS, and each
// wave's lanes load their own weight dwords, several chunks ahead through a
// ring of registers.  One MFMA
// step (v_mfma_f32_16x16x32_bf16) covers 32 k, which lies inside one scale
// group (group sizes 32, 64, 128), so the group's raw sums come out of the
// MFMA accumulator and are scaled once: y += s . sum_{k in group} e2m1 . x.
//
// MFMA operand layout (checked on the device): lane l holds A[l%16][8(l/16)+i]
// and B[8(l/16)+i][l%16] for i < 8, and gets D[4(l/16)+v][l%16] for v < 4.
// A's rows are weight rows, B's columns are activation rows.
#pragma once

#include "qgemv_common.hpp"
#include "qgemv_formats.hpp"

namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct GemmParams {
    const unsigned char *codes;    // [n, k/2]: column 2j in the low nibble of byte j
    const uint16_t *scales;        // [n, k/gs] bf16
    const uint16_t *biases;        // [n, k/gs] bf16 (affine 4-bit codes)
    const uint16_t *x;             // [m, k] bf16
    void *y;                       // [m, n] f32 or bf16
    int64_t n;
    int32_t k, m;
    int32_t groups;                // k / gs
    int32_t out_bf16;
};

constexpr int kGemmRows = 64;      // weight rows per workgroup, 16 per wave
constexpr int kGemmKC = 256;       // k per chunk: 8 MFMA steps of 32
constexpr int kGemmXPad = 8;       // LDS row padding (bf16) against bank conflicts

// chunks in flight per lane: the register ring holds PD chunks' loads (two
// with four K slices: 16 waves per workgroup hide the latency, and a deeper
// ring would not fit the 128 registers a 1024-thread workgroup leaves; one
// for the affine codes with 64 activation rows, whose second ring set, the
// sums' chains and the MFMA results would not fit 256 vector registers)
constexpr int gemm_depth(int tb, int ks, bool affine = false) {
    return ks == 4 ? 2 : (tb == 1 ? 4 : (tb == 2 ? 3 : (affine ? 1 : 2)));
}

// Exchange of a 4 x 4 block of dwords among lanes l, l + 16, l + 32, l + 48
// (index g = l >> 4): lane g's d[r] becomes lane r's d[g] before.  Two
// permlane32 swaps (lanes g and g + 2) then two permlane16 swaps (g and
// g + 1); swap32(a, b) trades a's upper 32 lanes for b's lower 32 lanes, and
// swap16(a, b) a's odd 16-lane rows for b's even rows.  All lanes active.
__device__ __forceinline__ void transpose4_lanes(uint4 &d) {
    auto sw32 = [](uint32_t &a, uint32_t &b) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    };
    auto sw16 = [](uint32_t &a, uint32_t &b) {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    };
    sw32(d.x, d.z);
    sw32(d.y, d.w);
    sw16(d.x, d.y);
    sw16(d.z, d.w);
}

// Whether qgemm_fp4_kernel double-buffers its staged chunks: for 16 or 32
// activation rows; with 64 the second buffer would halve the workgroups a CU
// holds (measured slower).
__host__ __device__ constexpr bool gemm_double_buffer(int tb) { return tb < 4; }

// SPG = MFMA steps per scale group (group size / 32): each group's steps form
// one straight-line chain of MFMAs from a zero accumulator, read once.
// TB = blocks of 16 activation rows per workgroup.
// KS = K slices: the workgroup has WPS KS waves, slice s (waves WPS s ..
// WPS s + WPS - 1) takes chunks s, s + KS, s + 2 KS, ... of the same 16 WPS
// rows, and the slices' sums are added in slice order at the end.
// WPS = waves per slice (4, or 1 where few row tiles would leave compute
// units idle; the order of additions is the same).  KS depends on n and k only, so a
// row's bits do not depend on the other activation rows.
//
// kAffine: min-max affine 4-bit codes (u32 low-first, the same nibble order
// as FP4) with a bf16 scale and bias per group.  The masked nibbles read as
// E4M3 are exactly q * 2^-9 (as in the matvec), in the column order (0, 2,
// 4, 6, 1, 3, 5, 7) of each 8, so x is staged in that order too; a group
// folds as y += (512 s) * raw + b * X, X the group's activation sum, which
// a second MFMA chain takes with A = 1 beside the weights' chain (exact
// products, fp32 sums, no vector work in the staging).
template <int SPG, int TB, int KS, int WPS, bool kAffine = false>
__global__ void __launch_bounds__(64 * WPS * KS) qgemm_fp4_kernel(const GemmParams p) {
    static_assert(KS * TB <= 4, "LDS holds KS chunks of 16 TB activation rows");
    constexpr int kTokens = 16 * TB;
    constexpr int ST = 64 * WPS;                   // threads per K slice
    constexpr int RW = 16 * WPS;                   // weight rows per workgroup
    static_assert((512 * TB) % ST == 0, "whole activation units per thread");
    constexpr int kXUnits = 512 * TB / ST;         // 16-byte activation units per thread per chunk
    constexpr int PD = gemm_depth(TB, KS, kAffine);
    constexpr int gpc = kGemmKC / 32 / SPG;        // scale groups per chunk
    // MFMA steps per batch of independent chains (affine, at 1024 threads:
    // half as many, its sums' chains beside them fit the 128 registers)
    constexpr int BS0 = kAffine && 64 * WPS * KS >= 1024 ? 4 / TB : 8 / TB;
    constexpr int BS = BS0 > SPG ? BS0 : SPG;
    constexpr int GB = BS / SPG;                   // scale groups per batch
    // LDS (dynamic, gemm_general_lds bytes): per K slice, buffers of a
    // chunk's activations and scales.  With two (DB), chunk i + 1 is staged
    // into one while chunk i is multiplied from the other, one barrier per
    // chunk; with 64 activation rows the second buffer would halve the
    // workgroups a CU holds, so those stage into one buffer between two
    // barriers.
    constexpr bool DB = gemm_double_buffer(TB);
    typedef uint16_t XBuf[kTokens][kGemmKC + kGemmXPad];
    typedef uint16_t SBuf[kGemmKC / 32][RW];
    constexpr int NB = (DB ? 2 : 1) * KS;          // buffers of each kind
    extern __shared__ __attribute__((aligned(16))) unsigned char gsmem[];
    XBuf *xsa = reinterpret_cast<XBuf *>(gsmem);                      // [2][KS]
    SBuf *ssa = reinterpret_cast<SBuf *>(gsmem + NB * sizeof(XBuf));   // [DB ? 2 : 1][KS]
    SBuf *bsa = ssa + NB;                                              // affine: biases, as the scales

    const int ks = threadIdx.x / ST;               // K slice
    const int tid = threadIdx.x % ST;              // thread in the slice
    const int lane = tid & (kWave - 1);
    const int w = tid >> 6;                        // wave in the slice: rows 16w..16w+15
    const int g = lane >> 4;                       // k quarter of an MFMA step / D row quarter
    const int li = lane & 15;                      // A row / B column inside a block
    const int64_t rbase = int64_t(blockIdx.x) * RW;
    const int t0 = blockIdx.y * kTokens;
    const int mt = min(kTokens, p.m - t0);         // activation rows of this workgroup
    const int nblk = (mt + 15) >> 4;               // blocks of 16 in use (uniform)
    const int64_t row_bytes = p.k / 2;
    const int nch = (p.k + kGemmKC - 1) / kGemmKC;
    const int nit = (nch + KS - 1) / KS;           // chunks per slice (the last may be short)

    // this lane's weight row (rows past n read row n-1; their results are dropped)
    const int64_t arow = min(rbase + 16 * w + li, p.n - 1);
    const unsigned char *wrow = p.codes + arow * row_bytes;

    // The ring: set d holds one chunk's weight dwords (one per MFMA step), the
    // thread's activation units and scales.  Every refill issues the same loads
    // (a chunk past the end reloads the last one, never used), so the
    // compiler's wait before a set is stored counts exactly the later sets.
    uint4 wn[PD][2];                               // 16-byte pieces 4j + g of the chunk row
    uint4 xr[PD][kXUnits];
    uint16_t sr[PD][2];
    uint16_t br[PD][kAffine ? 2 : 1];
    auto load_chunk = [&](int d, int c_in) __attribute__((always_inline)) {
        const int c = min(c_in, nch - 1);
        const int64_t kb = int64_t(c) * (kGemmKC / 2);        // byte offset of the chunk in a row
        // whole 16-byte pieces (4j + g) per lane; the MFMA layout (dword g of
        // every piece) comes from a 4 x 4 exchange among the row's four lanes
        // at consumption.  A piece past k reads the row's last 16 bytes
        // instead (never used).
#pragma unroll
        for (int j = 0; j < 2; ++j)
            wn[d][j] = *reinterpret_cast<const uint4 *>(wrow + min(kb + 16 * (4 * j + g), row_bytes - 16));
#pragma unroll
        for (int j = 0; j < kXUnits; ++j) {
            const int u = tid + ST * j;                       // unit of 8 activations
            const int tt = u >> 5, ku = u & 31;
            const int kk = min(c * kGemmKC + ku * 8, p.k - 8);   // past k: a unit never used
            const int tok = t0 + min(tt, mt - 1);
            xr[d][j] = load_x_unit(p.x + int64_t(tok) * p.k + kk);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + ST * j;
            const int grp = e / RW, r = e % RW;
            const int gg = min(c * gpc + min(grp, gpc - 1), p.groups - 1);
            const int64_t row = min(rbase + r, p.n - 1);
            sr[d][j] = p.scales[row * p.groups + gg];
            if constexpr (kAffine) br[d][j] = p.biases[row * p.groups + gg];
        }
    };

    f32x4_t acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[b][v] = 0.0f;

    // the ring is filled chunk by chunk: the scheduler may not interleave the
    // chunks' loads, or the first set's loads would no longer be the oldest
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        load_chunk(d, d * KS + ks);
        __builtin_amdgcn_sched_barrier(0);
    }
    // stage ring set d (chunk c of this slice) into buffer par; stored
    // whether the chunk exists or not (a branch here would cost the compiler
    // its count of the loads in flight: it would drain them)
    auto stage = [&](int d, int c, int par) __attribute__((always_inline)) {
        XBuf &xw = xsa[par * KS + ks];
        SBuf &sw = ssa[par * KS + ks];
#pragma unroll
        for (int j = 0; j < kXUnits; ++j) {
            const int u = tid + ST * j;
            const int kk = c * kGemmKC + (u & 31) * 8;
            // units past k are stored as zeros (the MFMA of a partial last
            // chunk stops at a whole group, but LDS stays defined)
            uint4 v = kk < p.k ? xr[d][j] : make_uint4(0, 0, 0, 0);
            if constexpr (kAffine) {
                uint4 pc[1];
                FmtAffineU4::unit_pieces(v, pc);
                v = pc[0];
            }
            *reinterpret_cast<uint4 *>(&xw[u >> 5][(u & 31) * 8]) = v;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + ST * j;
            sw[e / RW][e % RW] = sr[d][j];
            if constexpr (kAffine) bsa[par * KS + ks][e / RW][e % RW] = br[d][j];
        }
    };
    if constexpr (DB) {
        stage(0, ks, 0);
        __syncthreads();
    }
    for (int c0 = 0; c0 < nit; c0 += PD) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            const int i = c0 + d;                             // chunk of this slice, in order
            const int c = i * KS + ks;                        // chunk of the row
            const bool active = c < nch;                      // uniform in the wave
            const int par = DB ? (i & 1) : 0;
            if constexpr (DB) {
                // the next chunk (ring set d + 1) into the other buffer: every
                // wave finished reading it before the last barrier
                stage((d + 1) % PD, (i + 1) * KS + ks, par ^ 1);
            } else {
                stage(d, c, 0);
                __syncthreads();
            }
            const XBuf &xs = xsa[par * KS + ks];
            const SBuf &ss = ssa[par * KS + ks];
            uint4 wp[2] = {wn[d][0], wn[d][1]};
            load_chunk(d, c + PD * KS);
            transpose4_lanes(wp[0]);
            transpose4_lanes(wp[1]);
            const uint32_t wc[8] = {wp[0].x, wp[0].y, wp[0].z, wp[0].w, wp[1].x, wp[1].y, wp[1].z, wp[1].w};
            if (active) {
                // The chunk's MFMA chains (one per scale group and block of 16
                // activation rows) go out back to back, BS steps at a time,
                // and their sums are read and scaled afterwards: a result read
                // right behind its MFMA would stall each step for the MFMA's
                // whole latency.  The code has no branch: in a partial last
                // chunk the groups past k multiply the zeros staged for them
                // (the weights there are finite E2M1 codes read in bounds),
                // and blocks past m are computed but never stored.
#pragma unroll
                for (int s0 = 0; s0 < 8; s0 += BS) {
                    f32x4_t dd[GB][TB];
                    f32x4_t xg[kAffine ? GB : 1][kAffine ? TB : 1];   // affine: the group's activation sums
#pragma unroll
                    for (int gb = 0; gb < GB; ++gb) {
                        // 8 weights of row li per step, k = 32s + 8g + i: one dword, four pair conversions
                        bf16x8_t a[SPG];
#pragma unroll
                        for (int j = 0; j < SPG; ++j) {
                            const uint32_t q = wc[s0 + gb * SPG + j];
                            bf16x2_t p0, p1, p2, p3;
                            if constexpr (kAffine) {
                                const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
                                p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
                                p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
                                p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
                                p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
                            } else {
                                p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0);
                                p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1);
                                p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2);
                                p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3);
                            }
                            a[j] = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                                           __builtin_shufflevector(p2, p3, 0, 1, 2, 3),
                                                           0, 1, 2, 3, 4, 5, 6, 7);
                        }
#pragma unroll
                        for (int b = 0; b < TB; ++b) {
                            f32x4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f};
                            f32x4_t o0 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                            for (int j = 0; j < SPG; ++j) {
                                const int s = s0 + gb * SPG + j;
                                const bf16x8_t xv =
                                    *reinterpret_cast<const bf16x8_t *>(&xs[16 * b + li][32 * s + 8 * g]);
                                d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], xv, d0, 0, 0, 0);
                                if constexpr (kAffine) {
                                    const bf16x8_t ones = {__bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f),
                                                           __bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f)};
                                    o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, xv, o0, 0, 0, 0);
                                }
                            }
                            dd[gb][b] = d0;
                            if constexpr (kAffine) xg[gb][b] = o0;
                        }
                    }
#pragma unroll
                    for (int gb = 0; gb < GB; ++gb) {
                        const int gi = s0 / SPG + gb;
                        const uint2 sp = *reinterpret_cast<const uint2 *>(&ss[gi][16 * w + 4 * g]);
                        const float sc[4] = {bf16_to_f32(sp.x & 0xFFFFu), bf16_to_f32(sp.x >> 16),
                                             bf16_to_f32(sp.y & 0xFFFFu), bf16_to_f32(sp.y >> 16)};
                        if constexpr (kAffine) {
                            const uint2 bp =
                                *reinterpret_cast<const uint2 *>(&bsa[par * KS + ks][gi][16 * w + 4 * g]);
                            const float bi[4] = {bf16_to_f32(bp.x & 0xFFFFu), bf16_to_f32(bp.x >> 16),
                                                 bf16_to_f32(bp.y & 0xFFFFu), bf16_to_f32(bp.y >> 16)};
#pragma unroll
                            for (int b = 0; b < TB; ++b) {
                                // (every element of the sums' D is activation row 16b + li's sum)
                                const float xsg = xg[gb][b][0];
#pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    acc[b][v] = fmaf(sc[v] * 512.0f, dd[gb][b][v], acc[b][v]);
                                    acc[b][v] = fmaf(bi[v], xsg, acc[b][v]);
                                }
                            }
                        } else {
#pragma unroll
                            for (int b = 0; b < TB; ++b)
#pragma unroll
                                for (int v = 0; v < 4; ++v) acc[b][v] = fmaf(sc[v], dd[gb][b][v], acc[b][v]);
                        }
                    }
                }
            }
            __syncthreads();
        }
    }

    if constexpr (KS > 1) {
        // slices 1.. leave their sums in LDS (over the staged chunks, free
        // after the loop's last barrier); slice 0 adds them in slice order
        f32x4_t *red = reinterpret_cast<f32x4_t *>(gsmem);
        static_assert((DB ? 2 : 1) * KS * sizeof(XBuf) >= (KS - 1) * WPS * TB * 64 * sizeof(f32x4_t), "reduction space");
        if (ks > 0) {
#pragma unroll
            for (int b = 0; b < TB; ++b) red[(((ks - 1) * WPS + w) * TB + b) * 64 + lane] = acc[b];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                const f32x4_t o = red[(((q - 1) * WPS + w) * TB + b) * 64 + lane];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[b][v] += o[v];
            }
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
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

// LDS bytes of qgemm_fp4_kernel<SPG, TB, KS, WPS, kAffine>: one or two
// buffers per K slice of a chunk's activations and scales (and, affine, its
// biases)
__host__ __device__ constexpr int64_t gemm_general_lds(int tb, int ks, int wps, bool affine = false) {
    return (gemm_double_buffer(tb) ? 2 : 1) * int64_t(ks) *
           (16 * tb * (kGemmKC + kGemmXPad) * 2 + (affine ? 2 : 1) * (kGemmKC / 32) * 16 * wps * 2);
}

// ------------------------------------------------------------------ m <= 16

// Up to 16 activation rows, whose x (m rows, k rounded up to whole 256-wide
// chunks, zeros past k) fits in LDS: the workgroup stages all of x once, and
// each wave then streams its own 16-row weight tiles with no barrier, loads
// running several chunks ahead in a register ring.  The MFMA takes x as A
// (rows = activation rows) and the weights as B, so lane l gets
// D[4(l/16)+v][l%16] = the sums of activation rows 4(l/16)+v for weight row
// l%16: the weight row whose codes and group scale the lane loaded itself.
//
// The order of every addition is that of qgemm_fp4_kernel with the same KS
// (which depends on n and k alone): chunk c is summed into slice c % KS, a
// group's MFMA chain starts from zero and is scaled into its slice in group
// order, and the slices are added in slice order at the end.  The MFMA
// operands of a group are the same values in both kernels.  So a row's bits
// are the same whichever kernel, m or launch computes it.
//
// kAffine: the affine 4-bit codes, as in qgemm_fp4_kernel: x staged in the
// decode's column order, the codes decoded to q * 2^-9, a second MFMA chain
// per group with B = 1 giving each activation row's group sum, and the fold
// y += (512 s) * raw + b * X in group order.
constexpr int kGemmSmallWaves = 8;                 // most waves per workgroup
// chunks in flight per lane (8 measured slower, with eight waves per CU and
// with two or four)
constexpr int kGemmSmallDepth = 4;

// VS: a chunk's gpc group scales of a row are read as one vector (they are
// aligned to 2 * gpc bytes when the groups per row are a multiple of gpc).
template <int SPG, int KS, bool VS, bool kAffine = false>
__global__ void __launch_bounds__(64 * kGemmSmallWaves) qgemm_fp4_small_kernel(const GemmParams p) {
    constexpr int gpc = kGemmKC / 32 / SPG;        // scale groups per chunk
    constexpr int PD = kGemmSmallDepth;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;                       // k quarter of an MFMA step; D row quarter
    const int li = lane & 15;                      // A row (activation row) and B column (weight row)
    const int nch = (p.k + kGemmKC - 1) / kGemmKC;
    const int xstride = nch * kGemmKC + kGemmXPad; // bf16 per staged activation row
    const int64_t row_bytes = p.k / 2;

    // 16-row tiles split evenly over the grid's waves (contiguous ranges);
    // a wave's items are its tiles' chunks in order
    const int64_t tiles = (p.n + 15) / 16;
    const int wpb = blockDim.x >> 6;
    const int64_t gw = int64_t(blockIdx.x) * wpb + wave_in_block();
    const int64_t nw = int64_t(gridDim.x) * wpb;
    const int64_t tb = gw * tiles / nw, te = (gw + 1) * tiles / nw;
    const int items = int(te - tb) * nch;
    // activation row this lane's A operand reads (rows past m repeat row
    // m - 1: their sums are never stored)
    const uint16_t *xrow = xs + min(li, p.m - 1) * xstride + 8 * g;

    struct Buf {
        uint4 w[2];                                // 16-byte pieces 4j + g of the chunk row
        uint32_t sc[gpc];                          // the lane's row's group scales (bf16 bits)
        uint32_t bi[kAffine ? gpc : 1];            // affine: its group biases (bf16 bits)
    };
    typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
    typedef unsigned short u16x4_t __attribute__((ext_vector_type(4)));
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    auto issue = [&](Buf &bf, int item_in) __attribute__((always_inline)) {
        const int item = __builtin_amdgcn_readfirstlane(min(item_in, max(items - 1, 0)));
        const int tq = __builtin_amdgcn_readfirstlane(item / nch);
        const int c = item - tq * nch;
        // rows past n read row n - 1; pieces past k read the row's last 16
        // bytes (their activations are zeros).  Each lane reads whole 16-byte
        // pieces (piece 4j + g of its row's chunk); the MFMA's layout (dword
        // g of every piece) comes from a 4 x 4 exchange among the four lanes
        // of the row at consumption.
        const int64_t row = min((tb + tq) * 16 + li, p.n - 1);
        const unsigned char *wrow = p.codes + row * row_bytes;
        const int64_t kb = int64_t(c) * (kGemmKC / 2);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf.w[j] = *reinterpret_cast<const uint4 *>(wrow + min(kb + 16 * (4 * j + g), row_bytes - 16));
        // the chunk's group parameters of the row (as one vector with VS: the
        // row's last gpc groups past the end)
        auto params = [&](const uint16_t *arr, uint32_t (&out)[gpc]) __attribute__((always_inline)) {
            const uint16_t *srow = arr + row * p.groups;
            if constexpr (VS) {
                const int g0 = min(c * gpc, p.groups - gpc);
                if constexpr (gpc == 8) {
                    const u16x8_t v = *reinterpret_cast<const u16x8_t *>(srow + g0);
#pragma unroll
                    for (int j = 0; j < 8; ++j) out[j] = v[j];
                } else if constexpr (gpc == 4) {
                    const u16x4_t v = *reinterpret_cast<const u16x4_t *>(srow + g0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) out[j] = v[j];
                } else {
                    const u16x2_t v = *reinterpret_cast<const u16x2_t *>(srow + g0);
#pragma unroll
                    for (int j = 0; j < 2; ++j) out[j] = v[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < gpc; ++j) out[j] = srow[min(c * gpc + j, p.groups - 1)];
            }
        };
        params(p.scales, bf.sc);
        if constexpr (kAffine) params(p.biases, bf.bi);
    };

    f32x4_t acc[KS];
#pragma unroll
    for (int q = 0; q < KS; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[q][v] = 0.0f;

    auto consume = [&](const Buf &bf_in, int item) __attribute__((always_inline)) {
        const int tq = __builtin_amdgcn_readfirstlane(item / nch);
        const int c = item - tq * nch;
        Buf bf = bf_in;
        // dword g of each MFMA step's 16-byte piece: w[s] below
        transpose4_lanes(bf.w[0]);
        transpose4_lanes(bf.w[1]);
        const uint32_t wst[8] = {bf.w[0].x, bf.w[0].y, bf.w[0].z, bf.w[0].w,
                                 bf.w[1].x, bf.w[1].y, bf.w[1].z, bf.w[1].w};
        // past the end of a partial chunk the vector scales belong to the
        // row's last groups: those groups multiply zeros, as do the general
        // kernel's (whose scale there is the last group's)
        // every group's chain first, then the folds in group order
        f32x4_t dd[gpc];
        f32x4_t xg[kAffine ? gpc : 1];             // affine: each activation row's group sums
#pragma unroll
        for (int j = 0; j < gpc; ++j) {
            f32x4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4_t o0 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < SPG; ++t) {
                const int s = j * SPG + t;
                const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(xrow + c * kGemmKC + 32 * s);
                const uint32_t q = wst[s];
                bf16x2_t p0, p1, p2, p3;
                if constexpr (kAffine) {
                    const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
                    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
                    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
                    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
                    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
                } else {
                    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0);
                    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1);
                    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2);
                    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3);
                }
                const bf16x8_t wb = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                                            __builtin_shufflevector(p2, p3, 0, 1, 2, 3),
                                                            0, 1, 2, 3, 4, 5, 6, 7);
                d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, d0, 0, 0, 0);
                if constexpr (kAffine) {
                    const bf16x8_t ones = {__bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f),
                                           __bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f)};
                    o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ones, o0, 0, 0, 0);
                }
            }
            dd[j] = d0;
            if constexpr (kAffine) xg[j] = o0;
        }
        auto fold = [&](f32x4_t &a) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < gpc; ++j) {
                const float sv = bf16_to_f32(bf.sc[j] & 0xFFFFu);
                if constexpr (kAffine) {
                    const float bv = bf16_to_f32(bf.bi[j] & 0xFFFFu);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        a[v] = fmaf(sv * 512.0f, dd[j][v], a[v]);
                        a[v] = fmaf(bv, xg[j][v], a[v]);
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v) a[v] = fmaf(sv, dd[j][v], a[v]);
                }
            }
        };
        if constexpr (KS == 1) {
            fold(acc[0]);
        } else {
            const int sl = c % KS;                 // uniform
#pragma unroll
            for (int q = 0; q < KS; ++q)
                if (sl == q) fold(acc[q]);
        }
        if (c == nch - 1) {
            f32x4_t tot = acc[0];
#pragma unroll
            for (int q = 1; q < KS; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) tot[v] += acc[q][v];
            const int64_t row = (tb + tq) * 16 + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = 4 * g + v;
                if (tok < p.m && row < p.n) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t *>(p.y)[int64_t(tok) * p.n + row] =
                            static_cast<uint16_t>(f32_to_bf16_rne(tot[v]));
                    else
                        reinterpret_cast<float *>(p.y)[int64_t(tok) * p.n + row] = tot[v];
                }
            }
#pragma unroll
            for (int q = 0; q < KS; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[q][v] = 0.0f;
        }
    };

    // the ring: buffers hold items in increasing order; refills past the end
    // reload the last item (never consumed)
    Buf buf[PD];
    int sl[PD];
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        sl[d] = d;
        issue(buf[d], d);
    }
    // (the ring's weight loads go out first: they do not depend on x, and
    // arrive while x is staged; the fence keeps the compiler from sinking
    // them to their first use)
    issue_fence();
    // x -> LDS once: m rows, zeros from k to the end of the last chunk;
    // kStage loads in flight per thread (one at a time, every thread would
    // wait out the load latency once per unit)
    constexpr int kStage = 16;
    const int upr = xstride / 8;                   // 16-byte units per staged row
    const int units = p.m * upr;
    for (int u0 = threadIdx.x; u0 < units; u0 += kStage * int(blockDim.x)) {
        uint4 v[kStage];
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int u = min(u0 + i * int(blockDim.x), units - 1);
            const int t = u / upr, ku = (u - t * upr) * 8;
            v[i] = load_x_unit(p.x + int64_t(t) * p.k + min(ku, p.k - 8));
        }
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int u = u0 + i * int(blockDim.x);
            if (u < units) {
                const int t = u / upr, ku = (u - t * upr) * 8;
                uint4 vv = ku < p.k ? v[i] : make_uint4(0u, 0u, 0u, 0u);
                if constexpr (kAffine) {
                    uint4 pc[1];
                    FmtAffineU4::unit_pieces(vv, pc);
                    vv = pc[0];
                }
                *reinterpret_cast<uint4 *>(xs + t * xstride + ku) = vv;
            }
        }
    }
    __syncthreads();

    while (sl[PD - 1] < items) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            consume(buf[d], sl[d]);
            sl[d] += PD;
            issue(buf[d], sl[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < PD - 1; ++d)
        if (sl[d] < items) consume(buf[d], sl[d]);
}

// LDS bytes of qgemm_fp4_small_kernel's staged activations
__host__ __device__ constexpr int64_t gemm_small_lds(int64_t k, int m) {
    return int64_t(m) * (((k + kGemmKC - 1) / kGemmKC) * kGemmKC + kGemmXPad) * 2;
}

}  // namespace qg
