// The int8 activation route for affine 4-bit and 8-bit weights: the
// activation is quantized in blocks of 32 to int8 codes with an fp16 pair
// {d, s} in one 32-bit word (d in the low half, s = d * sum q in the high
// half), the weight codes are widened to int8 bytes (4-bit: nibble masks;
// 8-bit: c - 128 by flipping the top bit) and meet the activation codes in
// 4-wide integer dots, and the affine bias is applied once per block
// through s.
//
// Prior art, not the blueprint: "perf(cuda): generalize Gemma 4 batched
// prefill + flash attn + decode graphs to dense Q4_K models", section
// "Item C2" (int8 q8_1 blocks whose ds word carries d and, in its high half,
// the fp16 activation sum s; nibbles widened to int8; the min term applied
// through the activation sum).  There it feeds int8 matrix products and a
// 4-wide integer-dot matvec; here it is the matvec, on gfx950's
// v_dot4_i32_i8.
//
// A block of 32 weights is one 16-byte chunk of 4-bit codes or two of 8-bit
// codes, and its fold is  acc += scale * (d * idot) + bias * s, with idot the
// exact integer sum of code times activation code (8-bit: two halves, each
// taken as a dot of c - 128 plus 128 times the half's activation-code sum).

#include "qgemv.h"
#include "qgemv_kernels.hpp"
#include "qgemv_device.hpp"

#include <mutex>

namespace qg {

constexpr int kQ8Block = 32;
constexpr int kQuadXor1 = 0xB1;      // DPP quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;      // DPP quad_perm [2, 3, 0, 1]

// ------------------------------------------------------------------ quantize

// fp32 -> fp16 bits, round to nearest even (the hardware conversion in the
// default rounding mode; overflow gives infinity), and back (exact).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// One lane's share of a block of 32 activations: eight bf16 values w of a
// block held by four consecutive lanes (lanes 4m..4m+3; every lane of the
// wave calls this together).  amax is a max over the four lanes; the block
// stores d = fp16_rne(amax / 127), its codes are rne(x / d) with that stored
// d, clamped to +-127 (0 when d is 0), and s = fp16_rne(d * sum(q)) (an
// integer sum over the four lanes; d * sum is exact in fp32).  amax / 127 is
// a correctly rounded fp32 division: a quotient of a bf16 by 127 is never
// within fp32 rounding of an fp16 midpoint unless it lies on it.  The codes
// come from rne_quotient below.  Every decision is the exact-arithmetic one,
// and the result does not depend on how the block is split.  packed holds the
// lane's eight codes in column order; ds is the block's {d, s} word.
//
// rne_quotient: rne(v / d) for a bf16 v and an fp16-valued d > 0 with
// |v / d| <= 128, given r4096 = 4096 * rcp(d), rcp within an ulp of 1 / d.
// v * r4096 is 4096 * v / d to within 2^-4.4, so its rint t is the integer
// nearest 4096 * v / d whenever that value is not within 0.05 of a
// half-integer, and t / 4096 is exact.  A quotient of a bf16 by an fp16 value
// is either a half-integer or more than 2^-12 from every half-integer (write
// both over the coarser of their last-bit units), so t / 4096 equals v / d
// when v / d is a half-integer and lies on the same side of every
// half-integer as v / d otherwise: its rint (ties to even) is rne(v / d).
// (Checked exhaustively on the CPU over every fp16 d and every bf16 v in
// range, with rcp rounded to nearest and one ulp either way.)
__device__ __forceinline__ float rne_quotient(float v, float r4096) {
    return __builtin_rintf(__builtin_rintf(v * r4096) * 0x1p-12f);
}

__device__ __forceinline__ void quantize_unit(const uint4 w, uint32_t (&packed)[2], uint32_t &ds) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(ws[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(ws[i] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // quad permutes (lanes l ^ 1, then l ^ 2) as DPP moves
    amax = fmaxf(amax, dpp_f<kQuadXor1>(amax));
    amax = fmaxf(amax, dpp_f<kQuadXor2>(amax));
    const uint32_t dh = f32_to_f16_bits(__fdiv_rn(amax, 127.0f));
    const float d = f16_bits_to_f32(dh);
    const bool live = d > 0.0f;
    const float r4096 = __builtin_amdgcn_rcpf(live ? d : 1.0f) * 4096.0f;
    int sum = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float r = live ? fminf(fmaxf(rne_quotient(v[4 * h + j], r4096), -127.0f), 127.0f) : 0.0f;
            const int qi = int(r);
            sum += qi;
            word |= (uint32_t(qi) & 0xFFu) << (8 * j);
        }
        packed[h] = word;
    }
    sum += __builtin_amdgcn_update_dpp(0, sum, kQuadXor1, 0xF, 0xF, false);
    sum += __builtin_amdgcn_update_dpp(0, sum, kQuadXor2, 0xF, 0xF, false);
    ds = dh | (f32_to_f16_bits(d * float(sum)) << 16);
}

// One lane per 8 activations (a block is four consecutive lanes).  Threads
// past the last unit compute on a clamped unit and store nothing; the four
// lanes of a block are always in range together (units come in fours).
__global__ void __launch_bounds__(256) qg_quantize_q8_kernel(const uint16_t *__restrict__ x, int64_t units,
                                                             int8_t *__restrict__ xq, uint32_t *__restrict__ ds) {
    const int64_t u_in = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool live = u_in < units;
    const int64_t u = live ? u_in : units - 1;
    uint32_t packed[2], dsw;
    quantize_unit(*reinterpret_cast<const uint4 *>(x + u * 8), packed, dsw);
    if (live) {
        *reinterpret_cast<uint2 *>(xq + u * 8) = make_uint2(packed[0], packed[1]);
        if ((u & 3) == 0) ds[u >> 2] = dsw;
    }
}

// ------------------------------------------------------------------ matvec

struct Q8Args {
    const int8_t *xq;       // int8 [B, k], natural order
    const uint32_t *ds;     // {d, s} fp16 pairs [B, k/32], d in the low half
    const uint16_t *x;      // bf16 [B, k], quantized in the staging (kFuse)
};

// Bytes 0..3 and 4..7 of an 8-column group (x0..x7) regrouped as the even
// columns (x0, x2, x4, x6) and the odd ones (x1, x3, x5, x7): the order in
// which the masked low and high nibbles of a code word hold their columns.
__device__ __forceinline__ uint2 even_odd(uint32_t lo4, uint32_t hi4) {
    return make_uint2(__builtin_amdgcn_perm(hi4, lo4, 0x06040200u), __builtin_amdgcn_perm(hi4, lo4, 0x07050301u));
}

// Integer dot of one chunk of u4 codes (word i: columns 8i..8i+7, code j at
// bits 4j) with the chunk's activation codes, as two regrouped 16-byte pieces
// (piece p: .x/.y even/odd of columns 16p..16p+7, .z/.w of 16p+8..16p+15).
__device__ __forceinline__ int dot_u4_i8(const uint4 q, const uint4 (&xp)[2]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 p = xp[i >> 1];
        const uint32_t ev = (i & 1) ? p.z : p.x;
        const uint32_t od = (i & 1) ? p.w : p.y;
        acc = __builtin_amdgcn_sdot4(int(w[i] & 0x0F0F0F0Fu), int(ev), acc, false);
        acc = __builtin_amdgcn_sdot4(int((w[i] >> 4) & 0x0F0F0F0Fu), int(od), acc, false);
    }
    return acc;
}

// Integer dot of one 16-byte piece of 8-bit codes (half a block; word i:
// columns 4i..4i+3 of the piece, one byte each) with the matching 16
// activation codes in natural order.  Flipping a byte's top bit turns code c
// into the signed byte c - 128; the caller adds 128 * sum(q) back.
__device__ __forceinline__ int dot_u8_i8(const uint4 q, const uint4 xp) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const uint32_t x[4] = {xp.x, xp.y, xp.z, xp.w};
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_sdot4(int(w[i] ^ 0x80808080u), int(x[i]), acc, false);
    return acc;
}

// Sum of the 16 signed activation codes of a piece (4-wide dots with ones).
__device__ __forceinline__ int code_sum_i8(const uint4 xp) {
    int acc = __builtin_amdgcn_sdot4(int(xp.x), 0x01010101, 0, false);
    acc = __builtin_amdgcn_sdot4(int(xp.y), 0x01010101, acc, false);
    acc = __builtin_amdgcn_sdot4(int(xp.z), 0x01010101, acc, false);
    return __builtin_amdgcn_sdot4(int(xp.w), 0x01010101, acc, false);
}

__host__ __device__ constexpr int64_t q8_lds_bytes(int64_t batch, int64_t chunks) {
    return batch * chunks * (2 * 16 + 4);
}

// Waves take contiguous row ranges (wave_rows); a step is one pass of 64
// 16-byte code pieces (one per lane, so every load is contiguous) over an
// R-row tile, D steps in flight.  Bits is the code width, 4 or 8: a block of
// 32 weights is one piece or two, and with two the lanes of a pair share the
// block's {d, s} and only the first adds the bias term.  The workgroup first
// stages every batch row's activation codes (for 4-bit weights regrouped into
// even and odd columns) and {d, s} pairs in LDS, piece-major so that
// consecutive lanes read consecutive 16 bytes.
template <int Bits, int R, int B, int D, bool kFuse>
__global__ void __launch_bounds__(512) qgemv_affine_q8_kernel(const Params p, const Q8Args a) {
    constexpr int PPB = Bits / 4;            // 16-byte code pieces per block
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    struct Buf {
        uint4 c[R];
        uint32_t s[R], b[R];
    };
    const int lane = threadIdx.x & (kWave - 1);
    const int chunks = p.chunks;
    uint4 *xl = reinterpret_cast<uint4 *>(smem);                                   // [B][2][chunks]
    uint32_t *dl = reinterpret_cast<uint32_t *>(smem + int64_t(B) * chunks * 32); // [B][chunks]

    int64_t r_begin, r_end;
    wave_rows(p, r_begin, r_end);
    const int tiles = int((r_end - r_begin + R - 1) / R);
    const int passes = p.passes;
    const int steps = tiles * passes;
    const int64_t row_hi = r_end > r_begin ? r_end - 1 : min(r_begin, p.n - 1);
    const int pieces = chunks * PPB;         // code pieces per row

    auto issue = [&](Buf &bf, int s) {
        const int t = s / passes;
        const int j = s - t * passes;
        const int pc = min(lane + kWave * j, pieces - 1);
        const int64_t row0 = r_begin + int64_t(t) * R;
        const int g = (pc / PPB) >> p.group_shift;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t row = min(row0 + i, row_hi);
            bf.c[i] = load_code_chunk(p.codes + row * p.row_bytes + uint32_t(pc) * kChunkBytes);
            bf.s[i] = load_param(p.scales + row * p.groups + g);
            bf.b[i] = load_param(p.biases + row * p.groups + g);
        }
    };

    Buf buf[D];
    if constexpr (kFuse) {
        // Quantize x into LDS: a lane per 8 activations (16 bytes of bf16),
        // the first kSX units per thread loaded before the weight prefetch
        // as in the other branch.  Every lane runs quantize_unit (its block's
        // four lanes together); only in-range units are stored.
        constexpr int kSX = 4;
        const int nt = int(blockDim.x), tid = int(threadIdx.x);
        const int upr = p.k / 8;
        const int units = B * upr;
        const rsrc_t rxb = make_rsrc(a.x, uint32_t(units) * 16u);
        auto load_u = [&](int u) -> uint4 {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rxb, int(u < units ? uint32_t(u) * 16u : kOutOfRange), 0, 0);
            return make_uint4(v.x, v.y, v.z, v.w);
        };
        auto quant_store = [&](int u, const uint4 w) {
            uint32_t packed[2], dsw;
            quantize_unit(w, packed, dsw);
            if (u < units) {
                const int b = u / upr;
                const int e = u - b * upr;           // 8-column unit in the row
                const int c = e >> 2, h = e & 3;     // chunk, 8-column group in it
                const uint2 eo = Bits == 4 ? even_odd(packed[0], packed[1]) : make_uint2(packed[0], packed[1]);
                reinterpret_cast<uint2 *>(&xl[(b * 2 + (h >> 1)) * chunks + c])[h & 1] = eo;
                if (h == 0) dl[b * chunks + c] = dsw;
            }
        };
        uint4 xv[kSX];
#pragma unroll
        for (int i = 0; i < kSX; ++i) xv[i] = load_u(i * nt + tid);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D; ++d) issue(buf[d], max(0, min(d, steps - 1)));
        issue_fence();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kSX; ++i) quant_store(i * nt + tid, xv[i]);
        for (int base = kSX * nt; base < units; base += kSX * nt) {
#pragma unroll
            for (int i = 0; i < kSX; ++i) xv[i] = load_u(base + i * nt + tid);
#pragma unroll
            for (int i = 0; i < kSX; ++i) quant_store(base + i * nt + tid, xv[i]);
        }
    } else {
        // Stage the activation codes (regrouped) and pairs in LDS.  The first
        // kSU + kSD loads per thread go out before the weight prefetch, as buffer
        // loads whose out-of-range lanes fetch nothing: the load counter retires
        // in order, so storing them waits for them alone.  Longer activations
        // stage the rest in further rounds after the prefetch.
        constexpr int kSU = 4, kSD = 2;
        const int nt = int(blockDim.x), tid = int(threadIdx.x);
        const int units_per_row = p.k / 16;
        const int x_units = B * units_per_row;
        const int d_units = B * chunks;
        const rsrc_t rx = make_rsrc(a.xq, uint32_t(x_units) * 16u);
        const rsrc_t rd = make_rsrc(a.ds, uint32_t(d_units) * 4u);
        auto load_x = [&](int u) -> uint4 {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, int(u < x_units ? uint32_t(u) * 16u : kOutOfRange), 0, 0);
            return make_uint4(v.x, v.y, v.z, v.w);
        };
        auto load_d = [&](int u) -> uint32_t {
            return __builtin_amdgcn_raw_buffer_load_b32(rd, int(u < d_units ? uint32_t(u) * 4u : kOutOfRange), 0, 0);
        };
        auto store_x = [&](int u, const uint4 v) {
            if (u < x_units) {
                const int b = u / units_per_row;
                const int e = u - b * units_per_row;
                if constexpr (Bits == 4) {
                    const uint2 e0 = even_odd(v.x, v.y), e1 = even_odd(v.z, v.w);
                    xl[(b * 2 + (e & 1)) * chunks + (e >> 1)] = make_uint4(e0.x, e0.y, e1.x, e1.y);
                } else {
                    xl[(b * 2 + (e & 1)) * chunks + (e >> 1)] = v;
                }
            }
        };
        uint4 xv[kSU];
        uint32_t dv[kSD];
    #pragma unroll
        for (int i = 0; i < kSU; ++i) xv[i] = load_x(i * nt + tid);
    #pragma unroll
        for (int i = 0; i < kSD; ++i) dv[i] = load_d(i * nt + tid);
        __builtin_amdgcn_sched_barrier(0);       // keep these loads ahead of the prefetch

    #pragma unroll
        for (int d = 0; d < D; ++d) issue(buf[d], max(0, min(d, steps - 1)));
        issue_fence();
        __builtin_amdgcn_sched_barrier(0);

    #pragma unroll
        for (int i = 0; i < kSU; ++i) store_x(i * nt + tid, xv[i]);
    #pragma unroll
        for (int i = 0; i < kSD; ++i)
            if (i * nt + tid < d_units) dl[i * nt + tid] = dv[i];
        for (int base = kSU * nt; base < x_units; base += kSU * nt) {
    #pragma unroll
            for (int i = 0; i < kSU; ++i) xv[i] = load_x(base + i * nt + tid);
    #pragma unroll
            for (int i = 0; i < kSU; ++i) store_x(base + i * nt + tid, xv[i]);
        }
        for (int base = kSD * nt; base < d_units; base += kSD * nt) {
    #pragma unroll
            for (int i = 0; i < kSD; ++i) dv[i] = load_d(base + i * nt + tid);
    #pragma unroll
            for (int i = 0; i < kSD; ++i)
                if (base + i * nt + tid < d_units) dl[base + i * nt + tid] = dv[i];
        }
    }
    __syncthreads();

    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;

    auto consume = [&](const Buf &bf, int s) {
        const int t = s / passes;
        const int j = s - t * passes;
        const int pc = lane + kWave * j;
        const int64_t row0 = r_begin + int64_t(t) * R;
        if (pc < pieces) {
            const int c = pc / PPB, h = pc % PPB;    // block, half of it
            uint4 xp[B][2];
            float dv[B], sv[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if constexpr (Bits == 4) {
                    xp[b][0] = xl[(b * 2) * chunks + c];
                    xp[b][1] = xl[(b * 2 + 1) * chunks + c];
                } else {
                    xp[b][0] = xl[(b * 2 + h) * chunks + c];
                }
                const uint32_t dsw = dl[b * chunks + c];
                dv[b] = f16_bits_to_f32(dsw & 0xFFFFu);
                sv[b] = f16_bits_to_f32(dsw >> 16);
            }
            // 8-bit codes enter the dot as c - 128; 128 times the sum of the
            // piece's activation codes puts the difference back in the
            // integer sum, exactly (once per piece and batch row, shared by
            // the tile's rows)
            int qsum[B];
#pragma unroll
            for (int b = 0; b < B; ++b) qsum[b] = Bits == 8 ? 128 * code_sum_i8(xp[b][0]) : 0;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                if (row0 + i < r_end) {
                    const float sc = bf16_to_f32(bf.s[i]);
                    // the bias term once per block (8-bit: on its first half)
                    const float bi = (Bits == 4 || h == 0) ? bf16_to_f32(bf.b[i]) : 0.0f;
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        int idot;
                        if constexpr (Bits == 4) idot = dot_u4_i8(bf.c[i], xp[b]);
                        else idot = dot_u8_i8(bf.c[i], xp[b][0]) + qsum[b];
                        const float t_ = dv[b] * float(idot);
                        acc[i][b] = fmaf(bi, sv[b], fmaf(sc, t_, acc[i][b]));
                    }
                }
            }
        }
        if (j == passes - 1) reduce_store<R, B>(p, acc, row0, tile_rows<R>(row0, r_end), lane, [](int) { return 1.0f; });
    };

    run_pipeline<D>(buf, steps, issue, consume);
}

}  // namespace qg

// ------------------------------------------------------------------ C ABI

namespace {

constexpr int64_t kQ8MaxLds = 128 * 1024;
// rows per tile and steps in flight per wave: 8 code chunks in flight per
// lane either way; 4-row tiles halve the LDS activation reads per weight
// and are taken where every wave has at least 4 rows
constexpr int q8_depth(int r) { return 8 / r; }
// Eight waves per compute unit: two workgroups of four, or one workgroup of
// eight where staging costs more than the second workgroup brings, so each CU
// stages the activations once: beyond 32 KiB of them, and beyond 16 KiB when
// the staging also quantizes x or the batch is 3-4 (measured on the affine
// shapes of the decode step).
constexpr int64_t kQ8WideStage = 32 * 1024;
constexpr int64_t kQ8WideStageHeavy = 16 * 1024;

using qgl::aligned_to;

qg_status q8_cus(int *cus) {
    const int v = qgl::device_cu_count();
    if (v <= 0) return QG_ERR_DEVICE;
    *cus = v;
    return QG_OK;
}

template <int Bits, int R, int B, bool kFuse>
qg_status launch_q8(const qg::Params &p, const qg::Q8Args &a, int blocks, int waves, int64_t lds,
                    hipStream_t stream) {
    auto kern = qg::qgemv_affine_q8_kernel<Bits, R, B, q8_depth(R), kFuse>;
    if (lds > 64 * 1024) {
        static std::once_flag once;
        static hipError_t err = hipSuccess;
        std::call_once(once, [&] {
            err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, int(kQ8MaxLds));
        });
        if (err != hipSuccess) return QG_ERR_LAUNCH;
    }
    return qgl::launch_kernel(kern, dim3(blocks), dim3(waves * qg::kWave), size_t(lds), stream, p, a);
}

// The instance for a code width, batch size, tile shape and activation side
// (4-row tiles where every wave has at least 4 rows).
template <int Bits>
qg_status dispatch_q8(const qg::Params &p, const qg::Q8Args &a, int32_t batch, bool wide, int nb, int waves,
                      int64_t lds, hipStream_t stream) {
    if (a.x) {
        switch (batch) {
            case 1: return wide ? launch_q8<Bits, 4, 1, true>(p, a, nb, waves, lds, stream)
                                : launch_q8<Bits, 2, 1, true>(p, a, nb, waves, lds, stream);
            case 2: return wide ? launch_q8<Bits, 4, 2, true>(p, a, nb, waves, lds, stream)
                                : launch_q8<Bits, 2, 2, true>(p, a, nb, waves, lds, stream);
            case 3: return wide ? launch_q8<Bits, 4, 3, true>(p, a, nb, waves, lds, stream)
                                : launch_q8<Bits, 2, 3, true>(p, a, nb, waves, lds, stream);
            default: return wide ? launch_q8<Bits, 4, 4, true>(p, a, nb, waves, lds, stream)
                                 : launch_q8<Bits, 2, 4, true>(p, a, nb, waves, lds, stream);
        }
    }
    switch (batch) {
        case 1: return wide ? launch_q8<Bits, 4, 1, false>(p, a, nb, waves, lds, stream)
                            : launch_q8<Bits, 2, 1, false>(p, a, nb, waves, lds, stream);
        case 2: return wide ? launch_q8<Bits, 4, 2, false>(p, a, nb, waves, lds, stream)
                            : launch_q8<Bits, 2, 2, false>(p, a, nb, waves, lds, stream);
        case 3: return wide ? launch_q8<Bits, 4, 3, false>(p, a, nb, waves, lds, stream)
                            : launch_q8<Bits, 2, 3, false>(p, a, nb, waves, lds, stream);
        default: return wide ? launch_q8<Bits, 4, 4, false>(p, a, nb, waves, lds, stream)
                             : launch_q8<Bits, 2, 4, false>(p, a, nb, waves, lds, stream);
    }
}

// Validation (complete before any HIP call) and launch of the matvec for
// affine codes of `bits` bits; the activation side (a) is checked by the
// entry points.
qg_status run_q8(int bits, const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                 const qg::Q8Args &a, void *y, int64_t n, int64_t k, int32_t group_size, int32_t batch,
                 qg_out_dtype out_dtype, hipStream_t stream) {
    if (!codes || !scales || !biases || !y) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 1 || k % qg::kQ8Block) return QG_ERR_BAD_SHAPE;
    if (n > (int64_t(1) << 31) || k > (int64_t(1) << 30)) return QG_ERR_BAD_SHAPE;
    if (group_size != 32 && group_size != 64 && group_size != 128) return QG_ERR_BAD_GROUP_SIZE;
    if (k % group_size) return QG_ERR_BAD_GROUP_SIZE;
    if (batch < 1 || batch > 4) return QG_ERR_BAD_BATCH;
    if (out_dtype != QG_OUT_F32 && out_dtype != QG_OUT_BF16) return QG_ERR_BAD_DTYPE;
    if (!aligned_to(codes, 16)) return QG_ERR_MISALIGNED;
    if (!aligned_to(scales, 2) || !aligned_to(biases, 2)) return QG_ERR_MISALIGNED;
    if (!aligned_to(y, out_dtype == QG_OUT_F32 ? 4 : 2)) return QG_ERR_MISALIGNED;
    const int64_t chunks = k / qg::kQ8Block;
    const int64_t lds = qg::q8_lds_bytes(batch, chunks);
    if (lds > kQ8MaxLds) return QG_ERR_TOO_LARGE;
    int cus = 0;
    const qg_status st = q8_cus(&cus);
    if (st != QG_OK) return st;

    qg::Params p{};
    p.codes = reinterpret_cast<const unsigned char *>(codes);
    p.scales = scales;
    p.biases = biases;
    p.y = y;
    p.n = n;
    p.row_bytes = k * bits / 8;
    p.k = int32_t(k);
    p.chunks = int32_t(chunks);
    p.passes = int32_t((chunks * (bits / 4) + qg::kWave - 1) / qg::kWave);   // 16-byte code pieces per lane
    p.groups = int32_t(k / group_size);
    int shift = 0;
    while ((qg::kQ8Block << shift) < group_size) ++shift;
    p.group_shift = shift;
    p.out_bf16 = out_dtype == QG_OUT_BF16;
    const bool heavy = a.x != nullptr || batch >= 3;
    const int waves = (lds > kQ8WideStage || (heavy && lds > kQ8WideStageHeavy)) ? 8 : 4;
    int64_t blocks = int64_t(cus) * 8 / waves;          // fewer when rows are few
    const int64_t max_blocks = (n + waves - 1) / waves;
    if (blocks > max_blocks) blocks = max_blocks;
    p.total_waves = int32_t(blocks * waves);
    const int nb = int(blocks);
    const bool wide = n >= int64_t(4) * p.total_waves;
    return bits == 4 ? dispatch_q8<4>(p, a, batch, wide, nb, waves, lds, stream)
                     : dispatch_q8<8>(p, a, batch, wide, nb, waves, lds, stream);
}

}  // namespace

extern "C" {

qg_status qg_quantize_q8_1(const uint16_t *x, int64_t k, int32_t batch, int8_t *xq, uint16_t *ds,
                           hipStream_t stream) {
    if (!x || !xq || !ds) return QG_ERR_NULL_POINTER;
    if (k < 1 || k % qg::kQ8Block || k > (int64_t(1) << 30)) return QG_ERR_BAD_SHAPE;
    if (batch < 1 || batch > 4) return QG_ERR_BAD_BATCH;
    if (!aligned_to(x, 16) || !aligned_to(xq, 16) || !aligned_to(ds, 4)) return QG_ERR_MISALIGNED;
    const int64_t units = int64_t(batch) * k / 8;
    const int64_t grid = (units + 255) / 256;
    return qgl::launch_kernel(qg::qg_quantize_q8_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, x, units, xq,
                              reinterpret_cast<uint32_t *>(ds));
}

qg_status qgemv_affine_u4_q8(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                             const int8_t *xq, const uint16_t *ds, void *y, int64_t n, int64_t k,
                             int32_t group_size, int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    if (!xq || !ds) return QG_ERR_NULL_POINTER;
    if (!aligned_to(xq, 16) || !aligned_to(ds, 4)) return QG_ERR_MISALIGNED;
    return run_q8(4, codes, scales, biases, qg::Q8Args{xq, reinterpret_cast<const uint32_t *>(ds), nullptr}, y, n, k, group_size, batch, out_dtype,
                  stream);
}

qg_status qgemv_affine_u4_q8_fused(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                   const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                                   int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    if (!x) return QG_ERR_NULL_POINTER;
    if (!aligned_to(x, 16)) return QG_ERR_MISALIGNED;
    return run_q8(4, codes, scales, biases, qg::Q8Args{nullptr, nullptr, x}, y, n, k, group_size, batch,
                  out_dtype, stream);
}

qg_status qgemv_affine_u8_q8(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                             const int8_t *xq, const uint16_t *ds, void *y, int64_t n, int64_t k,
                             int32_t group_size, int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    if (!xq || !ds) return QG_ERR_NULL_POINTER;
    if (!aligned_to(xq, 16) || !aligned_to(ds, 4)) return QG_ERR_MISALIGNED;
    return run_q8(8, codes, scales, biases, qg::Q8Args{xq, reinterpret_cast<const uint32_t *>(ds), nullptr}, y, n, k, group_size, batch, out_dtype,
                  stream);
}

qg_status qgemv_affine_u8_q8_fused(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                                   const uint16_t *x, void *y, int64_t n, int64_t k, int32_t group_size,
                                   int32_t batch, qg_out_dtype out_dtype, hipStream_t stream) {
    if (!x) return QG_ERR_NULL_POINTER;
    if (!aligned_to(x, 16)) return QG_ERR_MISALIGNED;
    return run_q8(8, codes, scales, biases, qg::Q8Args{nullptr, nullptr, x}, y, n, k, group_size, batch,
                  out_dtype, stream);
}

}  // extern "C"
