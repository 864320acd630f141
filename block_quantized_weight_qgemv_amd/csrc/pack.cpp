// Host pack/layout module: offline quantizers, code packers and layout sizes.
//
// These produce the packed layouts the device entry points read (include/qgemv.h).
// The quantizer rules follow the pages' statement of the formats:
//  - FP4-E2M1 with per-group scales ("Hand-Writing Gemma 4 Flash-Decoding + an
//    FP4 Matvec Bonus (Part 2)", section "The assumption that failed the
//    profiler"); the scale is the group absmax over 6 rounded to bf16.
//  - min-max affine 4/8-bit, group 64, u32 low-first, with scale and bias
//    rounded to bf16 before q is computed (mlxcel issue #683, "Step 2 result").
//  - FP8-E4M3 with one fp32 scale per row (Part 2 post, the FP8 lm_head).
//  - the two-level super-block 4-bit format, its storage records and the
//    pre-unpacked device layout ("perf(cuda): generalize Gemma 4 batched
//    prefill + flash attn + decode graphs to dense Q4_K models", sections
//    "Work Item C (C1) done", "Item C2" and "All work items complete").
//
// All arithmetic is IEEE double (or the single binary32 division of the FP8
// row scale) with one rounding per operation; this file must be built without
// floating-point contraction (-ffp-contract=off).  Rounding to bf16 and E4M3
// works on the binary64 bit pattern; nearest-E2M1 uses the format's midpoints.

#include "qgemv.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- rounding

inline uint64_t f64_bits(double v) {
    uint64_t b;
    std::memcpy(&b, &v, sizeof b);
    return b;
}

inline double bf16_to_double(uint16_t h) {
    uint32_t b = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &b, sizeof f);
    return static_cast<double>(f);
}

// Round a double to the nearest bf16, ties to even.  Normal results keep the
// top 7 fraction bits of the binary64 pattern (45 bits dropped, rounded on the
// combined exponent|fraction field so a carry bumps the exponent); results
// below 2^-126 are multiples of the bf16 subnormal step 2^-133.
uint16_t bf16_rne(double v) {
    const uint64_t bits = f64_bits(v);
    const uint16_t sign = static_cast<uint16_t>((bits >> 48) & 0x8000u);
    const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
    if (mag > 0x7FF0000000000000ull) return 0x7FC0;               // NaN
    if (mag == 0x7FF0000000000000ull) return sign | 0x7F80;       // inf
    const double a = std::fabs(v);
    if (a < 0x1p-126) {
        const double q = std::nearbyint(a * 0x1p133);             // exact scaling
        return sign | static_cast<uint16_t>(q);                   // 128 -> min normal
    }
    const uint64_t r = (mag + ((1ull << 44) - 1) + ((mag >> 45) & 1)) >> 45;
    const int64_t exp_bf = static_cast<int64_t>(r >> 7) - 1023 + 127;
    if (exp_bf >= 255) return sign | 0x7F80;
    return sign | static_cast<uint16_t>((exp_bf << 7) | (r & 0x7F));
}

// Round a double to the nearest fp16, ties to even: normal results keep the
// top 10 fraction bits of the binary64 pattern (42 bits dropped, rounded on
// the combined exponent|fraction field); results below 2^-14 are multiples of
// the fp16 subnormal step 2^-24; 65520 and above overflow to infinity.
uint16_t f16_rne(double v) {
    const uint64_t bits = f64_bits(v);
    const uint16_t sign = static_cast<uint16_t>((bits >> 48) & 0x8000u);
    const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
    if (mag > 0x7FF0000000000000ull) return 0x7E00;               // NaN
    const double a = std::fabs(v);
    if (a < 0x1p-14) {
        const double q = std::nearbyint(a * 0x1p24);              // exact scaling
        return sign | static_cast<uint16_t>(q);                   // 1024 -> min normal
    }
    const uint64_t r = (mag + ((1ull << 41) - 1) + ((mag >> 42) & 1)) >> 42;
    const int64_t exp16 = static_cast<int64_t>(r >> 10) - 1023 + 15;
    if (exp16 >= 31) return sign | 0x7C00;
    return sign | static_cast<uint16_t>((exp16 << 10) | (r & 0x3FF));
}

double f16_to_double(uint16_t h) {
    const int e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double m;
    if (e == 0) m = std::ldexp(static_cast<double>(f), -24);
    else if (e == 31) m = f ? NAN : INFINITY;
    else m = std::ldexp(static_cast<double>(1024 + f), e - 25);
    return (h & 0x8000) ? -m : m;
}

// Nearest E2M1 magnitude index (0..7) of a >= 0, ties to even mantissa bit.
// Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; midpoints .25 .75 1.25 1.75 2.5 3.5 5
// resolve to the even index on either side.
inline uint8_t e2m1_mag_index(double a) {
    if (a <= 0.25) return 0;
    if (a < 0.75) return 1;
    if (a <= 1.25) return 2;
    if (a < 1.75) return 3;
    if (a <= 2.5) return 4;
    if (a < 3.5) return 5;
    if (a <= 5.0) return 6;
    return 7;
}

// Nearest finite E4M3 (OCP FN) code of a in [0, 448], ties to even.
inline uint8_t e4m3_mag_code(double a) {
    if (a < 0x1p-6) {                                              // subnormal step 2^-9
        return static_cast<uint8_t>(std::nearbyint(a * 0x1p9));   // 8 -> min normal
    }
    const uint64_t mag = f64_bits(a);
    const uint64_t r = (mag + ((1ull << 48) - 1) + ((mag >> 49) & 1)) >> 49;
    const int64_t exp8 = static_cast<int64_t>(r >> 3) - 1023 + 7;
    return static_cast<uint8_t>((exp8 << 3) | (r & 7));
}

// ---------------------------------------------------------------- threading

template <class F>
void parallel_rows(int64_t n, F &&fn) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t threads = std::min<int64_t>(std::max(1u, std::min(hw, 16u)), (n + 255) / 256);
    if (threads <= 1) {
        fn(int64_t(0), n);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(threads);
    for (int64_t t = 0; t < threads; ++t) {
        int64_t r0 = n * t / threads, r1 = n * (t + 1) / threads;
        pool.emplace_back([&fn, r0, r1] { fn(r0, r1); });
    }
    for (auto &th : pool) th.join();
}

bool all_finite(const float *w, int64_t count) {
    for (int64_t i = 0; i < count; ++i)
        if (!std::isfinite(w[i])) return false;
    return true;
}

bool valid_group(int32_t gs) { return gs == 32 || gs == 64 || gs == 128; }

}  // namespace

extern "C" {

qg_status qg_quantize_fp4_e2m1(const float *w, int64_t n, int64_t k, int32_t group_size,
                               uint8_t *codes, uint16_t *scales) {
    if (!w || !codes || !scales) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 2 || k % 2) return QG_ERR_BAD_SHAPE;
    if (!valid_group(group_size) || k % group_size) return QG_ERR_BAD_GROUP_SIZE;
    if (!all_finite(w, n * k)) return QG_ERR_BAD_VALUE;
    const int64_t ng = k / group_size;
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            const float *row = w + r * k;
            uint8_t *crow = codes + r * (k / 2);
            for (int64_t g = 0; g < ng; ++g) {
                const float *grp = row + g * group_size;
                float absmax = 0.0f;
                for (int32_t i = 0; i < group_size; ++i) absmax = std::max(absmax, std::fabs(grp[i]));
                const uint16_t sb = bf16_rne(static_cast<double>(absmax) / 6.0);
                scales[r * ng + g] = sb;
                const double s = bf16_to_double(sb);
                for (int32_t i = 0; i < group_size; ++i) {
                    uint8_t c = 0;
                    if (s != 0.0) {
                        const double q = static_cast<double>(grp[i]) / s;
                        c = e2m1_mag_index(std::min(std::fabs(q), 6.0)) | (q < 0.0 ? 8 : 0);
                    }
                    const int64_t col = g * group_size + i;
                    uint8_t &byte = crow[col / 2];
                    if (col % 2 == 0) byte = c;
                    else byte = static_cast<uint8_t>(byte | (c << 4));
                }
            }
        }
    });
    return QG_OK;
}

qg_status qg_quantize_affine(const float *w, int64_t n, int64_t k, int32_t bits,
                             int32_t group_size, uint32_t *codes, uint16_t *scales,
                             uint16_t *biases) {
    if (!w || !codes || !scales || !biases) return QG_ERR_NULL_POINTER;
    if (bits != 4 && bits != 8) return QG_ERR_BAD_BITS;
    const int32_t per = 32 / bits;
    if (n < 1 || k < per || k % per) return QG_ERR_BAD_SHAPE;
    if (!valid_group(group_size) || k % group_size) return QG_ERR_BAD_GROUP_SIZE;
    if (!all_finite(w, n * k)) return QG_ERR_BAD_VALUE;
    const int64_t ng = k / group_size;
    const double qmax = static_cast<double>((1 << bits) - 1);
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            const float *row = w + r * k;
            uint32_t *wrow = codes + r * (k / per);
            std::fill(wrow, wrow + k / per, 0u);
            for (int64_t g = 0; g < ng; ++g) {
                const float *grp = row + g * group_size;
                float mn = grp[0], mx = grp[0];
                for (int32_t i = 1; i < group_size; ++i) {
                    mn = std::min(mn, grp[i]);
                    mx = std::max(mx, grp[i]);
                }
                const uint16_t sb = bf16_rne((static_cast<double>(mx) - static_cast<double>(mn)) / qmax);
                const uint16_t bb = bf16_rne(static_cast<double>(mn));
                scales[r * ng + g] = sb;
                biases[r * ng + g] = bb;
                const double s = bf16_to_double(sb), b = bf16_to_double(bb);
                for (int32_t i = 0; i < group_size; ++i) {
                    uint32_t q = 0;
                    if (s != 0.0) {
                        double t = std::nearbyint((static_cast<double>(grp[i]) - b) / s);
                        t = std::min(std::max(t, 0.0), qmax);
                        q = static_cast<uint32_t>(t);
                    }
                    const int64_t col = g * group_size + i;
                    wrow[col / per] |= q << (bits * (col % per));
                }
            }
        }
    });
    return QG_OK;
}

qg_status qg_quantize_fp8_e4m3_rowwise(const float *w, int64_t n, int64_t k,
                                       uint8_t *codes, float *row_scale) {
    if (!w || !codes || !row_scale) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 1) return QG_ERR_BAD_SHAPE;
    if (!all_finite(w, n * k)) return QG_ERR_BAD_VALUE;
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            const float *row = w + r * k;
            float absmax = 0.0f;
            for (int64_t i = 0; i < k; ++i) absmax = std::max(absmax, std::fabs(row[i]));
            const float s = absmax / 448.0f;                       // one binary32 division
            row_scale[r] = s;
            uint8_t *crow = codes + r * k;
            for (int64_t i = 0; i < k; ++i) {
                uint8_t c = 0;
                if (s != 0.0f) {
                    const double q = static_cast<double>(row[i]) / static_cast<double>(s);
                    c = e4m3_mag_code(std::min(std::fabs(q), 448.0)) | (q < 0.0 ? 0x80 : 0);
                }
                crow[i] = c;
            }
        }
    });
    return QG_OK;
}

qg_status qg_pack_nibbles(const uint8_t *in, int64_t count, uint8_t *packed) {
    if (!in || !packed) return QG_ERR_NULL_POINTER;
    if (count < 0 || count % 2) return QG_ERR_BAD_SHAPE;
    for (int64_t i = 0; i < count; ++i)
        if (in[i] > 15) return QG_ERR_BAD_VALUE;
    for (int64_t i = 0; i < count / 2; ++i)
        packed[i] = static_cast<uint8_t>(in[2 * i] | (in[2 * i + 1] << 4));
    return QG_OK;
}

qg_status qg_unpack_nibbles(const uint8_t *packed, int64_t count, uint8_t *out) {
    if (!packed || !out) return QG_ERR_NULL_POINTER;
    if (count < 0 || count % 2) return QG_ERR_BAD_SHAPE;
    for (int64_t i = 0; i < count / 2; ++i) {
        out[2 * i] = packed[i] & 0x0F;
        out[2 * i + 1] = packed[i] >> 4;
    }
    return QG_OK;
}

qg_status qg_pack_u32(const uint8_t *in, int64_t count, int32_t bits, uint32_t *packed) {
    if (!in || !packed) return QG_ERR_NULL_POINTER;
    if (bits != 4 && bits != 8) return QG_ERR_BAD_BITS;
    const int32_t per = 32 / bits;
    if (count < 0 || count % per) return QG_ERR_BAD_SHAPE;
    for (int64_t i = 0; i < count; ++i)
        if (in[i] >> bits) return QG_ERR_BAD_VALUE;
    for (int64_t wd = 0; wd < count / per; ++wd) {
        uint32_t v = 0;
        for (int32_t j = 0; j < per; ++j) v |= static_cast<uint32_t>(in[wd * per + j]) << (bits * j);
        packed[wd] = v;
    }
    return QG_OK;
}

qg_status qg_unpack_u32(const uint32_t *packed, int64_t count, int32_t bits, uint8_t *out) {
    if (!packed || !out) return QG_ERR_NULL_POINTER;
    if (bits != 4 && bits != 8) return QG_ERR_BAD_BITS;
    const int32_t per = 32 / bits;
    if (count < 0 || count % per) return QG_ERR_BAD_SHAPE;
    const uint32_t mask = (1u << bits) - 1;
    for (int64_t i = 0; i < count; ++i)
        out[i] = static_cast<uint8_t>((packed[i / per] >> (bits * (i % per))) & mask);
    return QG_OK;
}

// Two-level super-block 4-bit format: see include/qgemv.h for the record
// layout and the rule; one super-block (256 weights, 8 sub-blocks) at a time.
qg_status qg_quantize_q4k(const float *w, int64_t n, int64_t k, uint8_t *records) {
    if (!w || !records) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 256 || k % 256) return QG_ERR_BAD_SHAPE;
    if (!all_finite(w, n * k)) return QG_ERR_BAD_VALUE;
    const int64_t nsb = k / 256;
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t b = 0; b < nsb; ++b) {
                const float *blk = w + r * k + b * 256;
                uint8_t *rec = records + (r * nsb + b) * 144;
                double s[8], off[8], smax = 0.0, omax = 0.0;
                for (int j = 0; j < 8; ++j) {
                    float mn = blk[32 * j], mx = blk[32 * j];
                    for (int i = 1; i < 32; ++i) {
                        mn = std::min(mn, blk[32 * j + i]);
                        mx = std::max(mx, blk[32 * j + i]);
                    }
                    const double lo = std::min(static_cast<double>(mn), 0.0);
                    s[j] = (static_cast<double>(mx) - lo) / 15.0 + 0.0;
                    off[j] = 0.0 - lo;
                    smax = std::max(smax, s[j]);
                    omax = std::max(omax, off[j]);
                }
                const uint16_t db = f16_rne(smax / 63.0), mb = f16_rne(omax / 63.0);
                const double d = f16_to_double(db), dmin = f16_to_double(mb);
                uint64_t fsc = 0, fm = 0;
                int sc[8], m[8];
                for (int j = 0; j < 8; ++j) {
                    sc[j] = d > 0.0 ? static_cast<int>(std::min(std::max(std::nearbyint(s[j] / d), 0.0), 63.0)) : 0;
                    m[j] = dmin > 0.0 ? static_cast<int>(std::min(std::max(std::nearbyint(off[j] / dmin), 0.0), 63.0))
                                      : 0;
                    fsc |= static_cast<uint64_t>(sc[j]) << (6 * j);
                    fm |= static_cast<uint64_t>(m[j]) << (6 * j);
                }
                rec[0] = static_cast<uint8_t>(db & 0xFF);
                rec[1] = static_cast<uint8_t>(db >> 8);
                rec[2] = static_cast<uint8_t>(mb & 0xFF);
                rec[3] = static_cast<uint8_t>(mb >> 8);
                for (int i = 0; i < 6; ++i) {
                    rec[4 + i] = static_cast<uint8_t>((fsc >> (8 * i)) & 0xFF);
                    rec[10 + i] = static_cast<uint8_t>((fm >> (8 * i)) & 0xFF);
                }
                for (int j = 0; j < 8; ++j) {
                    const double S = d * sc[j], M = dmin * m[j];            // exact
                    for (int i = 0; i < 32; ++i) {
                        uint8_t q = 0;
                        if (S > 0.0) {
                            const double t = std::nearbyint((static_cast<double>(blk[32 * j + i]) + M) / S);
                            q = static_cast<uint8_t>(std::min(std::max(t, 0.0), 15.0));
                        }
                        const int col = 32 * j + i;
                        uint8_t &byte = rec[16 + col / 2];
                        if (col % 2 == 0) byte = q;
                        else byte = static_cast<uint8_t>(byte | (q << 4));
                    }
                }
            }
        }
    });
    return QG_OK;
}

qg_status qg_repack_q4k(const uint8_t *records, int64_t n, int64_t k, uint32_t *codes, uint16_t *sub,
                        uint32_t *super) {
    if (!records || !codes || !sub || !super) return QG_ERR_NULL_POINTER;
    if (n < 1 || k < 256 || k % 256) return QG_ERR_BAD_SHAPE;
    const int64_t nsb = k / 256;
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t b = 0; b < nsb; ++b) {
                const uint8_t *rec = records + (r * nsb + b) * 144;
                super[r * nsb + b] = static_cast<uint32_t>(rec[0]) | (static_cast<uint32_t>(rec[1]) << 8) |
                                     (static_cast<uint32_t>(rec[2]) << 16) | (static_cast<uint32_t>(rec[3]) << 24);
                uint64_t fsc = 0, fm = 0;
                for (int i = 0; i < 6; ++i) {
                    fsc |= static_cast<uint64_t>(rec[4 + i]) << (8 * i);
                    fm |= static_cast<uint64_t>(rec[10 + i]) << (8 * i);
                }
                for (int j = 0; j < 8; ++j)
                    sub[r * (k / 32) + b * 8 + j] = static_cast<uint16_t>(((fsc >> (6 * j)) & 63) |
                                                                          (((fm >> (6 * j)) & 63) << 8));
                // the 128 code bytes are the 32 words of the super-block, low byte first
                for (int wd = 0; wd < 32; ++wd)
                    codes[r * (k / 8) + b * 32 + wd] =
                        static_cast<uint32_t>(rec[16 + 4 * wd]) | (static_cast<uint32_t>(rec[17 + 4 * wd]) << 8) |
                        (static_cast<uint32_t>(rec[18 + 4 * wd]) << 16) | (static_cast<uint32_t>(rec[19 + 4 * wd]) << 24);
            }
        }
    });
    return QG_OK;
}

int64_t qg_bytes_q4k_records(int64_t n, int64_t k) {
    if (n < 1 || k < 256 || k % 256) return -1;
    return n * (k / 256) * 144;
}

int64_t qg_bytes_q4k(int64_t n, int64_t k) {
    if (n < 1 || k < 256 || k % 256) return -1;
    return n * (k / 2) + n * (k / 32) * 2 + n * (k / 256) * 4;
}

int64_t qg_bytes_fp4(int64_t n, int64_t k, int32_t group_size) {
    if (n < 1 || k < 2 || k % 2 || !valid_group(group_size) || k % group_size) return -1;
    return n * (k / 2) + n * (k / group_size) * 2;
}

int64_t qg_bytes_affine(int64_t n, int64_t k, int32_t bits, int32_t group_size) {
    if (bits != 4 && bits != 8) return -1;
    if (n < 1 || k < 1 || k % (32 / bits) || !valid_group(group_size) || k % group_size) return -1;
    return n * (k * bits / 8) + n * (k / group_size) * 4;
}

int64_t qg_bytes_fp8(int64_t n, int64_t k) {
    if (n < 1 || k < 1) return -1;
    return n * k + n * 4;
}

}  // extern "C"
